// Device helpers shared by the merge kernel and the fused split epilogue: the
// exact merge of S split states of one (sequence, query head) row
// ("Flash-Decoding: Split-KV Attention for Long-Context Decode", kanthi.in,
// §2 stable form; xuujii KB "Decode 专项 Attention" §04).
//
// Two forms.
// - Merge kernel: each row gets SG groups of D/4 lanes that fold its splits
//   split by split; its many workgroups keep the memory system busy.
// - Fused tail: one workgroup merges a whole group of rows, so it needs more
//   loads in flight per lane. One wave (or WPR waves) takes a row; lane
//   (grp, dl) covers dims [4 dl, 4 dl + 4) of splits grp, grp + NG, ... (NG
//   lane groups on the row), issues the loads of NB of them together and
//   folds the batch with one rescale to the larger maximum, so a row of S
//   splits costs about S / (NG * NB) memory round trips. The lane groups are
//   combined by cross-lane shuffles and, with WPR > 1, through LDS.
// A split whose m (lse) is -inf weighs exactly 0; a row whose splits are all
// empty gives O = 0 and LSE = -inf. Every sum has a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

typedef float mf32x4 __attribute__((ext_vector_type(4)));
typedef float mf32x2 __attribute__((ext_vector_type(2)));

struct RowState {
  mf32x4 acc;
  float m;
  float den;
};

// ---- merge kernel (split states of a finished launch): SG groups of D/4 lanes
// share a row's splits (split s goes to group s % SG); each lane folds its
// splits one at a time, rebasing its running sums whenever a larger maximum
// arrives, and the SG partial states are then merged through LDS.

// Fold splits grp, grp + SG, ... of one row. `stats` points at the row's first
// split statistic, `ws` at the row's first split vector plus this lane's dims.
template <int D>
__device__ __forceinline__ RowState fold_splits(const float* __restrict__ ws, const float* __restrict__ stats,
                                                int S, bool uml, int grp, int SG) {
  const int sstride = uml ? 2 : 1;
  RowState st;
  st.acc = mf32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.den = 0.f;
#pragma unroll 4
  for (int s = grp; s < S; s += SG) {
    const float ms = stats[s * sstride];
    const float ls = uml ? stats[s * sstride + 1] : 1.f;
    const mf32x4 u = *reinterpret_cast<const mf32x4*>(ws + (int64_t)s * D);
    const bool valid = ms != -INFINITY;
    const float mn = valid ? fmaxf(st.m, ms) : st.m;
    const float a = st.m == -INFINITY ? 0.f : expf(st.m - mn);
    const float w = valid ? expf(ms - mn) : 0.f;
    st.acc = st.acc * a + (valid ? u * w : mf32x4{0.f, 0.f, 0.f, 0.f});
    st.den = st.den * a + (valid ? ls * w : 0.f);
    st.m = mn;
  }
  return st;
}

// Merge SG partial states stored at part[base + g*stride] (g < SG) and write the
// row's output (4 floats at out_row + 4*dl) and, for dl == 0, its LSE.
__device__ __forceinline__ void finish_row(const mf32x4* part, const float* part_m, const float* part_d,
                                           int base, int stride, int SG, float* out_row, int dl, float* lse) {
  float M = -INFINITY;
  for (int g = 0; g < SG; ++g) M = fmaxf(M, part_m[base + g * stride]);
  mf32x4 o = {0.f, 0.f, 0.f, 0.f};
  float dr = 0.f;
  if (M != -INFINITY) {
    for (int g = 0; g < SG; ++g) {
      const float mg = part_m[base + g * stride];
      const float a = mg == -INFINITY ? 0.f : expf(mg - M);
      o += part[base + g * stride] * a;
      dr += part_d[base + g * stride] * a;
    }
  }
  const bool empty = !(dr > 0.f);
  const float inv = empty ? 0.f : 1.f / dr;
  *reinterpret_cast<mf32x4*>(out_row + 4 * dl) = o * inv;
  if (lse && dl == 0) *lse = empty ? -INFINITY : M + logf(dr);
}

// Split groups per row for `rows` rows sharing `threads` threads (power of two).
__host__ __device__ inline int split_groups_log2(int S, int lanes_per_row, int rows, int threads) {
  int sg = 0;
  while ((1 << sg) < S && rows * (lanes_per_row << (sg + 1)) <= threads) ++sg;
  return sg;
}

// ---- fused tail (states published in the same launch): one or more waves per row.

// Cache policy bits of the fused tail's state loads: sc1, the form the
// compiler gives agent-scope atomic loads on gfx950, so they read states that
// other workgroups of the same launch published with device-coherent stores.
constexpr int LOAD_COHERENT = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same pointer, marked wave-uniform (a buffer resource lives in SGPRs).
__device__ __forceinline__ const float* uniform_ptr(const float* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
}

// Fold splits gi, gi + NG, ... of one row into a lane state. ws_row and st_row
// (wave-uniform) are the row's first split vector and statistic.
// NB: splits whose loads one lane has in flight together.
template <int D, bool UML, int NB>
__device__ __forceinline__ RowState fold_row(const float* ws_row, const float* st_row, int S, int gi, int NG, int dl) {
  constexpr int SW = UML ? 2 : 1;
  const __amdgpu_buffer_rsrc_t ru = row_rsrc(ws_row, (uint32_t)S * D * 4);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(st_row, (uint32_t)S * SW * 4);
  RowState st = {mf32x4{0.f, 0.f, 0.f, 0.f}, -INFINITY, 0.f};
  for (int s0 = gi; s0 < S; s0 += NB * NG) {
    mf32x4 u[NB];
    float m[NB], l[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int s = s0 + j * NG;
      u[j] = mf32x4{0.f, 0.f, 0.f, 0.f};
      m[j] = -INFINITY;
      l[j] = 0.f;
      if (s < S) {                              // issued back to back; first used after the batch
        u[j] = __builtin_bit_cast(mf32x4, __builtin_amdgcn_raw_buffer_load_b128(ru, (uint32_t)(s * D + 4 * dl) * 4,
                                                                              0, LOAD_COHERENT));
        if (UML) {
          const mf32x2 ml =
              __builtin_bit_cast(mf32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)s * 8, 0, LOAD_COHERENT));
          m[j] = ml.x;
          l[j] = ml.y;
        } else {
          m[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)s * 4, 0, LOAD_COHERENT));
          l[j] = 1.f;
        }
      }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NB; ++j) bm = fmaxf(bm, m[j]);
    if (bm == -INFINITY) continue;
    const float mn = fmaxf(st.m, bm);
    const float a = st.m == -INFINITY ? 0.f : expf(st.m - mn);
    st.acc = st.acc * a;
    st.den = st.den * a;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool valid = m[j] != -INFINITY;
      const float w = valid ? expf(m[j] - mn) : 0.f;
      st.acc += valid ? u[j] * w : mf32x4{0.f, 0.f, 0.f, 0.f};
      st.den += valid ? l[j] * w : 0.f;
    }
    st.m = mn;
  }
  return st;
}

// a <- merge(a, b), both rescaled to the larger maximum.
__device__ __forceinline__ void combine(RowState& a, const RowState& b) {
  const float M = fmaxf(a.m, b.m);
  const float wa = a.m == -INFINITY ? 0.f : expf(a.m - M);
  const float wb = b.m == -INFINITY ? 0.f : expf(b.m - M);
  a.acc = a.acc * wa + b.acc * wb;
  a.den = a.den * wa + b.den * wb;
  a.m = M;
}

// Combine the lane groups of a wave (lanes dl, dl + LPR, ...): afterwards
// every lane holds the state of its dims over all of the wave's splits.
template <int LPR>
__device__ __forceinline__ RowState wave_combine(RowState st) {
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    RowState o;
    o.m = __shfl_xor(st.m, off);
    o.den = __shfl_xor(st.den, off);
    o.acc = mf32x4{__shfl_xor(st.acc.x, off), __shfl_xor(st.acc.y, off), __shfl_xor(st.acc.z, off),
                   __shfl_xor(st.acc.w, off)};
    combine(st, o);
  }
  return st;
}

// Final O = acc / den (4 floats at out_row + 4 dl) and, for dl == 0, LSE.
__device__ __forceinline__ void write_row(const RowState& st, float* out_row, float* lse, int dl) {
  const bool empty = !(st.den > 0.f);
  const float inv = empty ? 0.f : 1.f / st.den;
  *reinterpret_cast<mf32x4*>(out_row + 4 * dl) = st.acc * inv;
  if (lse && dl == 0) *lse = empty ? -INFINITY : st.m + logf(st.den);
}

template <int NW> struct MergeLds {
  mf32x4 acc[NW][32];
  float m[NW];
  float den[NW];
};

// Waves per row (log2) for `rows` rows on NW waves: the most that still
// merges every row in one pass, at least one.
__host__ __device__ inline int waves_per_row_log2(int rows, int nw) {
  int w = 0;
  while ((2 << w) <= nw && rows * (2 << w) <= nw) ++w;
  return w;
}

// One pass of the workgroup over NW >> wpr_log2 rows: waves [k WPR, k WPR + WPR)
// merge state row `row` (wave-uniform; `active` false for a wave without a row).
// Every thread of the workgroup calls it; with wpr_log2 > 0 it holds barriers.
template <int D, int NW, int NB>
__device__ __forceinline__ void merge_row_pass(int64_t row, bool active, int S, bool uml, int wpr_log2,
                                               const float* ws_o, const float* ws_stats, float* out, float* lse,
                                               MergeLds<NW>& sh) {
  constexpr int LPR = D / 4;
  constexpr int SGW = 64 / LPR;                // lane groups per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wsub = wave & ((1 << wpr_log2) - 1);
  const int grp = lane / LPR;
  const int dl = lane - grp * LPR;
  RowState st = {mf32x4{0.f, 0.f, 0.f, 0.f}, -INFINITY, 0.f};
  if (active) {
    const float* wr = uniform_ptr(ws_o + row * S * D);
    const float* sr = uniform_ptr(ws_stats + row * S * (uml ? 2 : 1));
    const int NG = SGW << wpr_log2;
    const int gi = wsub * SGW + grp;
    st = uml ? fold_row<D, true, NB>(wr, sr, S, gi, NG, dl) : fold_row<D, false, NB>(wr, sr, S, gi, NG, dl);
    st = wave_combine<LPR>(st);
  }
  if (wpr_log2 == 0) {
    if (active && grp == 0) write_row(st, out + row * D, lse ? lse + row : nullptr, dl);
    return;
  }
  if (grp == 0) {
    sh.acc[wave][dl] = st.acc;
    if (dl == 0) {
      sh.m[wave] = st.m;
      sh.den[wave] = st.den;
    }
  }
  __syncthreads();
  if (active && wsub == 0 && grp == 0) {
    for (int k = 1; k < (1 << wpr_log2); ++k) {
      const RowState o = {sh.acc[wave + k][dl], sh.m[wave + k], sh.den[wave + k]};
      combine(st, o);
    }
    write_row(st, out + row * D, lse ? lse + row : nullptr, dl);
  }
  __syncthreads();
}

}  // namespace fd

#include "fd_internal.h"

namespace fd {

// Stores of split states that another workgroup may read in the same launch
// (fused merge) go out as agent-scope atomic stores: device-coherent
// write-through stores, so publishing them needs no cache-wide write-back.
// Output / workspace row of state row r (< g * q_len) of group (b, kvh): query
// row i = r / g of the block, head kvh * g + r % g.
__device__ __forceinline__ int64_t state_row(const SplitParams& p, int b, int kvh, int r) {
  const int i = r / p.g;
  const int h = r - i * p.g;
  return ((int64_t)b * p.q_len + i) * p.Hq + (int64_t)kvh * p.g + h;
}

__device__ __forceinline__ void ws_store(float* p, float v, bool coherent) {
  if (coherent)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Fused merge at the end of a split workgroup (or of one piece of it) (the "last CTA merges" variant of
// the kanthi.in chapter's decode contract). Every workgroup of a (sequence,
// KV head) group has written its split states with ws_store(..., true); once
// its own stores have completed (s_waitcnt) the workgroup counts itself in
// with a device-scope atomic, and the one that arrives as number `expected`
// (the group's writer count) reads the group's
// states back with device-coherent loads, merges the group's g * q_len rows
// into out/lse and resets the counter to 0 so the next stream-ordered call
// starts from zero.
template <int D, int NTHREADS, int NB>
__device__ __forceinline__ void fused_group_merge(const SplitParams& p, int b, int kvh, int expected) {
  __shared__ int s_last;
  // Publication: the state stores are device-scope (sc1) stores, which write
  // through to the device's coherence point, so once the wait below has seen
  // them complete they are visible to sc1 loads from any CU of any XCD. The
  // two compiler-only fences keep the stores before the wait and the counter
  // atomic after it (the wait intrinsic itself claims no memory effects).
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);            // this thread's state stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(p.counters + (int64_t)b * p.Hkv + kvh, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (unsigned)(expected - 1);
  }
  __syncthreads();
  if (!s_last) return;

  constexpr int NWV = NTHREADS / 64;
  __shared__ MergeLds<NWV> sh;
  const bool uml = p.ws_format == FD_WS_UML;
  const int wpr_log2 = waves_per_row_log2(p.R, NWV);
  const int per_pass = NWV >> wpr_log2;
  const int k = (threadIdx.x >> 6) >> wpr_log2;
  for (int r0 = 0; r0 < p.R; r0 += per_pass) {            // the group's rows, per_pass of them at a time
    const bool active = r0 + k < p.R;
    const int64_t row = state_row(p, b, kvh, active ? r0 + k : 0);
    merge_row_pass<D, NWV, NB>(row, active, p.S, uml, wpr_log2, p.ws_o, p.ws_stats, p.out, p.lse, sh);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(p.counters + (int64_t)b * p.Hkv + kvh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace fd
