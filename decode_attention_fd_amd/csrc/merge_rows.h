// Device helpers shared by the merge kernel and the fused split epilogue: the
// exact merge of S split states of one (sequence, query head) row
// ("Flash-Decoding: Split-KV Attention for Long-Context Decode", kanthi.in,
// §2 stable form; xuujii KB "Decode 专项 Attention" §04).
//
// A row of D floats is read by D/4 lanes (16 bytes each). SG groups of such
// lanes share the row's splits (split s goes to group s % SG); each lane folds
// its splits in one pass, rebasing its running sums whenever a larger maximum
// arrives, and the SG partial states are then merged through LDS the same way.
// A split whose m (lse) is -inf weighs exactly 0; a row whose splits are all
// empty gives O = 0 and LSE = -inf. Every sum has a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "fd.h"

namespace fd {

typedef float mf32x4 __attribute__((ext_vector_type(4)));

struct RowState {
  mf32x4 acc;
  float m;
  float den;
};

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
    st.acc = st.acc * a + u * w;
    st.den = st.den * a + ls * w;
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

__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fold_splits for states published in the same launch: device-coherent loads,
// eight splits in flight per lane.
template <int D>
__device__ __forceinline__ RowState fold_splits_coherent(const float* ws, const float* stats, int S, bool uml,
                                                         int grp, int SG) {
  const int sstride = uml ? 2 : 1;
  RowState st;
  st.acc = mf32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.den = 0.f;
#pragma unroll 8
  for (int s = grp; s < S; s += SG) {
    const float ms = coherent_load(stats + s * sstride);
    const float ls = uml ? coherent_load(stats + s * sstride + 1) : 1.f;
    const float* u4 = ws + (int64_t)s * D;
    const mf32x4 u = {coherent_load(u4), coherent_load(u4 + 1), coherent_load(u4 + 2), coherent_load(u4 + 3)};
    const bool valid = ms != -INFINITY;
    const float mn = valid ? fmaxf(st.m, ms) : st.m;
    const float a = st.m == -INFINITY ? 0.f : expf(st.m - mn);
    const float w = valid ? expf(ms - mn) : 0.f;
    st.acc = st.acc * a + u * w;
    st.den = st.den * a + ls * w;
    st.m = mn;
  }
  return st;
}

// Fused merge at the end of a split workgroup (or of one piece of it) (the "last CTA merges" variant of
// the kanthi.in chapter's decode contract). Every workgroup of a (sequence,
// KV head) group has written its split states with ws_store(..., true); once
// its own stores have completed (s_waitcnt) the workgroup counts itself in
// with a device-scope atomic, and the one that arrives as number `expected`
// (the group's writer count) reads the group's
// states back with device-coherent loads, merges the g rows into out/lse and
// resets the counter to 0 so the next stream-ordered call starts from zero.
template <int D, int NTHREADS>
__device__ __forceinline__ void fused_group_merge(const SplitParams& p, int b, int kvh, int expected) {
  __shared__ int s_last;
  __shared__ mf32x4 part[NTHREADS];
  __shared__ float part_m[NTHREADS];
  __shared__ float part_d[NTHREADS];
  __builtin_amdgcn_s_waitcnt(0);            // this thread's state stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(p.counters + (int64_t)b * p.Hkv + kvh, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (unsigned)(expected - 1);
  }
  __syncthreads();
  if (!s_last) return;

  constexpr int LPR = D / 4;
  constexpr int ROWS_PER_PASS = NTHREADS / LPR;
  const bool uml = p.ws_format == FD_WS_UML;
  for (int r0 = 0; r0 < p.R; r0 += ROWS_PER_PASS) {       // the group's rows, a block of them at a time
    const int g = p.R - r0 < ROWS_PER_PASS ? p.R - r0 : ROWS_PER_PASS;
    const int SG = 1 << split_groups_log2(p.S, LPR, g, NTHREADS);
    const int tpr = LPR * SG;
    const int h = threadIdx.x / tpr;
    const int t = threadIdx.x - h * tpr;
    const int grp = t / LPR;
    const int dl = t - grp * LPR;
    const bool active = h < g;
    const int64_t row = state_row(p, b, kvh, r0 + (active ? h : 0));

    RowState st = {mf32x4{0.f, 0.f, 0.f, 0.f}, -INFINITY, 0.f};
    if (active)
      st = fold_splits_coherent<D>(p.ws_o + row * p.S * D + dl * 4, p.ws_stats + row * p.S * (uml ? 2 : 1), p.S,
                                   uml, grp, SG);
    if (r0 > 0) __syncthreads();                           // the previous block's reads of part[] are done
    part[threadIdx.x] = st.acc;
    part_m[threadIdx.x] = st.m;
    part_d[threadIdx.x] = st.den;
    __syncthreads();
    if (active && grp == 0)
      finish_row(part, part_m, part_d, h * tpr + dl, LPR, SG, p.out + row * D, dl, p.lse ? p.lse + row : nullptr);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(p.counters + (int64_t)b * p.Hkv + kvh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace fd
