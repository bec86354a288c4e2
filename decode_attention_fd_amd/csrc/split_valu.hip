// Split kernel on the vector ALUs: a piece of one (sequence, KV head) segment
// per workgroup of 4 waves (one split under the uniform schedule, a walk over
// an equal share under the balanced one, balance.h), for MHA (g = 1), small
// groups and fp32 caches; the R = g * q_len query rows (<= 4) of a group are
// the kernel's rows, each masking the tokens its block row may not see.
//
// A K/V row of D elements is spread over LPR lanes, 16 bytes per lane, so one
// wave load instruction reads RPI = 64 / LPR whole rows (coalesced). Each lane
// forms its partial dot products with the q slice it holds (v_dot2_f32_f16 /
// v_dot2_f32_bf16 on packed 16-bit pairs, fp32 FMA otherwise) and the LPR
// partials are summed by a DPP butterfly (quad_perm, row_half_mirror,
// row_mirror) that leaves the full score in every lane of the row. Every row
// group of LPR lanes keeps its own fp32 online-softmax state for the tokens
// it sees ("Flash-Decoding: Split-KV Attention for Long-Context Decode",
// kanthi.in, §4 kernel 1 loop), so the loop needs no cross-row traffic and no
// barrier; the NW x RPI states are merged exactly at the end (§2 stable form).
// Where a row group has seen only masked tokens its max stays -inf and the
// rescale uses 0 as the reference, so e^(-inf - (-inf)) is never formed
// (xuujii KB "Decode 专项 Attention" §06).
#include <hip/hip_runtime.h>
#include <math.h>

#include "fd_internal.h"
#include "geometry.h"
#include "merge_rows.h"
#include "balance.h"
#include "stamps.h"

namespace fd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NW = kSplitWaves;
constexpr int FUSED_BATCH = 8;   // splits per lane in flight in the fused merge
constexpr int U = kValuLoadsPerTile;   // load instructions per tile per tensor
constexpr float LN2 = 0.69314718055994530942f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes; every lane of a group gets the same value.
template <int LPR>
__device__ __forceinline__ float rowsum(float x) {
  x += dpp<0xB1>(x);                      // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                      // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);                     // row_half_mirror: quad sums of the other quad
  if (LPR >= 16) x += dpp<0x140>(x);      // row_mirror: the other half-row
  if (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Partial dot product of a 16-byte K slice with the matching q slice.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int EPL = 4;
  typedef u32x4 QPack;
  static __device__ __forceinline__ float dot(const QPack& q, const u32x4& k) {
    float a = __uint_as_float(q[0]) * __uint_as_float(k[0]);
    a = fmaf(__uint_as_float(q[1]), __uint_as_float(k[1]), a);
    a = fmaf(__uint_as_float(q[2]), __uint_as_float(k[2]), a);
    a = fmaf(__uint_as_float(q[3]), __uint_as_float(k[3]), a);
    return a;
  }
  static __device__ __forceinline__ float get(const u32x4& v, int e) { return __uint_as_float(v[e]); }
};
// The 16-bit dots bit-cast the whole 16-byte slice and pick pairs with
// __builtin_shufflevector: bit-casting single words of a vector held by
// reference compiled all four pairs to the first one.
template <> struct Elt<_Float16> {
  static constexpr int EPL = 8;
  typedef u32x4 QPack;
  static __device__ __forceinline__ float dot(const QPack& q, const u32x4& k) {
    const f16x8 a = __builtin_bit_cast(f16x8, q), b = __builtin_bit_cast(f16x8, k);
    float r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), 0.f, false);
    r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), r, false);
    r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), r, false);
    r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), r, false);
    return r;
  }
  static __device__ __forceinline__ float get(const u32x4& v, int e) {
    const f16x8 h = __builtin_bit_cast(f16x8, v);
    return (float)h[e];
  }
};
template <> struct Elt<__bf16> {
  static constexpr int EPL = 8;
  typedef u32x4 QPack;
  static __device__ __forceinline__ float dot(const QPack& q, const u32x4& k) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, q), b = __builtin_bit_cast(bf16x8, k);
    float r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1),
                                              0.f, false);
    r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), r,
                                        false);
    r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), r,
                                        false);
    r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), r,
                                        false);
    return r;
  }
  static __device__ __forceinline__ float get(const u32x4& v, int e) {
    const unsigned w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

template <int D, typename T> struct VGeo {
  static constexpr int EPL = Elt<T>::EPL;
  static constexpr int LPR = D / EPL;        // lanes per row
  static constexpr int RPI = 64 / LPR;       // rows per load instruction
  static constexpr int TT = U * RPI;         // tokens per wave tile
  static constexpr int ELT = sizeof(T);
  static_assert(TT == valu_tile_tokens_for(D, sizeof(T)), "planner and kernel tile sizes differ");
};

template <int D, typename T, int G> struct VSmem {
  float st_o[NW][VGeo<D, T>::RPI][G][D];
  float st_m[NW][VGeo<D, T>::RPI][G];
  float st_l[NW][VGeo<D, T>::RPI][G];
};

// Tokens [start, end) of segment (b, kvh) (possibly empty) for the R query
// rows of the group; the state goes to split slot `slot`, or, with `direct`
// (the segment's only piece, fused call), straight to out/lse. Block row i
// sees tokens below vis0 + i.
template <int D, typename T, int G, bool PAGED>
__device__ __forceinline__ void valu_piece(const SplitParams& p, VSmem<D, T, G>& sm, int b, int kvh, int start,
                                           int end, int slot, int vis0, bool direct) {
  using VG = VGeo<D, T>;
  constexpr int EPL = VG::EPL, LPR = VG::LPR, RPI = VG::RPI, TT = VG::TT;
  auto& st_o = sm.st_o;
  auto& st_m = sm.st_m;
  auto& st_l = sm.st_l;

  const int s = slot;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int g = p.g;
  const int R = p.R;             // query rows of the group: g heads x q_len block rows (<= G)
  const int rg = lane / LPR;     // row group
  const int li = lane % LPR;     // lane inside the row
  const int ntiles = end > start ? (end - start + TT - 1) / TT : 0;

  // q slices of the R query rows of this group (row r: block row r / g, head
  // r % g; rows >= R read as zero). Block row i sees tokens below vis0 + i.
  const int mask_from = min(end, vis0);
  u32x4 q[G];
  int row_end[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int r = h < R ? h : 0;
    const int i = r / g;
    const T* qrow = reinterpret_cast<const T*>(p.q) + (int64_t)b * p.q_sb + (int64_t)i * p.q_sq +
                    (int64_t)(kvh * g + r - i * g) * p.q_sh;
    u32x4 v = *reinterpret_cast<const u32x4*>(qrow + li * EPL);
    q[h] = h < R ? v : u32x4{0u, 0u, 0u, 0u};
    row_end[h] = min(end, vis0 + i);
  }

  const char* kbase;
  const char* vbase;
  int64_t row_stride;
  if (!PAGED) {
    const int64_t off = ((int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh) * VG::ELT;
    kbase = reinterpret_cast<const char*>(p.k) + off;
    vbase = reinterpret_cast<const char*>(p.v) + off;
    row_stride = p.kv_st * VG::ELT;
  } else {
    kbase = reinterpret_cast<const char*>(p.k) + (int64_t)kvh * p.pool_sh * VG::ELT;
    vbase = reinterpret_cast<const char*>(p.v) + (int64_t)kvh * p.pool_sh * VG::ELT;
    row_stride = p.pool_st * VG::ELT;
  }
  const int32_t* bt_row = PAGED ? p.block_table + (int64_t)b * p.bt_sb : nullptr;
  const int page_mask = (1 << p.page_log2) - 1;
  auto page_ids = [&](int t0) -> int {
    int t = t0 + (lane < U ? lane : 0) * RPI;
    t = t < end - 1 ? t : end - 1;
    int pid = bt_row[t >> p.page_log2];
    return pid < 0 ? 0 : (pid >= p.num_pages ? p.num_pages - 1 : pid);
  };
  auto offset = [&](int t0, int u, int pids) -> int64_t {
    int t = t0 + u * RPI + rg;
    t = t < end - 1 ? t : end - 1;
    int64_t off;
    if (!PAGED) {
      off = (int64_t)t * row_stride;
    } else {
      const int pid = __builtin_amdgcn_readlane(pids, u);
      off = (int64_t)pid * p.pool_sp * VG::ELT + (int64_t)(t & page_mask) * row_stride;
    }
    return off + li * 16;
  };

  u32x4 kb[U], vb[U];
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const float c2 = p.scale_log2;

  // Loads are unconditional (addresses of rows past the piece are clamped to
  // its last row) and the wave's last tile is peeled off the loop, so the
  // wait-count analysis knows exactly which loads are in flight and never has
  // to drain them all inside the loop.
  const int my_tiles = wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0;
  int tile = wave;
  int pid_cur = 0, pid_next = 0;
  if (my_tiles > 0) {
    const int t0 = start + tile * TT;
    if (PAGED) {
      pid_cur = page_ids(t0);
      pid_next = page_ids(t0 + NW * TT);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = offset(t0, u, pid_cur);
      kb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off));
      vb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
    }
  }

  // One tile; with `more` the wave's next tile (tile + NW) exists and is
  // requested: K after the scores, V after the PV update.
  auto step = [&](int tile, bool more) {
    const int t0 = start + tile * TT;
    const int tn0 = t0 + NW * TT;
    // Paged: the block-table entries of the tile after next are requested
    // before the next tile's K/V loads; loads complete in order, so they have
    // arrived once that K tile has, and requesting K never waits for a V tile.
    int pid_after = 0;
    if (PAGED && more) pid_after = page_ids(tn0 + NW * TT);

    float x[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) x[h][u] = Elt<T>::dot(q[h], kb[u]);
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) kb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + offset(tn0, u, pid_next)));
    }
    const bool tail = t0 + TT > mask_from;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float v = rowsum<LPR>(x[h][u]) * c2;
        if (tail && t0 + u * RPI + rg >= row_end[h]) v = -INFINITY;
        x[h][u] = v;
      }

    float mnew[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = x[h][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, x[h][u]);
      mnew[h] = fmaxf(m[h], mt);
      grow |= mnew[h] > m[h];
    }
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ref = mnew[h] == -INFINITY ? 0.f : mnew[h];
        const float alpha = exp2_fast(m[h] - ref);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        m[h] = mnew[h];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ref = m[h] == -INFINITY ? 0.f : m[h];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        x[h][u] = exp2_fast(x[h][u] - ref);
        ps += x[h][u];
      }
      l[h] += ps;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = Elt<T>::get(vb[u], e);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(x[h][u], v, acc[h][e]);
      }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) vb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + offset(tn0, u, pid_next)));
      if (PAGED) pid_next = pid_after;
    }
  };
  for (int it = 0; it + 1 < my_tiles; ++it, tile += NW) step(tile, true);
  if (my_tiles > 0) step(tile, false);
  FD_DEBUG_WG_BARRIER();                // every wave done with the stream, before the states go to LDS

  // ---- row-group states -> LDS, then one exact merge per (head, dim)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) st_o[wave][rg][h][li * EPL + e] = acc[h][e];
    if (li == 0) {
      st_m[wave][rg][h] = m[h];
      st_l[wave][rg][h] = l[h];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < R * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int r = 0; r < RPI; ++r) M = fmaxf(M, st_m[w][r][h]);
    float Uv = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int r = 0; r < RPI; ++r) {
          const float mw = st_m[w][r][h];
          const float a = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
          Uv += a * st_o[w][r][h][d];
          L += a * st_l[w][r][h];
        }
    }
    const int64_t row = state_row(p, b, kvh, h);
    const int64_t base = row * p.S + s;
    const bool co = p.fused != 0;
    if (direct) {                              // one split: the state is the row's result
      const bool empty = !(L > 0.f);
      p.out[row * D + d] = empty ? 0.f : Uv / L;
      if (d == 0 && p.lse) p.lse[row] = empty ? -INFINITY : (M + log2f(L)) * LN2;
    } else if (p.ws_format == FD_WS_UML) {
      ws_store(p.ws_o + base * D + d, Uv, co);
      if (d == 0) {
        ws_store(p.ws_stats + base * 2, M == -INFINITY ? -INFINITY : M * LN2, co);
        ws_store(p.ws_stats + base * 2 + 1, L, co);
      }
    } else {
      const bool empty = !(L > 0.f);
      ws_store(p.ws_o + base * D + d, empty ? 0.f : Uv / L, co);
      if (d == 0) ws_store(p.ws_stats + base, empty ? -INFINITY : (M + log2f(L)) * LN2, co);
    }
  }
  FD_DEBUG_WG_BARRIER();                // the states read from LDS, before any later reuse
}

// Uniform schedule: workgroup (s, kvh, b) owns split s of segment (b, kvh).
template <int D, typename T, int G, bool PAGED>
__global__ __launch_bounds__(NW * 64) void split_valu_kernel(SplitParams p) {
  __shared__ VSmem<D, T, G> sm;
  WgStamp stamp;
  stamp_begin(p, stamp);
  const int s = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  int seq_len = p.seq_lens[b];
  seq_len = seq_len < 0 ? 0 : (seq_len > p.cap_tokens ? p.cap_tokens : seq_len);
  // Split s covers [s0, s0 + len) clamped to the sequence, with even- and
  // odd-numbered splits of chunk and chunk_odd tokens; formed in 64 bits (the
  // plan bounds the splits' end by INT32_MAX, but a start past the sequence
  // must never wrap to a negative token index).
  const int64_t s0 = (int64_t)(s >> 1) * ((int64_t)p.chunk + p.chunk_odd) + ((s & 1) ? p.chunk : 0);
  const int64_t len = (s & 1) ? p.chunk_odd : p.chunk;
  const int start = (int)(s0 < seq_len ? s0 : seq_len);
  const int end = (int)(s0 + len < seq_len ? s0 + len : seq_len);
  const bool direct = p.fused && p.S == 1;    // fused call with one split: write out/lse directly
  valu_piece<D, T, G, PAGED>(p, sm, b, kvh, start, end, s, seq_len - (p.q_len - 1), direct);
  if (end > start) stamp_piece(stamp, end - start);
  if (p.fused && !direct) fused_group_merge<D, NW * 64, FUSED_BATCH>(p, b, kvh, p.S);
  stamp_end(p, stamp);
}

// Balanced schedule: workgroup w owns an equal share of the batch's granules.
template <int D, typename T, int G, bool PAGED>
__global__ __launch_bounds__(NW * 64) void split_valu_balanced_kernel(SplitParams p) {
  __shared__ VSmem<D, T, G> sm;
  WgStamp stamp;
  stamp_begin(p, stamp);
  balanced_walk<NW * 64>(
      p,
      [&](int b, int kvh, int start, int end, int slot, int count, bool last, int len) {
        b = __builtin_amdgcn_readfirstlane(b);
        kvh = __builtin_amdgcn_readfirstlane(kvh);
        start = __builtin_amdgcn_readfirstlane(start);
        end = __builtin_amdgcn_readfirstlane(end);
        slot = __builtin_amdgcn_readfirstlane(slot);
        if (slot >= p.S) return;                 // lengths differ from the plan's: write nothing
        const bool direct = p.fused && count == 1;
        valu_piece<D, T, G, PAGED>(p, sm, b, kvh, start, end, slot, len - (p.q_len - 1), direct);
        stamp_piece(stamp, end - start);
        if (!direct) {
          if (last) write_neutral<D, NW * 64>(p, b, kvh, slot + 1, p.S);
          if (p.fused) fused_group_merge<D, NW * 64, FUSED_BATCH>(p, b, kvh, count < p.S ? count : p.S);
        }
        __syncthreads();                         // LDS is reused by the next piece
      },
      [&](int b) { empty_row<D, NW * 64>(p, b); });
  stamp_end(p, stamp);
}

template <int D, typename T, int G>
int launch_g(const SplitParams& p, bool paged, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.nwg > 0) {
    if (paged)
      hipLaunchKernelGGL((split_valu_balanced_kernel<D, T, G, true>), dim3(p.nwg), dim3(NW * 64), 0, st, p);
    else
      hipLaunchKernelGGL((split_valu_balanced_kernel<D, T, G, false>), dim3(p.nwg), dim3(NW * 64), 0, st, p);
  } else {
    dim3 grid(p.S, p.Hkv, p.B);
    if (paged)
      hipLaunchKernelGGL((split_valu_kernel<D, T, G, true>), grid, dim3(NW * 64), 0, st, p);
    else
      hipLaunchKernelGGL((split_valu_kernel<D, T, G, false>), grid, dim3(NW * 64), 0, st, p);
  }
  return (int)hipGetLastError();
}

template <int D, typename T, int G>
int occupancy_g(bool paged, int* out) {
  if (paged) return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(out, split_valu_kernel<D, T, G, true>, NW * 64, 0);
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(out, split_valu_kernel<D, T, G, false>, NW * 64, 0);
}

template <int D, typename T>
int occupancy_t(bool paged, int group_tpl, int* out) {
  switch (group_tpl) {
    case 1: return occupancy_g<D, T, 1>(paged, out);
    case 2: return occupancy_g<D, T, 2>(paged, out);
    case 4: return occupancy_g<D, T, 4>(paged, out);
    default: return (int)hipErrorInvalidValue;
  }
}

template <int D, typename T>
int launch_t(const SplitParams& p, bool paged, int group_tpl, void* stream) {
  switch (group_tpl) {
    case 1: return launch_g<D, T, 1>(p, paged, stream);
    case 2: return launch_g<D, T, 2>(p, paged, stream);
    case 4: return launch_g<D, T, 4>(p, paged, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_split_valu(const SplitParams& p, int head_dim, int kv_dtype, int layout, int group_tpl,
                      void* stream) {
  const bool paged = layout == FD_LAYOUT_PAGED;
  if (head_dim == 128) {
    if (kv_dtype == FD_DTYPE_F32) return launch_t<128, float>(p, paged, group_tpl, stream);
    if (kv_dtype == FD_DTYPE_F16) return launch_t<128, _Float16>(p, paged, group_tpl, stream);
    if (kv_dtype == FD_DTYPE_BF16) return launch_t<128, __bf16>(p, paged, group_tpl, stream);
  } else if (head_dim == 64) {
    if (kv_dtype == FD_DTYPE_F32) return launch_t<64, float>(p, paged, group_tpl, stream);
    if (kv_dtype == FD_DTYPE_F16) return launch_t<64, _Float16>(p, paged, group_tpl, stream);
    if (kv_dtype == FD_DTYPE_BF16) return launch_t<64, __bf16>(p, paged, group_tpl, stream);
  }
  return (int)hipErrorInvalidValue;
}

int occupancy_split_valu(int head_dim, int kv_dtype, int layout, int group_tpl, int* out) {
  const bool paged = layout == FD_LAYOUT_PAGED;
  if (head_dim == 128) {
    if (kv_dtype == FD_DTYPE_F32) return occupancy_t<128, float>(paged, group_tpl, out);
    if (kv_dtype == FD_DTYPE_F16) return occupancy_t<128, _Float16>(paged, group_tpl, out);
    if (kv_dtype == FD_DTYPE_BF16) return occupancy_t<128, __bf16>(paged, group_tpl, out);
  } else if (head_dim == 64) {
    if (kv_dtype == FD_DTYPE_F32) return occupancy_t<64, float>(paged, group_tpl, out);
    if (kv_dtype == FD_DTYPE_F16) return occupancy_t<64, _Float16>(paged, group_tpl, out);
    if (kv_dtype == FD_DTYPE_BF16) return occupancy_t<64, __bf16>(paged, group_tpl, out);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace fd
