// Split kernel, packed-GQA tile on MFMA (gfx950), 16-bit K/V.
//
// One workgroup of 4 waves processes a piece of one (sequence b, KV head)
// segment for the g query heads that share the KV head, times the q_len rows
// of a short query block ("Flash-Decoding: Split-KV Attention for Long-Context
// Decode", kanthi.in, §1 GQA note: the query heads of a group are the rows of
// one tile so each KV block is read once per group; §7 short query blocks).
// Under the uniform schedule the piece is split s, [s*chunk, min(s*chunk +
// chunk, seq_len)) (§4 kernel 1); under the balanced schedule (balance.h) a
// workgroup walks the pieces of its equal share of the batch. A piece's
// 32-token wave tiles are dealt round-robin to the 4 waves; each wave runs its
// own fp32 online softmax (§4 kernel 1 loop; the recurrence of Milakov &
// Gimelshein) with no barrier inside the loop, and the four wave states are
// merged once at the end with the exact rescaled merge (§2 stable form).
//
// Per wave tile of 32 tokens:
//   * K and V rows are fetched with fully coalesced 16-byte nontemporal loads
//     (a wave instruction reads whole rows; the address is one scalar base per
//     instruction plus a constant lane offset; every byte is read once, so the
//     loads are marked streaming) into registers, one tile ahead of use, and
//     written to the wave's own LDS slice; K and V are staggered so the wave
//     always has loads in flight. Rows are padded by 16
//     bytes so the 16 rows one MFMA operand read touches fall in distinct bank
//     groups, while every LDS access is one base register plus an immediate.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16}: A = 16 tokens x 32 dims of
//     K, B = 32 dims x 16 query columns. Columns 0..R-1 hold the R = g * q_len
//     query rows (column c: block row c / g, head c % g); columns R..2R-1 hold
//     the same rows again; the rest are zero. Each column masks the tokens its
//     block row may not see.
//   * Online softmax in base 2: x = (q.k) * scale * log2(e); the running max
//     is exchanged across the four 16-lane groups; p = 2^(x - m).
//   * O^T += V^T P^T on the same MFMA: the S^T accumulator layout is already
//     the B-operand layout of P^T once the token order inside the 32-token
//     k-block is permuted the same way on the V side, so P never leaves
//     registers. On the V side each lane reads one contiguous D/8-byte slice
//     of a token row; output block e then holds dims d = (D/16)*m + e, so one
//     read feeds all D/16 MFMAs. P is split into a 16-bit high part (columns
//     < R) and the 16-bit rounding of its remainder (columns R..2R-1); the two
//     output columns are summed at the end, so P keeps ~22 (f16) / ~16 (bf16)
//     bits. The row sum l is accumulated from the unrounded fp32 p.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fd_internal.h"
#include "geometry.h"
#include "merge_rows.h"
#include "balance.h"
#include "stamps.h"

namespace fd {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;
template <> struct Mma<_Float16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

constexpr int NW = kSplitWaves;   // waves per workgroup
constexpr int FUSED_BATCH = 16;   // splits per lane in flight in the fused merge
constexpr int TT = kMfmaTileTokens;   // tokens per wave tile
constexpr float LN2 = 0.69314718055994530942f;

template <int D> struct Geo {
  static constexpr int ROWB = D * 2;        // bytes per K/V row
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row (16 or 8)
  static constexpr int RPI = 64 / CPR;      // rows per wave load instruction (4 or 8)
  static constexpr int NI = TT / RPI;       // load instructions per tile per tensor (8 or 4)
  static constexpr int ROWP = ROWB + 16;    // padded LDS row pitch
  static constexpr int TILEB = TT * ROWP;   // bytes of one K (or V) tile in LDS
  static constexpr int NDC = D / 32;        // QK^T k-blocks of 32 dims
  static constexpr int NDB = D / 16;        // PV output blocks (dims d = NDB*m + e)
  static constexpr int VW = NDB / 2;        // dwords of V one lane reads per token (4 or 2)
  static constexpr int OWP = D + 4;         // floats per column of a wave state in LDS: the 16
                                            // columns of one store fall on different banks
};

template <int N> struct VRead;
template <> struct VRead<4> { typedef u32x4 type; };
template <> struct VRead<2> { typedef u32x2 type; };

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Half `e & 1` of a and of b packed into one word (a's in the low half).
__device__ __forceinline__ unsigned pick_half(unsigned a, unsigned b, int e) {
  return (e & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u) : __builtin_amdgcn_perm(b, a, 0x05040100u);
}

template <int D> struct Smem {
  unsigned char lds[NW][2][Geo<D>::TILEB];
  float st_m[NW][32];
  float st_l[NW][32];
};

// Tokens [start, end) of segment (b, kvh), end > start, for the R = g * q_len
// query rows of the group (row r: block row r / g, head r % g); the state goes
// to split slot `slot`, or, with `direct` (the segment's only piece, fused
// call), straight to out/lse as the finished rows. Block row i sees tokens
// below vis0 + i (vis0 = seq_len - (q_len - 1)). NCT column tiles of the MFMA
// B operand: with NCT = 1 columns 0..R-1 hold rows 0..R-1 (R <= 8); with
// NCT = 2 tile ct holds rows 8*ct .. 8*ct + 7 (R <= 16). Within a tile of RT
// rows, columns RT..2RT-1 repeat them for the low half of P.
template <int D, typename T, bool PAGED, int NCT>
__device__ __forceinline__ void split_piece(const SplitParams& p, Smem<D>& sm, int b, int kvh, int start, int end,
                                            int slot, int vis0, bool direct) {
  using G = Geo<D>;
  using V8 = typename Mma<T>::vec;
  using VR = typename VRead<G::VW>::type;
  FD_DEBUG_WG_BARRIER();                // every thread calls split_piece
  auto& lds = sm.lds;
  auto& st_m = sm.st_m;
  auto& st_l = sm.st_l;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int g = p.g;
  const int R = p.R;             // query rows of the group (g heads x q_len block rows)
  const int col = lane & 15;     // MFMA column = query column
  const int grp = lane >> 4;     // 16-lane group
  const int ntiles = (end - start + TT - 1) / TT;

  // ---- Q^T as the B operand of S^T = K Q^T, one column tile at a time.
  const int mask_from = min(end, vis0);                       // first token any column may not see
  int RT[NCT];                                                // rows of tile ct
  int col_end[NCT];                                           // first token column col of tile ct may not see
  V8 qb[NCT][G::NDC];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    RT[ct] = NCT == 1 ? R : min(8, R - 8 * ct);
    const int hc = col < RT[ct] ? col : (col < 2 * RT[ct] ? col - RT[ct] : -1);
    const int r = hc < 0 ? R - 1 : 8 * ct + hc;              // state row of this column
    const int qi = r / g;                                     // its block row
    col_end[ct] = min(end, vis0 + qi);
    const T* qrow = reinterpret_cast<const T*>(p.q) + (int64_t)b * p.q_sb + (int64_t)qi * p.q_sq +
                    (int64_t)(kvh * g + r - qi * g) * p.q_sh;
#pragma unroll
    for (int c = 0; c < G::NDC; ++c) {
      V8 v = *reinterpret_cast<const V8*>(qrow + 32 * c + 8 * grp);
      qb[ct][c] = hc < 0 ? V8{} : v;
    }
  }

  // ---- addressing: byte offsets, d contiguous
  const char* kbase;
  const char* vbase;
  int64_t row_stride;                 // bytes between consecutive tokens (inside a page if paged)
  int64_t page_stride = 0;
  if (!PAGED) {
    const int64_t off = ((int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh) * 2;
    kbase = reinterpret_cast<const char*>(p.k) + off;
    vbase = reinterpret_cast<const char*>(p.v) + off;
    row_stride = p.kv_st * 2;
  } else {
    kbase = reinterpret_cast<const char*>(p.k) + (int64_t)kvh * p.pool_sh * 2;
    vbase = reinterpret_cast<const char*>(p.v) + (int64_t)kvh * p.pool_sh * 2;
    row_stride = p.pool_st * 2;
    page_stride = p.pool_sp * 2;
  }
  const int lrow = lane / G::CPR;           // row of this lane inside a load instruction
  const int lchunk = lane % G::CPR;         // 16-byte chunk of this lane
  const uint32_t lane_off = (uint32_t)(lrow * row_stride) + lchunk * 16;
  const int32_t* bt_row = PAGED ? p.block_table + (int64_t)b * p.bt_sb : nullptr;
  const int page_mask = (1 << p.page_log2) - 1;

  // Page id for load instruction `lane` of the tile starting at `t0` (lanes >= NI unused).
  auto page_ids = [&](int t0) -> int {
    int t = t0 + (lane < G::NI ? lane : 0) * G::RPI;
    t = t < end - 1 ? t : end - 1;
    int pid = bt_row[t >> p.page_log2];
    pid = pid < 0 ? 0 : (pid >= p.num_pages ? p.num_pages - 1 : pid);
    return pid;
  };

  // Loads of one tensor's tile starting at t0 into r. Instruction i reads rows
  // t0 + i*RPI + [0, RPI); rows past `end` (tail tile only) re-read row end-1.
  auto issue = [&](u32x4 (&r)[G::NI], const char* base, int t0, int pids) {
    const bool full = t0 + TT <= end;               // wave-uniform
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int ti = t0 + i * G::RPI;               // first row of the instruction (uniform)
      const int tu = ti < end - 1 ? ti : end - 1;
      int64_t ubase;                                // uniform byte offset of row tu
      if (!PAGED) {
        ubase = (int64_t)tu * row_stride;
      } else {
        const int pid = __builtin_amdgcn_readlane(pids, i);
        ubase = (int64_t)pid * page_stride + (int64_t)(tu & page_mask) * row_stride;
      }
      uint32_t loff = lane_off;
      if (!full) {
        const int t = ti + lrow;
        const int tc = t < end - 1 ? t : end - 1;
        loff = (uint32_t)((tc - tu) * row_stride) + lchunk * 16;
      }
      r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + ubase + loff));
    }
  };

  unsigned char* ldsK = lds[wave][0];
  unsigned char* ldsV = lds[wave][1];
  auto store = [&](const u32x4 (&r)[G::NI], unsigned char* dst) {
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
      *reinterpret_cast<u32x4*>(dst + (i * G::RPI + lrow) * G::ROWP + lchunk * 16) = r[i];
  };

  f32x4 oacc[NCT][G::NDB];
  float m_run[NCT];          // running max of x (base-2 scaled scores) for column col of tile ct
  float l_run[NCT];          // this lane's share of the running sum
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) oacc[ct][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
  }
  const float c2 = p.scale_log2;

  // One tile from the wave's LDS slice into the running state.
  auto compute = [&](int t0) {
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    // ---- S^T = K Q^T for tokens [0,16) and [16,32)
    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < G::NDC; ++c) {
        V8 a = *reinterpret_cast<const V8*>(ldsK + (tb * 16 + col) * G::ROWP + (4 * c + grp) * 16);
        sacc[tb] = Mma<T>::run(a, qb[ct][c], sacc[tb]);
      }
    }

    // ---- online softmax (base 2). Lane holds tokens tb*16 + 4*grp + i.
    float x[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[tb * 4 + i] = sacc[tb][i] * c2;
    if (t0 + TT > mask_from) {                // tail tile: mask tokens a column may not see
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + tb * 16 + 4 * grp + i >= col_end[ct]) x[tb * 4 + i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // A column of a query block can see no token of a tile (its max stays
    // -inf): the rescale and the exponent then use safe references, so
    // e^(-inf - (-inf)) is never formed.
    const float m_new = fmaxf(m_run[ct], mt);
    if (__any(m_new > m_run[ct])) {
      const float alpha = m_new > m_run[ct] ? exp2_fast(m_run[ct] - m_new) : 1.f;
      l_run[ct] *= alpha;
#pragma unroll
      for (int i = 0; i < G::NDB; ++i) oacc[ct][i] *= alpha;
      m_run[ct] = m_new;
    }
    const float m_ref = m_run[ct] == -INFINITY ? 0.f : m_run[ct];
    float pe[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = exp2_fast(x[e] - m_ref);
      psum += pe[e];
    }
    l_run[ct] += psum;

    // ---- P^T as the B operand: high part in columns < RT, remainder after.
    V8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const T hi = (T)pe[e];
      const float r = col < RT[ct] ? pe[e] : pe[e] - (float)hi;
      pb[e] = (T)r;
    }

    // ---- O^T += V^T P^T. k index j of group grp is token perm(8*grp + j):
    // j < 4 -> 4*grp + j, j >= 4 -> 16 + 4*grp + (j - 4). Lane (grp, col) reads
    // dims [NDB*col, NDB*col + NDB) of each of its 8 tokens.
    VR w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = j < 4 ? 4 * grp + j : 16 + 4 * grp + (j - 4);
      w[j] = *reinterpret_cast<const VR*>(ldsV + r * G::ROWP + col * (G::NDB * 2));
    }
#pragma unroll
    for (int e = 0; e < G::NDB; ++e) {
      u32x4 a;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) a[jj] = pick_half(w[2 * jj][e >> 1], w[2 * jj + 1][e >> 1], e);
      oacc[ct][e] = Mma<T>::run(__builtin_bit_cast(V8, a), pb, oacc[ct][e]);
    }
  }
  };

  // One register tile per tensor, staggered: the K tile is stored and the next
  // K tile requested before the V tile is stored and the next V tile
  // requested, so this wave always has loads in flight while it writes LDS and
  // while it computes. Tile indices past the split are clamped to its last
  // tile (a reload that hits in cache), so every load is unconditional.
  const int last = ntiles - 1;
  auto tstart = [&](int tile) { return start + (tile < last ? tile : last) * TT; };
  if (ntiles > 0) {
    u32x4 kr[G::NI], vr[G::NI];
    int tile = wave;
    // Paged: the block-table entries of a tile are requested before the K/V
    // loads of the tile before it. Loads complete in order, so they have
    // arrived once that K tile has, and requesting the next K tile never waits
    // for the V tile still in flight.
    int pid = 0, pid_next = 0, pid_after = 0;
    if (PAGED) pid = page_ids(tstart(tile));
    if (PAGED) pid_next = page_ids(tstart(tile + NW));
    issue(kr, kbase, tstart(tile), pid);
    issue(vr, vbase, tstart(tile), pid);
    // One exit at the bottom: the wait-count analysis then sees the same load
    // order on entry and on the back edge.
    const int my_tiles = (ntiles - wave + NW - 1) / NW;     // > 0 only if wave < ntiles
    for (int it = 0; it + 1 < my_tiles; ++it, tile += NW) {
      if (PAGED) pid_after = page_ids(tstart(tile + 2 * NW));
      store(kr, ldsK);
      issue(kr, kbase, tstart(tile + NW), pid_next);
      store(vr, ldsV);
      issue(vr, vbase, tstart(tile + NW), pid_next);
      if (PAGED) pid_next = pid_after;
      FD_DEBUG_WAVE_BARRIER();          // the tile stored, before the wave reads it
      compute(start + tile * TT);
      FD_DEBUG_WAVE_BARRIER();          // the tile read, before the next one overwrites it
    }
    if (my_tiles > 0) {                                     // the wave's last tile: nothing more to request
      store(kr, ldsK);
      store(vr, ldsV);
      FD_DEBUG_WAVE_BARRIER();
      compute(start + tile * TT);
    }
  }
  FD_DEBUG_WAVE_BARRIER();              // the last tile read, before the state overwrites the slice

  // ---- per-wave state -> LDS: tile ct in lds[wave][ct] as ow[column][d],
  // d = NDB*(4*grp + i) + e; statistics at st_m/st_l[wave][16*ct + column]
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float l = l_run[ct];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float* ow = reinterpret_cast<float*>(lds[wave][ct]);   // [16 columns][OWP] fp32 (<= TILEB bytes)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e4 = 0; e4 < G::NDB; e4 += 4) {
        f32x4 v = {oacc[ct][e4][i], oacc[ct][e4 + 1][i], oacc[ct][e4 + 2][i], oacc[ct][e4 + 3][i]};
        *reinterpret_cast<f32x4*>(ow + col * G::OWP + G::NDB * (4 * grp + i) + e4) = v;
      }
    if (grp == 0) {
      st_m[wave][16 * ct + col] = m_run[ct];
      st_l[wave][16 * ct + col] = l;
    }
  }
  __syncthreads();

  // ---- merge the four wave states (exact rescale to the common max) and
  // combine the high/low columns, then write the split's state; a thread
  // takes four consecutive dims of a row.
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < R * D4; idx += NW * 64) {
    const int h = idx / D4;                    // state row
    const int d = (idx - h * D4) * 4;
    const int ct = NCT == 1 ? 0 : h >> 3;      // its column tile
    const int c = NCT == 1 ? h : h & 7;        // and column
    const int rt = NCT == 1 ? R : min(8, R - 8 * ct);
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, st_m[w2][16 * ct + c]);
    f32x4 U = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const float mw = st_m[w2][16 * ct + c];
        const float a = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
        const float* o = reinterpret_cast<const float*>(lds[w2][ct]);
        U += a * (*reinterpret_cast<const f32x4*>(o + c * G::OWP + d) +
                  *reinterpret_cast<const f32x4*>(o + (c + rt) * G::OWP + d));
        L += a * st_l[w2][16 * ct + c];
      }
    }
    const int64_t row = state_row(p, b, kvh, h);
    const int64_t base = row * p.S + slot;
    const bool co = p.fused != 0;
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    if (direct) {                              // one piece: the state is the row's result
      *reinterpret_cast<f32x4*>(p.out + row * D + d) = U * inv;
      if (d == 0 && p.lse) p.lse[row] = empty ? -INFINITY : (M + log2f(L)) * LN2;
    } else {
      const bool uml = p.ws_format == FD_WS_UML;
      const f32x4 v = uml ? U : U * inv;
      float* dst = p.ws_o + base * D + d;
      if (!co) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else if (p.q_len == 1) {
        // One 16-byte device-coherent store (sc1, as ws_store's agent-scope
        // atomic stores) into the group's contiguous block of state rows.
        const float* blk = p.ws_o + state_row(p, b, kvh, 0) * p.S * D;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(blk), (short)0, (int)((int64_t)R * p.S * D * 4),
                                              0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v),
                                               rs, (int)(((int64_t)h * p.S + slot) * D + d) * 4, 0, 16);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ws_store(dst + e, v[e], true);
      }
      if (d == 0) {
        if (uml) {
          ws_store(p.ws_stats + base * 2, M == -INFINITY ? -INFINITY : M * LN2, co);
          ws_store(p.ws_stats + base * 2 + 1, L, co);
        } else {
          ws_store(p.ws_stats + base, empty ? -INFINITY : (M + log2f(L)) * LN2, co);
        }
      }
    }
  }
  FD_DEBUG_WG_BARRIER();                // the states read from LDS, before any later reuse
}

// Uniform schedule: workgroup (s, kvh, b) owns split s of segment (b, kvh).
template <int D, typename T, bool PAGED, int NCT>
__global__ __launch_bounds__(NW * 64) void split_mfma_kernel(SplitParams p) {
  __shared__ Smem<D> sm;
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
  const bool direct = p.fused && p.S == 1;
  if (end > start) {
    split_piece<D, T, PAGED, NCT>(p, sm, b, kvh, start, end, s, seq_len - (p.q_len - 1), direct);
    stamp_piece(stamp, end - start);
  } else if (direct)
    empty_group<D, NW * 64>(p, b, kvh);
  else
    write_neutral<D, NW * 64>(p, b, kvh, s, s + 1);
  if (p.fused && !direct) fused_group_merge<D, NW * 64, FUSED_BATCH>(p, b, kvh, p.S);
  stamp_end(p, stamp);
}

// Balanced schedule: workgroup w owns an equal share of the batch's granules.
template <int D, typename T, bool PAGED, int NCT>
__global__ __launch_bounds__(NW * 64) void split_mfma_balanced_kernel(SplitParams p) {
  __shared__ Smem<D> sm;
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
        split_piece<D, T, PAGED, NCT>(p, sm, b, kvh, start, end, slot, len - (p.q_len - 1), direct);
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

template <int D, typename T, bool PAGED>
int occupancy(int nct, int* out) {
  if (nct == 2)
    return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(out, split_mfma_kernel<D, T, PAGED, 2>, NW * 64, 0);
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(out, split_mfma_kernel<D, T, PAGED, 1>, NW * 64, 0);
}

template <int D, typename T, bool PAGED, int NCT>
int launch_nct(const SplitParams& p, hipStream_t st) {
  if (p.nwg > 0)
    hipLaunchKernelGGL((split_mfma_balanced_kernel<D, T, PAGED, NCT>), dim3(p.nwg), dim3(NW * 64), 0, st, p);
  else
    hipLaunchKernelGGL((split_mfma_kernel<D, T, PAGED, NCT>), dim3(p.S, p.Hkv, p.B), dim3(NW * 64), 0, st, p);
  return (int)hipGetLastError();
}

template <int D, typename T, bool PAGED>
int launch(const SplitParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.R > 16) return (int)hipErrorInvalidValue;
  return p.R > 8 ? launch_nct<D, T, PAGED, 2>(p, st) : launch_nct<D, T, PAGED, 1>(p, st);
}

}  // namespace

int launch_split_mfma(const SplitParams& p, int head_dim, int kv_dtype, int layout, void* stream) {
  const bool paged = layout == FD_LAYOUT_PAGED;
  if (kv_dtype == FD_DTYPE_F16) {
    if (head_dim == 128) return paged ? launch<128, _Float16, true>(p, stream) : launch<128, _Float16, false>(p, stream);
    if (head_dim == 64) return paged ? launch<64, _Float16, true>(p, stream) : launch<64, _Float16, false>(p, stream);
  } else if (kv_dtype == FD_DTYPE_BF16) {
    if (head_dim == 128) return paged ? launch<128, __bf16, true>(p, stream) : launch<128, __bf16, false>(p, stream);
    if (head_dim == 64) return paged ? launch<64, __bf16, true>(p, stream) : launch<64, __bf16, false>(p, stream);
  }
  return (int)hipErrorInvalidValue;
}

// Resident workgroups per CU of the uniform kernel with nct column tiles.
int occupancy_split_mfma(int head_dim, int kv_dtype, int layout, int nct, int* out) {
  const bool paged = layout == FD_LAYOUT_PAGED;
  if (kv_dtype == FD_DTYPE_F16) {
    if (head_dim == 128) return paged ? occupancy<128, _Float16, true>(nct, out) : occupancy<128, _Float16, false>(nct, out);
    if (head_dim == 64) return paged ? occupancy<64, _Float16, true>(nct, out) : occupancy<64, _Float16, false>(nct, out);
  } else if (kv_dtype == FD_DTYPE_BF16) {
    if (head_dim == 128) return paged ? occupancy<128, __bf16, true>(nct, out) : occupancy<128, __bf16, false>(nct, out);
    if (head_dim == 64) return paged ? occupancy<64, __bf16, true>(nct, out) : occupancy<64, __bf16, false>(nct, out);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace fd
