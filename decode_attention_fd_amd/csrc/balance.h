// Balanced split schedule (device side), shared by the two split kernels.
//
// The uniform schedule cuts every (sequence, KV head) segment into splits of
// one fixed chunk; with ragged lengths the launch then holds many workgroups
// of very different sizes and the longest sequences decide the time. The
// pages point at two remedies: a split plan made for the current batch,
// heads and lengths (xuujii KB "Decode 专项 Attention" §07) and Stream-K-style
// work partitioning against wave quantization (LeanAttention, listed in
// "Flash-Decoding: Split-KV Attention for Long-Context Decode", kanthi.in, §7).
//
// Here the whole batch is one line of granules: segment (b, h) is
// cdiv(len_b, G) granules of G tokens followed by piece_cost granules that
// hold no tokens and stand for a piece's start-up cost (q load, first-tile
// latency, epilogue), so a range of many short segments gets fewer tokens;
// segments are in (b, h) order. A grid of N
// workgroups cuts that line into N near-equal ranges, workgroup w taking
// granules [floor(w T / N), floor((w + 1) T / N)) of the T in total; or, with
// x = p.range_odd > 0, ranges of alternating size: w takes 1000 + x (w even)
// or 1000 - x (w odd) parts per 1000 of an equal share, starting at
// floor(c_w T / c_N) with c_w the parts of ranges 0 .. w-1, so that the odd
// XCDs (workgroup w runs on XCD w mod 8), which stream more slowly, get
// less. A range
// may cover the end of one segment and the start of the next; each part of a
// segment it covers is one "piece" and yields one attention state, stored at
// slot w - first(segment) of that segment's rows, where first(x) is the
// workgroup that owns granule x. Every workgroup derives the same line from
// the device seq_lens with one block scan, so no schedule has to be copied to
// the device. The workgroup that owns a segment's last granule also fills the
// segment's unused slots with the neutral state (u = 0, m = -inf, l = 0), and
// the owner of an empty row's position fills all of its slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"
#include "merge_rows.h"

namespace fd {

// Neutral state (u = 0 or o = 0, m = -inf or lse = -inf, l = 0) in split slots
// [s0, s1) of the g * q_len state rows of group (b, kvh).
template <int D, int NTHREADS>
__device__ __forceinline__ void write_neutral(const SplitParams& p, int b, int kvh, int s0, int s1) {
  const int n = s1 - s0;
  if (n <= 0) return;
  const bool co = p.fused != 0;
  const bool uml = p.ws_format == FD_WS_UML;
  const int per_row = n * D;
  for (int i = threadIdx.x; i < p.R * per_row; i += NTHREADS) {
    const int h = i / per_row;
    const int r = i - h * per_row;
    const int s = s0 + r / D;
    const int d = r - (r / D) * D;
    const int64_t base = state_row(p, b, kvh, h) * p.S + s;
    ws_store(p.ws_o + base * D + d, 0.f, co);
    if (d == 0) {
      if (uml) {
        ws_store(p.ws_stats + base * 2, -INFINITY, co);
        ws_store(p.ws_stats + base * 2 + 1, 0.f, co);
      } else {
        ws_store(p.ws_stats + base, -INFINITY, co);
      }
    }
  }
}

// The finished rows of an empty group (b, kvh) in a fused call: O = 0, LSE = -inf.
template <int D, int NTHREADS>
__device__ __forceinline__ void empty_group(const SplitParams& p, int b, int kvh) {
  for (int i = threadIdx.x; i < p.R * D; i += NTHREADS) {
    const int64_t row = state_row(p, b, kvh, i / D);
    p.out[row * D + i % D] = 0.f;
    if (p.lse && i % D == 0) p.lse[row] = -INFINITY;
  }
}

// A row of length 0: with the fused merge its output is written directly
// (O = 0, LSE = -inf); otherwise all of its split slots get the neutral state.
template <int D, int NTHREADS>
__device__ __forceinline__ void empty_row(const SplitParams& p, int b) {
  if (p.fused) {
    const int rows = p.q_len * p.Hq;          // the row's query block, contiguous in out/lse
    for (int i = threadIdx.x; i < rows * D; i += NTHREADS) {
      p.out[(int64_t)b * rows * D + i] = 0.f;
      if (p.lse && i % D == 0) p.lse[(int64_t)b * rows + i / D] = -INFINITY;
    }
  } else {
    for (int kvh = 0; kvh < p.Hkv; ++kvh) write_neutral<D, NTHREADS>(p, b, kvh, 0, p.S);
  }
}

// Parts of ranges 0 .. w-1 when range w has 1000 + x (w even) or 1000 - x (w odd).
__device__ __forceinline__ int64_t range_parts(int64_t w, int64_t x) {
  return (w >> 1) * 2000 + ((w & 1) ? 1000 + x : 0);
}

// First granule of range w of a line of `total` granules cut into `nwg` ranges.
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t total, int64_t nwg, int64_t x) {
  return x == 0 ? w * total / nwg : range_parts(w, x) * total / range_parts(nwg, x);
}

// Workgroup owning granule g: the last range w with range_start(w) <= g. With
// M = range_parts(nwg), floor(c_w total / M) <= g holds exactly when
// c_w <= ceil((g + 1) M / total) - 1 =: c; the last w with c_w <= c is 2 (c div
// 2000), plus one when c mod 2000 reaches an even range's 1000 + x.
__device__ __forceinline__ int64_t granule_owner(int64_t g, int64_t total, int64_t nwg, int64_t x) {
  if (x == 0) return ((g + 1) * nwg + total - 1) / total - 1;
  const int64_t c = ((g + 1) * range_parts(nwg, x) + total - 1) / total - 1;
  const int64_t w = 2 * (c / 2000) + (c % 2000 >= 1000 + x ? 1 : 0);
  return w < nwg - 1 ? w : nwg - 1;
}

__device__ __forceinline__ int clamp_len(const SplitParams& p, int b) {
  const int n = p.seq_lens[b];
  return n < 0 ? 0 : (n > p.cap_tokens ? p.cap_tokens : n);
}

struct BalancedStart {
  int64_t total;     // granules in the line
  int64_t gs, ge;    // this workgroup's range
  int b;             // first row the walk visits
  int64_t x;         // granule where row b starts
};

// Row lengths cached in LDS by balanced_start when the batch has at most
// NTHREADS rows (one row per thread), so the walk does not go back to memory.
template <int NTHREADS> struct BalancedLds {
  int64_t wave_sum[NTHREADS / 64];
  int64_t cand_x[NTHREADS / 64];
  int cand_b[NTHREADS / 64];
  int len[NTHREADS];
};

// Block-wide scan of the row lengths. Thread t sums rows [t*E, t*E + E);
// the per-thread sums are scanned across the block; then the first row that
// starts at or after gs, or ends after gs, is located (the predicate is
// monotone in the row, so the first thread, and in it the first row, that
// satisfies it is the answer). Two barriers. All threads return the same values.
template <int NTHREADS>
__device__ BalancedStart balanced_start(const SplitParams& p, BalancedLds<NTHREADS>& sh) {
  constexpr int NWV = NTHREADS / 64;
  const int B = p.B;
  const int64_t G = p.granule;
  const int64_t H = p.Hkv;
  const int64_t C = p.piece_cost;
  const int E = (B + NTHREADS - 1) / NTHREADS;
  const int r0 = threadIdx.x * E;
  const int r1 = min(B, r0 + E);
  int64_t local = 0;
  int n1 = 0;                          // the row's length when each thread has one row
  for (int r = r0; r < r1; ++r) {
    const int n = clamp_len(p, r);
    if (E == 1) {
      sh.len[threadIdx.x] = n;
      n1 = n;
    }
    const int64_t pl = (n + G - 1) / G;
    local += H * (pl > 0 ? pl + C : 0);
  }

  // inclusive scan inside the wave, then across the waves
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sh.wave_sum[wave] = incl;
  __syncthreads();
  int64_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    before += i < wave ? sh.wave_sum[i] : 0;
    total += sh.wave_sum[i];
  }
  const int64_t nwg = gridDim.x;
  const int64_t w = blockIdx.x;
  const int64_t gs = range_start(w, total, nwg, p.range_odd);
  const int64_t ge = range_start(w + 1, total, nwg, p.range_odd);

  int64_t x = before + incl - local;   // start of row r0
  int cand = B;
  int64_t cand_x = 0;
  for (int r = r0; r < r1; ++r) {
    const int64_t pl = ((E == 1 ? n1 : clamp_len(p, r)) + G - 1) / G;   // no second read of seq_lens
    const int64_t xn = x + H * (pl > 0 ? pl + C : 0);
    if (x >= gs || xn > gs) {
      cand = r;
      cand_x = x;
      break;
    }
    x = xn;
  }
  const uint64_t mask = __ballot(cand < B);
  const int first = mask ? __ffsll((unsigned long long)mask) - 1 : 0;
  if (lane == first) {
    sh.cand_b[wave] = cand;
    sh.cand_x[wave] = cand_x;
  }
  __syncthreads();
  BalancedStart st;
  st.total = total;
  st.gs = gs;
  st.ge = ge;
  st.b = B;
  st.x = total;
#pragma unroll
  for (int i = NWV - 1; i >= 0; --i)
    if (sh.cand_b[i] < B) {
      st.b = sh.cand_b[i];
      st.x = sh.cand_x[i];
    }
  st.b = __builtin_amdgcn_readfirstlane(st.b);
  return st;
}

// Walk this workgroup's range. piece(b, kvh, start, end, slot, count, last,
// len) handles tokens [start, end) of segment (b, kvh) of a row of length
// len: its state goes to `slot`, the segment has `count` pieces in all, and
// `last` says that this workgroup holds the segment's final granule. empty_row(b) handles a row of length 0
// whose position this workgroup owns.
template <int NTHREADS, typename Piece, typename EmptyRow>
__device__ __forceinline__ void balanced_walk(const SplitParams& p, Piece&& piece, EmptyRow&& empty_row) {
  __shared__ BalancedLds<NTHREADS> sh;
  const BalancedStart st = balanced_start<NTHREADS>(p, sh);
  const int64_t G = p.granule;
  const int64_t nwg = gridDim.x;
  const int64_t w = blockIdx.x;
  const bool last_wg = w == nwg - 1;
  const bool cached = p.B <= NTHREADS;
  int64_t x = st.x;
  for (int b = st.b; b < p.B; ++b) {
    if (x >= st.ge && !(last_wg && x == st.total)) break;
    const int len = cached ? sh.len[b] : clamp_len(p, b);
    const int64_t plen = (len + G - 1) / G;
    if (plen == 0) {
      empty_row(b);
      continue;
    }
    const int64_t slen = plen + p.piece_cost;           // the segment's place on the line
    const int h0 = x >= st.gs ? 0 : (int)((st.gs - x) / slen);
    for (int h = h0; h < p.Hkv; ++h) {
      const int64_t ss = x + h * slen;
      const int64_t se = ss + plen;                      // end of its token granules
      if (ss >= st.ge) break;
      if (se <= st.gs) continue;                         // only its cost granules fall in this range
      const int64_t ps = ss > st.gs ? ss : st.gs;
      const int64_t pe = se < st.ge ? se : st.ge;
      const int64_t first = granule_owner(ss, st.total, nwg, p.range_odd);
      const int slot = (int)(w - first);
      const int count = (int)(granule_owner(se - 1, st.total, nwg, p.range_odd) - first + 1);
      const int64_t t1 = (pe - ss) * G;
      piece(b, h, (int)((ps - ss) * G), (int)(t1 < len ? t1 : len), slot, count, se <= st.ge, len);
    }
    x += p.Hkv * slen;
  }
}

}  // namespace fd
