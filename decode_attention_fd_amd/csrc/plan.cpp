// Host planner: problem validation, kernel choice and the split-count rule.
// Pure C++ (no HIP calls), so it runs and is tested without a GPU.
//
// The split-count rule is the wave-efficiency rule of "Flash-Decoding:
// Split-KV Attention for Long-Context Decode" (kanthi.in) §6: S = 1 when the
// work units already fill 80 % of the slots; otherwise, among split counts
// that change the number of blocks per split, the smallest whose last-wave
// efficiency reaches a threshold of the best (85 % on the page).
//
// The MI355X variant is the same rule re-derived for a bandwidth-bound
// kernel on 256 CUs: one split workgroup per CU (4 waves, two 32-token tiles
// in flight each) already pulls that CU's share of HBM bandwidth, so a wave
// of work is CUs x 1 workgroups, and any idle CU in the last wave costs
// bandwidth directly, so the threshold is the best efficiency itself. Blocks
// are one workgroup iteration (4 waves x 32 tokens); chunks are cdiv(len, S),
// aligned to pages and tiles on paged caches only. Split counts whose fp32 workspace traffic (written
// by the split kernel and read back by the merge) exceeds a budget of the KV
// bytes are dropped -- the overhead check at the end of §6, generalised to g
// query heads per KV head.
#include <math.h>
#include <string.h>

#include "fd_internal.h"

namespace fd {

namespace {

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

double wave_eff(int64_t work, int s, int64_t slots) {
  double w = (double)work * (double)s / (double)slots;
  return w / ceil(w);
}

double ws_ratio(int s, int g, int d, int elt, int64_t max_len) {
  if (max_len <= 0) return INFINITY;
  return (2.0 * s * g * (d + 2) * 4.0) / (2.0 * (double)max_len * d * elt);
}

// The split-count rule of kanthi.in §6, organised by blocks per split. A split
// count s matters only through q = cdiv(n_blocks, s), the blocks each split
// streams, so the candidates are the fewest splits that give each distinct q:
// s = 1, then s' = cdiv(n_blocks, q - 1) after a count with q blocks, up to
// cap = min(max_splits, slots, n_blocks). The answer is S = 1 when the work
// units alone fill 80 % of the slots; otherwise the smallest candidate whose
// last-wave efficiency reaches `threshold` times the best candidate's. With
// budget >= 0, candidates above 1 whose workspace traffic exceeds the budget
// are left out (the overhead check at the end of §6).
int split_rule(int64_t work, int64_t slots, int64_t n_blocks, int max_splits, int g, int d, int elt,
               int64_t max_len, double budget, double threshold) {
  if ((double)work >= 0.8 * (double)slots) return 1;
  int64_t cap = max_splits;
  if (slots < cap) cap = slots;
  if (n_blocks < cap) cap = n_blocks;
  if (cap <= 1) return 1;
  // Visit the candidates in increasing order; f(s, eff) returns true to stop.
  auto visit = [&](auto&& f) {
    for (int64_t s = 1; s <= cap;) {
      if ((s == 1 || budget < 0.0 || ws_ratio((int)s, g, d, elt, max_len) <= budget) &&
          f((int)s, wave_eff(work, (int)s, slots)))
        return (int)s;
      const int64_t q = cdiv64(n_blocks, s);
      if (q <= 1) break;
      s = cdiv64(n_blocks, q - 1);
    }
    return 1;
  };
  double best = 0.0;
  visit([&](int, double e) {
    best = e > best ? e : best;
    return false;
  });
  return visit([&](int, double e) { return e >= threshold * best; });
}

}  // namespace

int validate_problem(const fd_problem* p) {
  if (!p) return FD_ERR_INVALID_ARG;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1) return FD_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads) return FD_ERR_INVALID_ARG;
  if (p->batch > 65535 || p->num_kv_heads > 65535) return FD_ERR_UNSUPPORTED;
  if (dtype_size(p->q_dtype) == 0 || dtype_size(p->kv_dtype) == 0) return FD_ERR_INVALID_ARG;
  if (p->layout != FD_LAYOUT_CONTIGUOUS && p->layout != FD_LAYOUT_PAGED) return FD_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return FD_ERR_UNSUPPORTED;
  if (p->q_dtype != p->kv_dtype) return FD_ERR_UNSUPPORTED;
  if (p->max_seq_len < 0) return FD_ERR_INVALID_ARG;
  if (p->q_len < 0 || p->q_len > 8) return FD_ERR_UNSUPPORTED;
  // Output rows B * q_len * Hq index 32-bit merge grids.
  if ((int64_t)p->batch * (p->q_len > 1 ? p->q_len : 1) * p->num_q_heads > FD_MAX_ROWS) return FD_ERR_UNSUPPORTED;
  if (!(isfinite(p->scale))) return FD_ERR_INVALID_ARG;
  const int64_t elt = dtype_size(p->kv_dtype);
  const int64_t D = p->head_dim;
  // Strides beyond FD_MAX_STRIDE elements address more memory than any device
  // holds; bounding them first keeps the byte products below from overflowing.
  // Only the strides this problem uses are looked at.
  const bool paged = p->layout == FD_LAYOUT_PAGED;
  const int64_t strides[] = {p->q_stride_b,
                             p->q_stride_h,
                             p->q_len > 1 ? p->q_stride_q : 0,
                             paged ? p->bt_stride_b : p->kv_stride_b,
                             paged ? p->pool_stride_page : p->kv_stride_h,
                             paged ? p->pool_stride_t : p->kv_stride_t,
                             paged ? p->pool_stride_h : 0};
  for (int64_t v : strides)
    if (v > FD_MAX_STRIDE) return FD_ERR_INVALID_ARG;
  if (p->q_stride_h < D || p->q_stride_b < 0) return FD_ERR_INVALID_ARG;
  if ((p->q_stride_h * elt) % 16 || (p->q_stride_b * elt) % 16) return FD_ERR_ALIGNMENT;
  if (p->q_len > 1) {
    if (p->q_stride_q < 0) return FD_ERR_INVALID_ARG;
    if ((p->q_stride_q * elt) % 16) return FD_ERR_ALIGNMENT;
  }
  if (p->layout == FD_LAYOUT_CONTIGUOUS) {
    if (p->kv_stride_t < D || p->kv_stride_h < 0 || p->kv_stride_b < 0) return FD_ERR_INVALID_ARG;
    if (p->kv_capacity < p->max_seq_len || p->kv_capacity < 0) return FD_ERR_INVALID_ARG;
    if ((p->kv_stride_t * elt) % 16 || (p->kv_stride_h * elt) % 16 || (p->kv_stride_b * elt) % 16)
      return FD_ERR_ALIGNMENT;
  } else {
    if (!is_pow2(p->page_size) || p->page_size < 16 || p->page_size > (1 << 20)) return FD_ERR_UNSUPPORTED;
    if (p->num_pages < 1 || p->max_pages_per_seq < 1 || p->bt_stride_b < 0) return FD_ERR_INVALID_ARG;
    if ((int64_t)p->max_pages_per_seq * p->page_size < p->max_seq_len) return FD_ERR_INVALID_ARG;
    if ((int64_t)p->max_pages_per_seq * p->page_size > (int64_t)0x7fffffff) return FD_ERR_UNSUPPORTED;
    if (p->pool_stride_t < D || p->pool_stride_page < 0 || p->pool_stride_h < 0) return FD_ERR_INVALID_ARG;
    if ((p->pool_stride_t * elt) % 16 || (p->pool_stride_page * elt) % 16 || (p->pool_stride_h * elt) % 16)
      return FD_ERR_ALIGNMENT;
  }
  return FD_OK;
}

int valu_group_template(int g) {
  if (g <= 1) return 1;
  if (g <= 2) return 2;
  if (g <= 4) return 4;
  return 0;
}

int choose_kernel(const fd_problem* p, int requested) {
  // g = query rows one KV head serves: the group's heads times the block's queries.
  const int g = p->num_q_heads / p->num_kv_heads * (p->q_len > 1 ? p->q_len : 1);
  const bool half = dtype_size(p->kv_dtype) == 2;
  const bool mfma_ok = half && g <= 16;          // one or two 8-row column tiles
  const bool valu_ok = valu_group_template(g) != 0;
  switch (requested) {
    case FD_KERNEL_AUTO:
      if (mfma_ok && g >= 2) return FD_KERNEL_MFMA;   // packed GQA: a dense enough contraction
      if (valu_ok) return FD_KERNEL_VALU;
      if (mfma_ok) return FD_KERNEL_MFMA;
      return -FD_ERR_UNSUPPORTED;
    case FD_KERNEL_MFMA:
      return mfma_ok ? FD_KERNEL_MFMA : -FD_ERR_UNSUPPORTED;
    case FD_KERNEL_VALU:
      return valu_ok ? FD_KERNEL_VALU : -FD_ERR_UNSUPPORTED;
    default:
      return -FD_ERR_INVALID_ARG;
  }
}

uint64_t plan_checksum(const fd_plan_t* plan) {
  // FNV-1a over every byte before the checksum field.
  const unsigned char* b = (const unsigned char*)plan;
  const size_t n = offsetof(fd_plan_t, checksum);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

int plan_core(const fd_problem* prob, const fd_plan_opts* o, int balanced_wgs_per_cu, fd_plan_t* out) {
  if (!prob || !o || !out) return FD_ERR_INVALID_ARG;
  int st = validate_problem(prob);
  if (st != FD_OK) return st;
  if (o->num_cus < 1 || o->wgs_per_cu < 1) return FD_ERR_INVALID_ARG;
  if (o->force_splits < 0 || o->force_chunk_tokens < 0 || o->max_splits < 0) return FD_ERR_INVALID_ARG;
  if (o->ws_format != FD_WS_UML && o->ws_format != FD_WS_OLSE) return FD_ERR_INVALID_ARG;
  if (o->heuristic != FD_HEURISTIC_MI355X && o->heuristic != FD_HEURISTIC_FA2) return FD_ERR_INVALID_ARG;
  if (!(o->overhead_budget >= 0.0f)) return FD_ERR_INVALID_ARG;
  if (o->piece_cost_tokens < -1 || o->piece_cost_tokens > (1 << 20)) return FD_ERR_INVALID_ARG;
  if (o->odd_xcd_permille < -1 || o->odd_xcd_permille >= 1000) return FD_ERR_INVALID_ARG;
  if (o->num_host_seq_lens < 0 || (o->num_host_seq_lens > 0 && !o->host_seq_lens)) return FD_ERR_INVALID_ARG;
  if (o->num_host_seq_lens > 0 && o->num_host_seq_lens != prob->batch) return FD_ERR_INVALID_ARG;
  if (o->schedule < FD_SCHEDULE_AUTO || o->schedule > FD_SCHEDULE_BALANCED) return FD_ERR_INVALID_ARG;
  if (o->schedule == FD_SCHEDULE_BALANCED &&
      (o->num_host_seq_lens == 0 || o->force_splits > 0 || o->force_chunk_tokens > 0))
    return FD_ERR_INVALID_ARG;
  for (int i = 0; i < o->num_host_seq_lens; ++i)
    if (o->host_seq_lens[i] > prob->max_seq_len) return FD_ERR_INVALID_ARG;

  const int kernel = choose_kernel(prob, o->kernel);
  if (kernel < 0) return -kernel;

  memset(out, 0, sizeof(*out));
  const int g = prob->num_q_heads / prob->num_kv_heads;
  const int qn = prob->q_len > 1 ? prob->q_len : 1;     // query rows per sequence
  const int R = g * qn;                                 // state rows per (sequence, KV head)
  const int elt = dtype_size(prob->kv_dtype);
  const int D = prob->head_dim;
  const int64_t max_len = prob->max_seq_len;
  const int tile = split_tile_tokens(kernel, D, prob->kv_dtype);
  const int waves = split_waves_per_wg(kernel);
  const bool paged = prob->layout == FD_LAYOUT_PAGED;
  // Paged addressing needs every wave tile inside one page run and tiles
  // starting on page boundaries: chunks are multiples of max(page, tile).
  const int64_t paged_align = paged ? (prob->page_size > tile ? prob->page_size : tile) : 1;

  int64_t S = 1, chunk = 1;
  int64_t odd_chunk = -1;               // uniform plans: odd-numbered splits' tokens (-1: chunk)
  int64_t slots = 0;
  int64_t nwg = 0;                      // balanced grid (0: uniform)
  int64_t piece_cost = 0;               // balanced: cost granules per non-empty segment
  int64_t odd_range = 0;                // balanced: alternating range sizes, per mille
  // AUTO takes the balanced schedule where it pays: ragged lengths (equal
  // lengths are already balanced by the uniform chunks) whose mean is at
  // least FD_BALANCED_MIN_MEAN_TOKENS. A balanced workgroup runs its pieces
  // one after another, each with its own start-up and epilogue, while a
  // uniform grid of many short workgroups has those overlapped by the
  // hardware dispatcher: on ragged batches (lengths U[1, hi], one workgroup
  // per CU) balanced was 3-35 % faster at mean lengths of 1000-2700 tokens,
  // level at ~700 and 2-30 % slower at 250-500.
  bool ragged = false;
  int64_t len_sum = 0;
  for (int b = 0; b < o->num_host_seq_lens; ++b) {
    ragged |= o->host_seq_lens[b] != o->host_seq_lens[0];
    len_sum += o->host_seq_lens[b] > 0 ? o->host_seq_lens[b] : 0;
  }
  const bool long_enough =
      o->num_host_seq_lens > 0 && len_sum >= (int64_t)FD_BALANCED_MIN_MEAN_TOKENS * o->num_host_seq_lens;
  // ... and enough work for every range: with a few hundred tokens per range
  // the pieces' start-up costs dominate, and the uniform length-aware plan was
  // 6-28 % faster (4-16 sequences of up to 2k-8k tokens, 210-400 tokens of
  // K/V rows per range), while from about 870 tokens per range up balanced
  // won by 3-19 %.
  const int64_t range_slots = (int64_t)o->num_cus * (balanced_wgs_per_cu > 0 ? balanced_wgs_per_cu : o->wgs_per_cu);
  const bool enough_work = (int64_t)prob->num_kv_heads * len_sum >= (int64_t)FD_BALANCED_MIN_RANGE_TOKENS * range_slots;
  const bool balanced =
      o->schedule == FD_SCHEDULE_BALANCED ||
      (o->schedule == FD_SCHEDULE_AUTO && o->num_host_seq_lens > 0 && o->force_splits <= 0 &&
       o->force_chunk_tokens <= 0 && o->heuristic == FD_HEURISTIC_MI355X && ragged && long_enough && enough_work);
  if (balanced) {
    {
      // The line of granules (see fd_schedule): N workgroups, range w =
      // [floor(w T / N), floor((w + 1) T / N)); S = the most ranges that any
      // one segment meets.
      // One range per CU by default (the caller's wgs_per_cu otherwise): on
      // ragged batches it was as fast or faster than two (64-sequence edge
      // batch 54 vs 59 us, 48 sequences of up to 4096 tokens 75 vs 79 us).
      slots = (int64_t)o->num_cus * (balanced_wgs_per_cu > 0 ? balanced_wgs_per_cu : o->wgs_per_cu);
      const int64_t G = tile > paged_align ? tile : paged_align;
      const int64_t H = prob->num_kv_heads;
      // Default start-up cost of a piece: 512 tokens (sweep with one range per
      // CU on sixteen ragged batches: the best of 256, 512 and 1024 tokens, or
      // within 1 % of it, on every batch where AUTO takes this schedule; no
      // cost at all was up to 60 % slower).
      const int64_t cost_tok =
          o->piece_cost_tokens > 0 ? o->piece_cost_tokens : (o->piece_cost_tokens < 0 ? 0 : FD_DEFAULT_PIECE_COST_TOKENS);
      piece_cost = cdiv64(cost_tok, G);
      auto seg_len = [&](int64_t plen) { return plen > 0 ? plen + piece_cost : 0; };
      int64_t T = 0;
      for (int b = 0; b < prob->batch; ++b) {
        const int32_t n = o->host_seq_lens[b] > 0 ? o->host_seq_lens[b] : 0;
        T += H * seg_len(cdiv64(n, G));
      }
      nwg = T > 0 ? cdiv64(T, 4) : 1;
      if (nwg > slots) nwg = slots;
      if (nwg > 0x7fffffff) return FD_ERR_UNSUPPORTED;
      // The kernels rebuild the line from the device lengths (clamped to the
      // capacity) and form products of granule positions with the grid size
      // in 64 bits: bound the longest line any device lengths could give.
      const int64_t cap = prob->layout == FD_LAYOUT_PAGED ? (int64_t)prob->max_pages_per_seq * prob->page_size
                                                          : (int64_t)prob->kv_capacity;
      const int64_t t_max = (int64_t)prob->batch * H * (cdiv64(cap, G) + piece_cost);
      if (t_max > ((int64_t)1 << 62) / (nwg + 1)) return FD_ERR_UNSUPPORTED;
      // Ranges of alternating size against the odd XCDs' slower streaming
      // (workgroup w runs on XCD w mod 8; the uniform rule below says more):
      // odd ranges take 1000 - x parts per 1000 of an equal share, even ones
      // 1000 + x. Only where ranges are long enough to be bound by streaming:
      // per-workgroup stamps of the 64-sequence edge batch (about 2100 tokens
      // per range, several pieces each) show no odd-XCD lag, those of the
      // paged ragged batch (about 10 000 per range) a 7 % one. The weighted
      // cut multiplies granule positions by about 1000 N. Every odd range
      // keeps at least one granule ((1000 - x) T >= 1000 N): the piece count
      // of a segment is the difference of its end and start owners, which
      // holds only while no range is empty.
      int64_t xr = 0;
      if (o->heuristic == FD_HEURISTIC_MI355X && o->num_cus == 256 && o->odd_xcd_permille >= 0 && nwg % 8 == 0 &&
          H * len_sum >= (int64_t)FD_XCD_SHIFT_MIN_RANGE_TOKENS * nwg &&
          t_max <= ((int64_t)1 << 62) / (1000 * (nwg + 2))) {
        xr = o->odd_xcd_permille > 0 ? o->odd_xcd_permille : FD_DEFAULT_ODD_XCD_PERMILLE;
        if ((1000 - xr) * T < 1000 * nwg) xr = 0;
      }
      odd_range = xr;
      const int64_t parts_all = (nwg / 2) * 2000 + (nwg % 2 ? 1000 + xr : 0);
      // Owner of granule x: the last range starting at or before it (range w
      // starts at floor(c_w T / c_N), c_w the parts of ranges 0 .. w-1).
      auto owner = [&](int64_t x) {
        if (xr == 0) return ((x + 1) * nwg + T - 1) / T - 1;
        const int64_t c = ((x + 1) * parts_all + T - 1) / T - 1;
        const int64_t w = 2 * (c / 2000) + (c % 2000 >= 1000 + xr ? 1 : 0);
        return w < nwg - 1 ? w : nwg - 1;
      };
      S = 1;
      int64_t x = 0;
      for (int b = 0; b < prob->batch; ++b) {
        const int32_t n = o->host_seq_lens[b] > 0 ? o->host_seq_lens[b] : 0;
        const int64_t plen = cdiv64(n, G);
        for (int64_t h = 0; h < H && plen > 0; ++h) {
          const int64_t ss = x + h * seg_len(plen);
          const int64_t c = owner(ss + plen - 1) - owner(ss) + 1;
          if (c > S) S = c;
        }
        x += H * seg_len(plen);
      }
      chunk = G;
    }
  }
  if (nwg > 0) {
    // planned above
  } else if (o->force_chunk_tokens > 0) {
    chunk = o->force_chunk_tokens;
    if (chunk % paged_align) return FD_ERR_INVALID_ARG;
    S = o->force_splits > 0 ? o->force_splits : (max_len > 0 ? cdiv64(max_len, chunk) : 1);
    if (S * chunk < max_len) return FD_ERR_INVALID_ARG;
  } else if (o->force_splits > 0) {
    S = o->force_splits;
    chunk = cdiv64(max_len > 0 ? max_len : 1, S);
    chunk = cdiv64(chunk, paged_align) * paged_align;
  } else {
    const int max_splits = o->max_splits > 0 ? o->max_splits : 128;
    const int64_t work = (int64_t)prob->batch * prob->num_kv_heads;
    int64_t block, align;
    double budget, threshold;
    if (o->heuristic == FD_HEURISTIC_FA2) {
      slots = 2 * (int64_t)o->num_cus;
      block = 128;
      align = block > paged_align ? block : paged_align;
      budget = -1.0;
      threshold = 0.85;
    } else {
      slots = (int64_t)o->num_cus * o->wgs_per_cu;
      block = (int64_t)tile * waves;
      // Contiguous caches take chunk = cdiv(len, S) exactly: rounding it up to
      // the wave tile made the split kernel 5-10 % slower at 32k-64k tokens
      // (e.g. 64 000 tokens over 32 splits: 2000-token chunks 44-45 us, 2016
      // 47-48 us, 2048 58-62 us), though the last tile of a split is then
      // partial. Paged splits keep page- and tile-aligned boundaries.
      align = paged ? (tile > paged_align ? tile : paged_align) : 1;
      // Default budget 0.25: with 2 % the rule starved short contexts of
      // splits (64/8 GQA at 4k-16k tokens took S = 4-18 where S = 32, one
      // workgroup per CU, made the step 15-24 % faster despite the extra
      // workspace traffic); long contexts are far below either bound.
      budget = o->overhead_budget > 0.0f ? (double)o->overhead_budget : 0.25;
      threshold = 1.0;
    }
    if (o->heuristic == FD_HEURISTIC_MI355X && o->host_seq_lens && o->num_host_seq_lens > 0) {
      // Length-aware: no split longer than one slot's share of the total work.
      int64_t total = 0;
      for (int i = 0; i < o->num_host_seq_lens; ++i) total += o->host_seq_lens[i] > 0 ? o->host_seq_lens[i] : 0;
      total *= prob->num_kv_heads;
      if (max_len <= 0) {
        chunk = align;
      } else {
        chunk = cdiv64(cdiv64(total, slots), align) * align;
        if (chunk < align) chunk = align;
        for (;;) {
          const int64_t s_try = cdiv64(max_len, chunk);
          if (s_try <= (max_splits > 0 ? max_splits : 1) &&
              (s_try == 1 || ws_ratio((int)s_try, R, D, elt, max_len) <= budget))
            break;
          chunk += align;
        }
      }
    } else {
      const int64_t n_blocks = max_len > 0 ? cdiv64(max_len, block) : 0;
      S = split_rule(work, slots, n_blocks, max_splits, R, D, elt, max_len, budget, threshold);
      chunk = cdiv64(cdiv64(max_len > 0 ? max_len : 1, S), align) * align;
    }
    S = max_len > 0 ? cdiv64(max_len, chunk) : 1;          // drop splits empty for every row
    // The hardware deals workgroups to the 8 XCDs of a 256-CU MI355X in turn,
    // so with an even split count split s runs on an XCD of its own parity,
    // and per-workgroup stamps show the odd XCDs streaming 7-10 % slower than
    // the even ones, launch after launch (while which half of the chip is
    // slowest changes from one launch to the next). Odd-numbered splits give
    // odd_xcd_permille of their tokens to the even-numbered ones; the splits
    // still cover S * chunk tokens. Only splits long enough to be bound by
    // streaming: at 64/8 GQA the split kernel gained 0.3-1.1 us at 2000-token
    // splits (64k tokens), 1.5-2.6 us at 4000-8192, and lost 0.5 us at 1000 and
    // 1.0-1.4 us at 500 (32k, 16k tokens).
    if (o->heuristic == FD_HEURISTIC_MI355X && !paged && S % 2 == 0 && o->num_cus == 256 &&
        o->odd_xcd_permille >= 0 && chunk >= FD_XCD_SHIFT_MIN_SPLIT_TOKENS) {
      const int64_t x = o->odd_xcd_permille > 0 ? o->odd_xcd_permille : FD_DEFAULT_ODD_XCD_PERMILLE;
      const int64_t shift = chunk * x / 1000;
      if (shift > 0 && shift < chunk) {
        odd_chunk = chunk - shift;
        chunk += shift;
      }
    }
  }
  if (odd_chunk < 0) odd_chunk = chunk;
  if (S < 1 || S > 65535 || chunk < 1 || chunk > 0x7fffffff) return FD_ERR_UNSUPPORTED;
  // Uniform splits start at s * chunk, a 32-bit token index in the kernels:
  // every split boundary must fit (forced counts and chunks can ask for more).
  if (nwg == 0 && S * chunk > (int64_t)0x7fffffff) return FD_ERR_UNSUPPORTED;
  if (slots == 0) slots = (int64_t)o->num_cus * o->wgs_per_cu;

  out->magic = FD_PLAN_MAGIC;
  out->num_splits = (int32_t)S;
  out->chunk_tokens = (int32_t)chunk;
  out->odd_chunk_tokens = (int32_t)odd_chunk;
  out->kernel = kernel;
  out->ws_format = o->ws_format;
  out->group = g;
  out->tile_tokens = tile;
  out->waves_per_wg = waves;
  out->slots = (int32_t)slots;
  out->schedule = nwg > 0 ? FD_SCHEDULE_BALANCED : FD_SCHEDULE_UNIFORM;
  out->piece_cost = (int32_t)piece_cost;
  out->odd_range_permille = (int32_t)odd_range;
  out->grid_x = nwg > 0 ? (int32_t)nwg : (int32_t)S;
  out->grid_y = nwg > 0 ? 1 : prob->num_kv_heads;
  out->grid_z = nwg > 0 ? 1 : prob->batch;
  out->scale = prob->scale != 0.0f ? prob->scale : (float)(1.0 / sqrt((double)D));
  const int64_t heads = (int64_t)prob->batch * qn * prob->num_q_heads;
  out->ws_o_bytes = heads * S * D * 4;
  out->ws_stats_bytes = heads * S * (o->ws_format == FD_WS_UML ? 2 : 1) * 4;
  out->ws_counter_bytes = (int64_t)prob->batch * prob->num_kv_heads * 4;
  out->prob = *prob;
  out->checksum = plan_checksum(out);
  return FD_OK;
}

}  // namespace fd
