/*
 * fd.h -- C ABI of the split-KV (Flash-Decoding) decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes. For every sequence b and query head hq, one decode query
 * row q[b, hq, :] attends over the first seq_lens[b] cached keys/values of KV
 * head hkv = hq / g (g = Hq / Hkv):
 *     s_i = scale * q . k_i,   O = sum_i softmax(s)_i v_i,   LSE = ln sum_i e^{s_i}
 * ("Flash-Decoding: Split-KV Attention for Long-Context Decode", kanthi.in,
 * §1 equation and §2 definition of the attention state). The KV sequence is cut
 * into num_splits splits; fd_decode_split computes one attention state per
 * split (§4 kernel 1; per-split (m, l, u) of the xuujii KB page "Decode 专项
 * Attention" §04), and fd_merge combines them exactly by rescaling to the common
 * maximum (kanthi.in §2 stable form; xuujii §04 rebase).
 *
 * Call sequence: fd_plan (host only, once per shape) -> fd_decode_split ->
 * fd_merge, the last two on the caller's stream, back to back.
 *
 * Ownership and threading. The caller owns every buffer (q, K/V or pools,
 * block table, seq_lens, workspace, output, LSE). The library allocates no
 * device memory, keeps no state between calls (apart from a per-process cache
 * of the device's CU count), launches asynchronously on the given stream and
 * never synchronises. All entry points are thread-safe. Device pointers must
 * stay valid until the launched work completes.
 *
 * Errors. Every entry point returns an fd_status. All validation runs on the
 * host before any launch; on an error nothing is launched and no output is
 * written. FD_ERR_HIP reports a failed launch (the HIP status is folded into
 * the message of fd_last_hip_error()). No C++ exception crosses this ABI.
 *
 * Numerics. Accumulation, scores, running max/sum and the workspace are fp32
 * whatever the cache dtype (kanthi.in §4 "FP32 everywhere it matters"); the
 * output is fp32; LSE values are NATURAL logarithms (kanthi.in §8 asks that the
 * base be stated). An empty split stores the neutral state (o = 0 / u = 0,
 * m = LSE = -inf, l = 0) (kanthi.in §4); a row with seq_len 0 gets O = 0 and
 * LSE = -inf. For a fixed plan, results are bitwise reproducible run to run.
 */
#ifndef FD_H_
#define FD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FD_API __attribute__((visibility("default")))

#define FD_VERSION_STRING "0.1.0"
#define FD_PLAN_MAGIC 0x46445031u /* "FDP1" */

typedef enum {
  FD_OK = 0,
  FD_ERR_INVALID_ARG = 1,  /* null pointer, bad size/stride, Hq % Hkv != 0, ... */
  FD_ERR_UNSUPPORTED = 2,  /* head_dim, dtype or layout combination not built */
  FD_ERR_ALIGNMENT = 3,    /* a pointer or row stride is not 16-byte aligned */
  FD_ERR_WORKSPACE = 4,    /* workspace smaller than the plan requires */
  FD_ERR_HIP = 5,          /* a HIP call or kernel launch failed */
  FD_ERR_BAD_PLAN = 6      /* plan not produced by fd_plan, or modified since */
} fd_status;

typedef enum { FD_DTYPE_F32 = 0, FD_DTYPE_F16 = 1, FD_DTYPE_BF16 = 2 } fd_dtype;

typedef enum {
  /* K, V: [B, Hkv, T_cap, D] with element strides (b, h, t) and d contiguous
   * (kanthi.in §4 wrapper and §9 decode contract). */
  FD_LAYOUT_CONTIGUOUS = 0,
  /* K, V pools: [num_pages, page_size, Hkv, D] with element strides
   * (page, token, head) and d contiguous; block_table int32 [B, max_pages],
   * token t of sequence b is row t % page_size of page block_table[b, t /
   * page_size] (kanthi.in §7 paged-KV row and §9; the pool layout itself is
   * this library's choice). */
  FD_LAYOUT_PAGED = 1
} fd_layout;

typedef enum {
  /* Per split: u = sum e^{s-m} v (unnormalised), m = max s, l = sum e^{s-m}
   * (xuujii §04; tinyvolt "Write partial": the split kernel divides nothing). */
  FD_WS_UML = 0,
  /* Per split: o = u / l (normalised) and lse = m + ln l (kanthi.in §4 kernel 1
   * workspace: fp32 partial output plus its LSE). */
  FD_WS_OLSE = 1
} fd_ws_format;

typedef enum {
  FD_KERNEL_AUTO = 0,  /* MFMA for 16-bit KV with 2 <= g * q_len <= 16, VALU otherwise */
  FD_KERNEL_MFMA = 1,  /* packed-GQA tile on MFMA 16x16x32 (16-bit KV, g * q_len <= 16) */
  FD_KERNEL_VALU = 2   /* one query head per lane row, DPP dot products */
} fd_kernel;

typedef enum {
  /* Wave-efficiency rule of kanthi.in §6 re-derived for a bandwidth-bound
   * kernel on MI355X: slots = CUs x wgs_per_cu (1 by default), the smallest
   * split count reaching the best last-wave efficiency, chunk = cdiv(len, S)
   * (paged: rounded up to the page and the 32-token wave tile), and only split
   * counts whose workspace traffic stays within overhead_budget of the KV
   * bytes (§6 overhead check). */
  FD_HEURISTIC_MI355X = 0,
  /* The §6 rule exactly as printed: slots = 2 x CUs, block = 128 tokens, no
   * traffic bound. Kept to reproduce the page's table. */
  FD_HEURISTIC_FA2 = 1
} fd_heuristic;

/* How split work is laid out over workgroups. */
typedef enum {
  /* BALANCED when the planner has host_seq_lens, the lengths differ, their
   * mean is at least FD_BALANCED_MIN_MEAN_TOKENS, the batch holds at least
   * FD_BALANCED_MIN_RANGE_TOKENS tokens of K/V rows (Hkv * sum of lengths) per
   * balanced range, no split count or chunk is forced and the MI355X rule is
   * in use; else UNIFORM. */
  FD_SCHEDULE_AUTO = 0,
  /* One workgroup per (split, KV head, sequence); split s of every segment is
   * [s*chunk, s*chunk + chunk) (kanthi.in §4 kernel 1), or with alternating
   * even and odd lengths (fd_plan_t::chunk_tokens, odd_chunk_tokens). */
  FD_SCHEDULE_UNIFORM = 1,
  /* Needs host_seq_lens. The batch's (sequence, KV head) segments, each cut
   * into granules of G tokens (G = the wave tile, or the page if larger), are
   * laid end to end, each followed by a few granules that stand for the
   * start-up cost of a piece (q load, first tile, epilogue; no tokens), and
   * cut into N near-equal ranges, one per workgroup
   * (N = min(CUs, or CUs x wgs_per_cu (at most the resident 2) when the
   * caller sets it, and cdiv(total granules, 4))). A segment crossing a range
   * boundary yields one state per range: a Stream-K-style partition of the
   * kind kanthi.in §7 lists (LeanAttention) against wave quantization, here
   * so that every workgroup streams the same number of bytes. With
   * fd_plan_t::odd_range_permille = x > 0 the ranges alternate in size:
   * range w takes 1000 + x (w even) or 1000 - x (w odd) parts per 1000 of an
   * equal share, range w starting at granule floor(c_w T / c_N) where c_w is
   * the sum of the parts of ranges 0 .. w-1. */
  FD_SCHEDULE_BALANCED = 2
} fd_schedule;

/* AUTO's thresholds for the balanced schedule: the mean host length, and the
 * K/V rows (KV heads x tokens) per balanced range. */
#define FD_BALANCED_MIN_MEAN_TOKENS 768
#define FD_BALANCED_MIN_RANGE_TOKENS 768

/* Largest accepted stride, in elements, of any fd_problem stride field the
 * problem uses (2^40: more than any device memory holds). A larger one is
 * FD_ERR_INVALID_ARG. */
#define FD_MAX_STRIDE ((int64_t)1 << 40)

/* Largest number of output rows B * q_len * Hq of a problem (and of
 * fd_merge_states): merge grids are indexed in 32 bits. A larger problem is
 * FD_ERR_UNSUPPORTED. */
#define FD_MAX_ROWS ((int64_t)0x7fffffff - 4096)

/* Default shift of tokens from odd-XCD to even-XCD splits, per mille
 * (fd_plan_opts::odd_xcd_permille). */
#define FD_DEFAULT_ODD_XCD_PERMILLE 45

/* Uniform plans shift tokens from odd-numbered splits only when a split
 * holds at least this many tokens: shorter splits are bound by their fixed
 * start-up and epilogue costs, where the shift only lengthens the even ones. */
#define FD_XCD_SHIFT_MIN_SPLIT_TOKENS 1536

/* The balanced schedule shifts work from odd-XCD ranges only when a range
 * averages at least this many tokens of K/V rows (KV heads x tokens / N):
 * shorter ranges are bound by their pieces' start-up latencies, not by the
 * XCD's streaming rate. */
#define FD_XCD_SHIFT_MIN_RANGE_TOKENS 4096

/* Default start-up cost of one balanced piece, in KV tokens. */
#define FD_DEFAULT_PIECE_COST_TOKENS 512

/* Shape and layout of one decode step. All strides are in ELEMENTS. */
typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t num_q_heads;    /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* D in {64, 128} */
  int32_t q_dtype;        /* fd_dtype; must equal kv_dtype */
  int32_t kv_dtype;       /* fd_dtype */
  int32_t layout;         /* fd_layout */
  int32_t max_seq_len;    /* host-side upper bound of seq_lens[]; the plan's splits cover it */
  int64_t q_stride_b;     /* q[b, h, d] at q + b*q_stride_b + h*q_stride_h + d */
  int64_t q_stride_h;
  /* FD_LAYOUT_CONTIGUOUS */
  int64_t kv_stride_b;
  int64_t kv_stride_h;
  int64_t kv_stride_t;
  int32_t kv_capacity;    /* T_cap: tokens allocated per (b, h); seq_lens are clamped to it */
  /* FD_LAYOUT_PAGED */
  int32_t page_size;      /* tokens per page: a power of two >= 16 */
  int32_t num_pages;      /* pages in the pool; block-table entries are clamped to it */
  int32_t max_pages_per_seq;  /* block_table row length used for addressing */
  int64_t bt_stride_b;    /* block_table[b, p] at block_table + b*bt_stride_b + p */
  int64_t pool_stride_page;
  int64_t pool_stride_t;
  int64_t pool_stride_h;
  float scale;            /* score scale; 0 selects 1/sqrt(D) */
  /* Short query blocks (speculative decode; kanthi.in §7 "Short query blocks",
   * §9 item 1: q is [B, q_len, Hq, D]). The block is the last q_len positions
   * of each sequence, whose K/V are already in the cache: query row i sees
   * tokens [0, seq_len - (q_len - 1 - i)) (each query keeps its own
   * visibility, xuujii §06); a row that sees nothing gets O = 0, LSE = -inf.
   * Needs g * q_len <= 16 (MFMA kernel, 16-bit caches; one 8-row column tile
   * up to 8 rows, two beyond) or <= 4 (VALU kernel).
   * out and lse gain the same row axis: [B, q_len, Hq, D] and [B, q_len, Hq];
   * the workspace holds B * q_len * Hq rows. */
  int32_t q_len;          /* query rows per sequence; 0 or 1: a single query */
  int64_t q_stride_q;     /* q[b, i, h, d] at q + b*q_stride_b + i*q_stride_q + h*q_stride_h + d */
} fd_problem;

/* Planner options. Zero-initialise for the defaults. */
typedef struct {
  int32_t num_cus;            /* 0: ask the current device (hipGetDeviceProperties) */
  int32_t wgs_per_cu;         /* split workgroups per CU in one wave of the MI355X rule; 0: 1
                                 (one streaming workgroup per CU saturates its HBM share);
                                 clamped to the kernel's resident workgroups per CU */
  int32_t force_splits;       /* > 0: use this many splits (0 = heuristic, FA2's num_splits=0) */
  int32_t force_chunk_tokens; /* > 0: tokens per split (e.g. 1024); S = cdiv(max_seq_len, chunk) */
  int32_t ws_format;          /* fd_ws_format */
  int32_t kernel;             /* fd_kernel */
  int32_t heuristic;          /* fd_heuristic */
  int32_t max_splits;         /* 0: 128 */
  float overhead_budget;      /* 0: 0.25 (workspace bytes written and read <= 25% of the KV bytes) */
  int32_t num_host_seq_lens;  /* entries in host_seq_lens (0: none; else must equal batch) */
  int32_t schedule;           /* fd_schedule */
  int32_t piece_cost_tokens;  /* balanced schedule: start-up cost of one piece, in KV tokens, added
                                 to every non-empty segment when the line is cut
                                 (0: FD_DEFAULT_PIECE_COST_TOKENS; -1: none) */
  int32_t odd_xcd_permille;   /* MI355X rule, 256 CUs, against the odd XCDs' slower streaming (the
                                 hardware places workgroup w on XCD w mod 8). Uniform plans it makes
                                 (not forced), contiguous cache, even split count, splits of at
                                 least FD_XCD_SHIFT_MIN_SPLIT_TOKENS: odd-numbered splits get
                                 1000 - x tokens per 1000 of an even split's 1000 + x.
                                 Balanced plans with a multiple of 8 ranges averaging at least
                                 FD_XCD_SHIFT_MIN_RANGE_TOKENS, where every odd range keeps at
                                 least one granule: odd ranges get the smaller parts
                                 (fd_plan_t::odd_range_permille). 0: FD_DEFAULT_ODD_XCD_PERMILLE;
                                 -1: equal splits and ranges */
  int32_t reserved[3];
  /* Optional HOST copy of seq_lens (int32 [batch]). With it the MI355X rule
   * sizes splits from the batch's total work: no split longer than one
   * slot's share, cdiv(Hkv * sum(len), slots) tokens, so a ragged batch is
   * not bounded by its longest sequence. The kernels still read the device
   * seq_lens; these must match them. */
  const int32_t* host_seq_lens;
} fd_plan_opts;

/* A plan: caller-owned plain data, produced by fd_plan and read by the other
 * calls. Do not modify; fd_decode_split/fd_merge re-validate it. */
typedef struct {
  uint32_t magic;             /* FD_PLAN_MAGIC */
  int32_t num_splits;         /* S >= 1 */
  int32_t chunk_tokens;       /* UNIFORM: split s covers [start_s, min(start_s + len_s, seq_len)) with
                                 len_s = chunk_tokens for even s, odd_chunk_tokens for odd s, and
                                 start_s = (s / 2) (chunk_tokens + odd_chunk_tokens) + (s odd ?
                                 chunk_tokens : 0): with equal lengths, [s*chunk, s*chunk + chunk) */
  int32_t kernel;             /* fd_kernel actually used (never AUTO) */
  int32_t ws_format;          /* fd_ws_format */
  int32_t group;              /* g = Hq / Hkv */
  int32_t tile_tokens;        /* KV tokens one wave consumes per loop iteration */
  int32_t waves_per_wg;       /* waves per split workgroup */
  int32_t slots;              /* workgroup slots of one wave in the split rule */
  int32_t grid_x, grid_y, grid_z;   /* split kernel grid: (S, Hkv, B) */
  float scale;                /* resolved score scale */
  int32_t schedule;           /* fd_schedule actually used (UNIFORM or BALANCED). BALANCED:
                                 chunk_tokens is the granule G, grid (N, 1, 1), and S is the
                                 largest number of pieces any (b, kv head) segment is cut into */
  int32_t piece_cost;         /* BALANCED: granules of start-up cost added per non-empty segment */
  int32_t odd_chunk_tokens;   /* UNIFORM: tokens of an odd-numbered split; chunk_tokens is an
                                 even-numbered split's (equal unless odd_xcd_permille shifted them) */
  int32_t odd_range_permille; /* BALANCED: x in 0..999, the alternating range sizes (fd_schedule);
                                 0: N equal ranges. UNIFORM: 0 */
  int32_t reserved3;
  int64_t ws_o_bytes;         /* float [B, Hq, S, D] */
  int64_t ws_stats_bytes;     /* float [B, Hq, S, 2] (UML: m, l) or [B, Hq, S] (OLSE: lse) */
  int64_t ws_counter_bytes;   /* uint32 [B, Hkv] arrival counters of fd_decode_fused */
  fd_problem prob;            /* copy of the problem */
  uint64_t checksum;          /* over the fields above */
} fd_plan_t;

/* Device pointers of one decode step. */
typedef struct {
  const void* q;              /* [B, Hq, D] (strided as in the problem) */
  const void* k;              /* contiguous K or the K pool */
  const void* v;              /* contiguous V or the V pool (same strides as K) */
  const int32_t* seq_lens;    /* [B] int32; values are clamped to [0, capacity] */
  const int32_t* block_table; /* paged only, else NULL */
} fd_args;

/* Choose the split count, chunk, kernel and workspace sizes for a problem
 * (kanthi.in §6; xuujii §07 "choose a split plan for the current batch/head/
 * length"). Host only; touches the device only when opts->num_cus == 0.
 * opts may be NULL (all defaults). A uniform plan whose split boundaries
 * would pass 2^31 - 1 tokens (num_splits * chunk_tokens > INT32_MAX, e.g. a
 * forced split count times a forced chunk) is FD_ERR_UNSUPPORTED. */
FD_API int fd_plan(const fd_problem* prob, const fd_plan_opts* opts, fd_plan_t* out);

/* Split kernel: for every (b, kv head, split) one workgroup streams the split's
 * K/V tokens, runs the fp32 online softmax for the g query heads of the group
 * and writes their states to the workspace (kanthi.in §4 kernel 1; tinyvolt
 * "fd_split"). ws_o: float [B, Hq, S, D]; ws_stats: see fd_plan_t. The
 * workspace is fully overwritten (empty splits write the neutral state). */
FD_API int fd_decode_split(const fd_plan_t* plan, const fd_args* args,
                           float* ws_o, size_t ws_o_bytes,
                           float* ws_stats, size_t ws_stats_bytes, void* stream);

/* Merge kernel: per (b, hq), O = sum_s w_s u_s / sum_s w_s l_s with
 * w_s = e^{m_s - max_s m_s} (UML) or O = sum_s w_s o_s / sum_s w_s with
 * w_s = e^{lse_s - max lse} (OLSE); LSE = max + ln(sum) (kanthi.in §2 stable
 * form, §4 kernel 2; xuujii §04). Splits with m = -inf weigh 0.
 * ws_o / ws_stats: the workspace fd_decode_split wrote, of ws_o_bytes /
 * ws_stats_bytes bytes; either smaller than the plan's ws_o_bytes /
 * ws_stats_bytes is FD_ERR_WORKSPACE (nothing is launched).
 * out: float [B, Hq, D] contiguous; lse: float [B, Hq] or NULL. */
FD_API int fd_merge(const fd_plan_t* plan, const float* ws_o, size_t ws_o_bytes, const float* ws_stats,
                    size_t ws_stats_bytes, float* out, float* lse, void* stream);

/* Split kernel with the merge fused in: as fd_decode_split, and in addition the
 * workgroup that finishes last for each (sequence, KV head) merges that
 * group's split states and writes out/lse as fd_merge would. A group that is
 * one split only (S = 1, or one piece under the balanced schedule) writes its
 * rows straight to out/lse and touches neither workspace nor counter. (kanthi.in
 * §9 allows a fused combine in place of the separate one as long as it is
 * documented; the chapter's exercises describe the last-CTA merge with an
 * atomic counter.) One launch instead of two. counters: uint32 [B * Hkv] (plan->ws_counter_bytes), all
 * zero before the first call (allocate it zeroed); every call leaves them
 * zero again. Calls that share counters or workspace must not overlap in
 * time (issue them on one stream). out: float [B, Hq, D]; lse: float [B, Hq]
 * or NULL. */
FD_API int fd_decode_fused(const fd_plan_t* plan, const fd_args* args, float* ws_o, size_t ws_o_bytes,
                           float* ws_stats, size_t ws_stats_bytes, uint32_t* counters, size_t counters_bytes,
                           float* out, float* lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as fd_decode_fused, with the workspace and the arrival counters in a
 * static device array of FD_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends, so the caller passes only the
 * inputs and outputs. Each call first clears the counters with a small fill
 * kernel, then launches the fused kernel, both on `stream`. Needs
 * align256(ws_counter_bytes) + align256(ws_o_bytes) + ws_stats_bytes of the
 * plan to be at most FD_NOALLOC_SCRATCH_BYTES, else FD_ERR_WORKSPACE (nothing
 * is launched). Every call on one GPU shares that GPU's array and leaves its
 * last contents there: calls that overlap in time on one GPU race, so issue
 * them on one stream. Allocates nothing (no hipMalloc, no allocating library
 * call); the first call on a device looks up that device's array address. */
#define FD_NOALLOC_SCRATCH_BYTES (32 << 20)
FD_API int fd_decode_fused_noalloc(const fd_plan_t* plan, const fd_args* args, float* out, float* lse, void* stream);

/* Merge externally produced attention states, one output per row: the ⊕
 * operator of kanthi.in §2 (stable form) exposed on its own, for cascade
 * attention over shared prefixes and for states gathered from other devices
 * (kanthi.in §2 and §7 apply the same merge across devices, and name
 * FlashInfer's merge_state / merge_states as this operation).
 *   ws_format FD_WS_OLSE: states[r, s, :] is a normalised output o_s and
 *     stats[r, s] its natural-log LSE; O = sum_s w_s o_s / sum_s w_s with
 *     w_s = e^{lse_s - max lse}, LSE = max + ln(sum_s w_s).
 *   ws_format FD_WS_UML: states[r, s, :] is u_s = sum_i e^{x_i - m_s} v_i,
 *     stats[r, s, 0:2] = (m_s, l_s) in natural log; O = sum w_s u_s / sum w_s
 *     l_s with w_s = e^{m_s - max m}, LSE = max + ln(sum w_s l_s).
 * A state with lse (m) = -inf weighs 0; a row whose states are all -inf gets
 * O = 0 and LSE = -inf. Layouts (float32, contiguous, device memory):
 * states [rows, num_states, head_dim], stats [rows, num_states] (OLSE) or
 * [rows, num_states, 2] (UML), out [rows, head_dim], lse_out [rows] or NULL.
 * head_dim in {64, 128}; 1 <= num_states <= 65535; 0 <= rows <= FD_MAX_ROWS
 * (rows = 0 launches nothing). Inputs are read only; the caller owns every
 * buffer. Arguments are checked on the host before any launch. */
FD_API int fd_merge_states(int ws_format, const float* states, const float* stats, int64_t rows,
                           int32_t num_states, int32_t head_dim, float* out, float* lse_out, void* stream);

/* Measurement aid, not part of the attention path: a streaming-read kernel
 * that reads `bytes` (a multiple of 16) of device memory at `buf` with the
 * split kernels' load form (16-byte nontemporal loads, 512 workgroups each on
 * a contiguous share), so a benchmark can report the read rate this device
 * reaches next to its nominal peak (the chapter's benchmark plan, kanthi.in
 * §8, judges kernels by achieved bandwidth against HBM peak). `sink` (device,
 * at least FD_READ_PROBE_SINK_BYTES) receives one digest word per thread and
 * nothing else. Time it with events on `stream`. */
#define FD_READ_PROBE_SINK_BYTES (512 * 256 * 4)
FD_API int fd_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_bytes, void* stream);

/* Measurement aid, not part of the attention path. A build with per-workgroup
 * stamps (decode_attention_fd_amd/build.py --wg-stamps) records, in every
 * split-kernel launch of at most FD_WG_STAMP_RECORDS workgroups, four uint64
 * per workgroup w (linear index over the grid x, y, z): its start and end on
 * the device's 100 MHz constant clock, the K/V tokens it streamed, and its
 * piece count | its XCD id << 32 | its CU's place in the XCD << 40 (bits 8..15
 * of the hardware id register: CU, shader array, shader engine). fd_wg_stamps copies the records of the
 * current device (the last launch's, for the workgroups it had) into device
 * memory dst (dst_bytes, at most FD_WG_STAMP_RECORDS * 32 bytes are copied)
 * on stream. Other builds record nothing and return FD_ERR_UNSUPPORTED. */
#define FD_WG_STAMP_RECORDS 65536
FD_API int fd_wg_stamps(void* dst, size_t dst_bytes, void* stream);

/* Human-readable text for an fd_status. Never NULL. */
FD_API const char* fd_status_str(int status);

/* Text of the last HIP error seen by this thread ("" if none). */
FD_API const char* fd_last_hip_error(void);

/* Library version, FD_VERSION_STRING. */
FD_API const char* fd_version(void);

/* sizeof of the ABI structs, so bindings can check their mirrors:
 * which = 0 fd_problem, 1 fd_plan_opts, 2 fd_plan_t, 3 fd_args; else 0. */
FD_API size_t fd_struct_size(int which);

#ifdef __cplusplus
}
#endif

#endif /* FD_H_ */
