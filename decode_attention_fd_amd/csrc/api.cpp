// The C ABI: argument validation, device queries for the planner, and the
// launches of the split and merge kernels on the caller's stream.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>

#include "fd_internal.h"
#include "geometry.h"

namespace fd {

int occupancy_split_mfma(int head_dim, int kv_dtype, int layout, int nct, int* out);
int occupancy_split_valu(int head_dim, int kv_dtype, int layout, int group_tpl, int* out);

// `variant`: MFMA column tiles (1 or 2) or the VALU row template (1, 2, 4).
int occupancy_split(int kernel, int head_dim, int kv_dtype, int layout, int variant, int* out) {
  if (kernel == FD_KERNEL_MFMA) return occupancy_split_mfma(head_dim, kv_dtype, layout, variant, out);
  return occupancy_split_valu(head_dim, kv_dtype, layout, variant, out);
}

int split_tile_tokens(int kernel, int head_dim, int kv_dtype) {
  return kernel == FD_KERNEL_MFMA ? kMfmaTileTokens : valu_tile_tokens_for(head_dim, dtype_size(kv_dtype));
}

int split_waves_per_wg(int /*kernel*/) { return kSplitWaves; }

// Resident split workgroups per CU of each compiled variant, generated at build
// time from the compiler's resource usage (VGPRs and LDS per workgroup); used
// when the planner runs without a device. tests/test_gpu_parity.py checks it
// against hipOccupancyMaxActiveBlocksPerMultiprocessor on the device.
namespace {
struct OccRow {
  int kernel, head_dim, kv_dtype, group_tpl, paged, wgs;
};
const OccRow kOccupancy[] = {
#include "fd_occupancy.inc"
};
}  // namespace

int default_wgs_per_cu(int kernel, int head_dim, int kv_dtype, int group_tpl, int layout) {
  const int paged = layout == FD_LAYOUT_PAGED;
  for (const OccRow& r : kOccupancy)
    if (r.kernel == kernel && r.head_dim == head_dim && r.kv_dtype == kv_dtype && r.paged == paged &&
        r.group_tpl == group_tpl)
      return r.wgs;
  return 1;
}

namespace {

thread_local char g_last_hip[256] = "";

int hip_fail(int err, const char* where) {
  snprintf(g_last_hip, sizeof(g_last_hip), "%s: %s (%d)", where,
           hipGetErrorString((hipError_t)err), err);
  return FD_ERR_HIP;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// Per-device cache of the CU count and of each split-kernel variant's
// resident workgroups per CU: the occupancy query costs about a millisecond,
// and a decode loop plans every step.
struct DeviceInfo {
  int num_cus = 0;
  std::map<int, int> resident;       // variant key -> resident workgroups per CU
};
std::mutex g_dev_mutex;
std::map<int, DeviceInfo> g_dev;

int device_query(int dev, int kernel, int head_dim, int kv_dtype, int layout, int gtpl, int* num_cus,
                 int* resident) {
  const int key = (((kernel * 256 + head_dim) * 4 + kv_dtype) * 2 + layout) * 8 + gtpl;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& info = g_dev[dev];
  if (info.num_cus == 0) {
    int n = 0;
    int err = (int)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err) return err;
    info.num_cus = n;
  }
  auto it = info.resident.find(key);
  if (it == info.resident.end()) {
    int r = 0;
    int err = occupancy_split(kernel, head_dim, kv_dtype, layout, gtpl, &r);
    if (err) return err;
    it = info.resident.emplace(key, r).first;
  }
  *num_cus = info.num_cus;
  *resident = it->second;
  return 0;
}

int check_plan(const fd_plan_t* plan) {
  if (!plan) return FD_ERR_INVALID_ARG;
  if (plan->magic != FD_PLAN_MAGIC || plan->checksum != plan_checksum(plan)) return FD_ERR_BAD_PLAN;
  if (validate_problem(&plan->prob) != FD_OK) return FD_ERR_BAD_PLAN;
  if (plan->num_splits < 1 || plan->chunk_tokens < 1 || plan->odd_chunk_tokens < 1) return FD_ERR_BAD_PLAN;
  if (plan->schedule != FD_SCHEDULE_UNIFORM && plan->schedule != FD_SCHEDULE_BALANCED) return FD_ERR_BAD_PLAN;
  if (plan->schedule == FD_SCHEDULE_BALANCED && (plan->grid_x < 1 || plan->piece_cost < 0)) return FD_ERR_BAD_PLAN;
  if (plan->odd_range_permille < 0 || plan->odd_range_permille > 999 ||
      (plan->schedule != FD_SCHEDULE_BALANCED && plan->odd_range_permille != 0))
    return FD_ERR_BAD_PLAN;
  return FD_OK;
}

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

}  // namespace
}  // namespace fd

using namespace fd;

extern "C" {

FD_API const char* fd_version(void) { return FD_VERSION_STRING; }

FD_API const char* fd_status_str(int status) {
  switch (status) {
    case FD_OK: return "ok";
    case FD_ERR_INVALID_ARG: return "invalid argument";
    case FD_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, group size or layout";
    case FD_ERR_ALIGNMENT: return "pointer or row stride not 16-byte aligned";
    case FD_ERR_WORKSPACE: return "workspace smaller than the plan requires";
    case FD_ERR_HIP: return "HIP call or kernel launch failed";
    case FD_ERR_BAD_PLAN: return "plan not produced by fd_plan or modified since";
    default: return "unknown status";
  }
}

FD_API const char* fd_last_hip_error(void) { return g_last_hip; }

FD_API size_t fd_struct_size(int which) {
  switch (which) {
    case 0: return sizeof(fd_problem);
    case 1: return sizeof(fd_plan_opts);
    case 2: return sizeof(fd_plan_t);
    case 3: return sizeof(fd_args);
    default: return 0;
  }
}

FD_API int fd_plan(const fd_problem* prob, const fd_plan_opts* opts, fd_plan_t* out) {
  if (!prob || !out) return FD_ERR_INVALID_ARG;
  fd_plan_opts o;
  memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.num_cus < 0 || o.wgs_per_cu < 0) return FD_ERR_INVALID_ARG;
  int st = validate_problem(prob);
  if (st != FD_OK) return st;
  const int kernel = choose_kernel(prob, o.kernel);
  if (kernel < 0) return -kernel;
  const int rows = prob->num_q_heads / prob->num_kv_heads * (prob->q_len > 1 ? prob->q_len : 1);
  const int gtpl = kernel == FD_KERNEL_MFMA ? (rows > 8 ? 2 : 1) : valu_group_template(rows);
  // Resident split workgroups per CU: the device's answer when we query it,
  // else the table generated from the compiler's resource usage.
  int resident = 0;
  if (o.num_cus == 0) {
    int dev = 0;
    int err = (int)hipGetDevice(&dev);
    if (err) return hip_fail(err, "hipGetDevice");
    err = device_query(dev, kernel, prob->head_dim, prob->kv_dtype, prob->layout, gtpl, &o.num_cus, &resident);
    if (err) return hip_fail(err, "device query (CU count, occupancy)");
  }
  if (resident <= 0) resident = default_wgs_per_cu(kernel, prob->head_dim, prob->kv_dtype, gtpl, prob->layout);
  // Workgroups per CU in one wave of the MI355X split rule: 1 by default (one
  // streaming split workgroup per CU saturates its share of HBM; measured by
  // split-count sweeps), never more than can be resident.
  // The balanced schedule takes one range per CU unless the caller asks for
  // more; its kernels carry the walk's state on top of the split loop's and
  // keep two workgroups per CU resident at most.
  const int balanced_resident = resident < 2 ? resident : 2;
  const int balanced_wgs =
      o.wgs_per_cu > 0 ? (o.wgs_per_cu < balanced_resident ? o.wgs_per_cu : balanced_resident) : 1;
  if (o.wgs_per_cu == 0) o.wgs_per_cu = 1;
  if (o.wgs_per_cu > resident) o.wgs_per_cu = resident;
  o.kernel = kernel;
  return plan_core(prob, &o, balanced_wgs, out);
}

namespace {

// Validation and parameter setup shared by fd_decode_split and fd_decode_fused.
int split_params(const fd_plan_t* plan, const fd_args* args, float* ws_o, size_t ws_o_bytes, float* ws_stats,
                 size_t ws_stats_bytes, SplitParams* out) {
  int st = check_plan(plan);
  if (st != FD_OK) return st;
  if (!args || !args->q || !args->k || !args->v || !args->seq_lens || !ws_o || !ws_stats)
    return FD_ERR_INVALID_ARG;
  const fd_problem& pr = plan->prob;
  const bool paged = pr.layout == FD_LAYOUT_PAGED;
  if (paged && !args->block_table) return FD_ERR_INVALID_ARG;
  if (!aligned(args->q, 16) || !aligned(args->k, 16) || !aligned(args->v, 16) || !aligned(args->seq_lens, 4) ||
      (paged && !aligned(args->block_table, 4)) || !aligned(ws_o, 16) || !aligned(ws_stats, 8))
    return FD_ERR_ALIGNMENT;
  if (ws_o_bytes < (size_t)plan->ws_o_bytes || ws_stats_bytes < (size_t)plan->ws_stats_bytes)
    return FD_ERR_WORKSPACE;

  SplitParams& p = *out;
  memset(&p, 0, sizeof(p));
  p.q = args->q;
  p.k = args->k;
  p.v = args->v;
  p.seq_lens = args->seq_lens;
  p.block_table = paged ? args->block_table : nullptr;
  p.ws_o = ws_o;
  p.ws_stats = ws_stats;
  p.q_sb = pr.q_stride_b;
  p.q_sh = pr.q_stride_h;
  p.kv_sb = pr.kv_stride_b;
  p.kv_sh = pr.kv_stride_h;
  p.kv_st = pr.kv_stride_t;
  p.pool_sp = pr.pool_stride_page;
  p.pool_st = pr.pool_stride_t;
  p.pool_sh = pr.pool_stride_h;
  p.bt_sb = pr.bt_stride_b;
  p.B = pr.batch;
  p.Hq = pr.num_q_heads;
  p.Hkv = pr.num_kv_heads;
  p.g = plan->group;
  p.q_len = pr.q_len > 1 ? pr.q_len : 1;
  p.q_sq = pr.q_stride_q;
  p.R = p.g * p.q_len;
  p.S = plan->num_splits;
  p.chunk = plan->chunk_tokens;
  p.chunk_odd = plan->odd_chunk_tokens;
  if (paged) {
    p.cap_tokens = pr.max_pages_per_seq * pr.page_size;
    p.page_log2 = ilog2(pr.page_size);
    p.num_pages = pr.num_pages;
  } else {
    p.cap_tokens = pr.kv_capacity;
  }
  if (plan->schedule == FD_SCHEDULE_BALANCED) {
    p.nwg = plan->grid_x;
    p.granule = plan->chunk_tokens;
    p.piece_cost = plan->piece_cost;
    p.range_odd = plan->odd_range_permille;
  } else {
    // Tokens past the last split belong to no split: clamp there as well.
    const int64_t covered = (int64_t)(plan->num_splits / 2) * ((int64_t)plan->chunk_tokens + plan->odd_chunk_tokens) +
                            (plan->num_splits % 2 ? plan->chunk_tokens : 0);
    if (covered < p.cap_tokens) p.cap_tokens = (int32_t)covered;
  }
  p.ws_format = plan->ws_format;
  p.scale_log2 = (float)((double)plan->scale * 1.4426950408889634);
  p.stamps = wg_stamp_records_for((int64_t)plan->grid_x * plan->grid_y * plan->grid_z);
  return FD_OK;
}

int launch_split(const fd_plan_t* plan, const SplitParams& p, void* stream) {
  const fd_problem& pr = plan->prob;
  int err;
  if (plan->kernel == FD_KERNEL_MFMA)
    err = launch_split_mfma(p, pr.head_dim, pr.kv_dtype, pr.layout, stream);
  else
    err = launch_split_valu(p, pr.head_dim, pr.kv_dtype, pr.layout, valu_group_template(p.R), stream);
  if (err) return hip_fail(err, "split kernel launch");
  return FD_OK;
}

}  // namespace

FD_API int fd_decode_split(const fd_plan_t* plan, const fd_args* args, float* ws_o, size_t ws_o_bytes,
                           float* ws_stats, size_t ws_stats_bytes, void* stream) {
  SplitParams p;
  int st = split_params(plan, args, ws_o, ws_o_bytes, ws_stats, ws_stats_bytes, &p);
  if (st != FD_OK) return st;
  return launch_split(plan, p, stream);
}

FD_API int fd_decode_fused(const fd_plan_t* plan, const fd_args* args, float* ws_o, size_t ws_o_bytes,
                           float* ws_stats, size_t ws_stats_bytes, uint32_t* counters, size_t counters_bytes,
                           float* out, float* lse, void* stream) {
  SplitParams p;
  int st = fd::fused_params(plan, args, ws_o, ws_o_bytes, ws_stats, ws_stats_bytes, counters, counters_bytes, out,
                            lse, &p);
  if (st != FD_OK) return st;
  return fd::launch_fused(plan, p, stream);
}

}  // extern "C"

// The validation and launch of fd_decode_fused, shared with
// fd_decode_fused_noalloc (noalloc.hip).
int fd::fused_params(const fd_plan_t* plan, const fd_args* args, float* ws_o, size_t ws_o_bytes, float* ws_stats,
                     size_t ws_stats_bytes, uint32_t* counters, size_t counters_bytes, float* out, float* lse,
                     SplitParams* out_params) {
  SplitParams& p = *out_params;
  int st = split_params(plan, args, ws_o, ws_o_bytes, ws_stats, ws_stats_bytes, &p);
  if (st != FD_OK) return st;
  if (!counters || !out) return FD_ERR_INVALID_ARG;
  if (!aligned(counters, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4))) return FD_ERR_ALIGNMENT;
  if (counters_bytes < (size_t)plan->ws_counter_bytes) return FD_ERR_WORKSPACE;
  p.fused = 1;
  p.counters = counters;
  p.out = out;
  p.lse = lse;
  return FD_OK;
}

int fd::launch_fused(const fd_plan_t* plan, const SplitParams& p, void* stream) { return launch_split(plan, p, stream); }

int fd::check_fused_plan(const fd_plan_t* plan) { return check_plan(plan); }

int fd::record_hip_error(int err, const char* where) { return hip_fail(err, where); }

extern "C" {

FD_API int fd_merge(const fd_plan_t* plan, const float* ws_o, size_t ws_o_bytes, const float* ws_stats,
                    size_t ws_stats_bytes, float* out, float* lse, void* stream) {
  int st = check_plan(plan);
  if (st != FD_OK) return st;
  if (!ws_o || !ws_stats || !out) return FD_ERR_INVALID_ARG;
  if (!aligned(ws_o, 16) || !aligned(ws_stats, 8) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
    return FD_ERR_ALIGNMENT;
  if (ws_o_bytes < (size_t)plan->ws_o_bytes || ws_stats_bytes < (size_t)plan->ws_stats_bytes)
    return FD_ERR_WORKSPACE;
  // validate_problem (through check_plan) bounded the rows by FD_MAX_ROWS.
  const int64_t rows = (int64_t)plan->prob.batch * (plan->prob.q_len > 1 ? plan->prob.q_len : 1) *
                       plan->prob.num_q_heads;
  MergeParams p;
  p.ws_o = ws_o;
  p.ws_stats = ws_stats;
  p.out = out;
  p.lse = lse;
  p.BH = (int32_t)rows;
  p.S = plan->num_splits;
  p.ws_format = plan->ws_format;
  int err = launch_merge(p, plan->prob.head_dim, stream);
  if (err) return hip_fail(err, "merge kernel launch");
  return FD_OK;
}

FD_API int fd_merge_states(int ws_format, const float* states, const float* stats, int64_t rows,
                           int32_t num_states, int32_t head_dim, float* out, float* lse_out, void* stream) {
  if (ws_format != FD_WS_UML && ws_format != FD_WS_OLSE) return FD_ERR_INVALID_ARG;
  if (rows < 0 || rows > FD_MAX_ROWS || num_states < 1 || num_states > 65535) return FD_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return FD_ERR_UNSUPPORTED;
  if (rows == 0) return FD_OK;
  if (!states || !stats || !out) return FD_ERR_INVALID_ARG;
  if (!aligned(states, 16) || !aligned(stats, ws_format == FD_WS_UML ? 8 : 4) || !aligned(out, 16) ||
      (lse_out && !aligned(lse_out, 4)))
    return FD_ERR_ALIGNMENT;
  MergeParams p;
  p.ws_o = states;
  p.ws_stats = stats;
  p.out = out;
  p.lse = lse_out;
  p.BH = (int32_t)rows;
  p.S = num_states;
  p.ws_format = ws_format;
  int err = launch_merge(p, head_dim, stream);
  if (err) return hip_fail(err, "merge kernel launch");
  return FD_OK;
}

FD_API int fd_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_bytes, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return FD_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return FD_ERR_ALIGNMENT;
  if (sink_bytes < (size_t)FD_READ_PROBE_SINK_BYTES) return FD_ERR_WORKSPACE;
  int err = launch_read_probe(buf, (int64_t)bytes, sink, FD_READ_PROBE_SINK_BYTES / (256 * 4), stream);
  if (err) return hip_fail(err, "read probe launch");
  return FD_OK;
}

}  // extern "C"
