// Internal interface between the host API (api.cpp), the planner (plan.cpp)
// and the HIP kernels (split_mfma.hip, split_valu.hip, merge.hip).
#pragma once

#include <stdint.h>

#include "fd.h"

// Race check: a build with FD_DEBUG_BARRIERS defined (build.py
// --debug-barriers) adds synchronisation around every hand-over of LDS, and
// its results must equal the release build's bit for bit. Workgroup barriers
// go only where every thread of the workgroup arrives; inside the per-wave
// streaming loops, whose trip counts differ between waves, the debug build
// waits for all of the wave's memory operations and adds a wave barrier.
#ifdef FD_DEBUG_BARRIERS
#define FD_DEBUG_WG_BARRIER() __syncthreads()
#define FD_DEBUG_WAVE_BARRIER()         \
  do {                                  \
    __builtin_amdgcn_s_waitcnt(0);      \
    __builtin_amdgcn_wave_barrier();    \
  } while (0)
#else
#define FD_DEBUG_WG_BARRIER() \
  do {                        \
  } while (0)
#define FD_DEBUG_WAVE_BARRIER() \
  do {                          \
  } while (0)
#endif

namespace fd {

// Everything one split-kernel launch needs, passed by value. Strides are in
// elements, as in fd_problem.
struct SplitParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* block_table;
  float* ws_o;
  float* ws_stats;
  int64_t q_sb, q_sh;
  int64_t kv_sb, kv_sh, kv_st;          // contiguous
  int64_t pool_sp, pool_st, pool_sh;    // paged
  int64_t bt_sb;
  int32_t B, Hq, Hkv, g;
  int32_t q_len;                        // query rows per sequence (>= 1)
  int64_t q_sq;                         // element stride between a sequence's query rows
  int32_t R;                            // state rows per (sequence, KV head): g * q_len
  int32_t S, chunk;                     // uniform: chunk = tokens of an even-numbered split
  int32_t chunk_odd;                    // uniform: tokens of an odd-numbered split
  int32_t cap_tokens;                   // seq_lens are clamped to [0, cap_tokens]
  int32_t page_log2, num_pages;
  int32_t ws_format;
  float scale_log2;                     // scale * log2(e): scores go straight to base 2
  // balanced schedule (nwg = 0: uniform grid (S, Hkv, B))
  int32_t nwg;                          // workgroups of the balanced grid
  int32_t granule;                      // tokens per granule of the balanced line
  int32_t piece_cost;                   // cost granules after each non-empty segment on the line
  int32_t range_odd;                    // alternating range sizes, parts per mille (0: equal ranges)
  // fused merge (0 = write split states only)
  int32_t fused;
  uint32_t* counters;                   // [B * Hkv], zero on entry, zero on exit
  uint64_t* stamps;                     // per-workgroup stamp records (measurement build), else null
  float* out;                           // [B, Hq, D]
  float* lse;                           // [B, Hq] or null
};

struct MergeParams {
  const float* ws_o;
  const float* ws_stats;
  float* out;
  float* lse;
  int32_t BH, S, ws_format;
};

// Launchers: return the HIP status of the launch (hipSuccess == 0).
int launch_split_mfma(const SplitParams& p, int head_dim, int kv_dtype, int layout, void* stream);
int launch_split_valu(const SplitParams& p, int head_dim, int kv_dtype, int layout, int group_tpl,
                      void* stream);
int launch_merge(const MergeParams& p, int head_dim, void* stream);
int launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int grid, void* stream);

// Per-kernel geometry the planner needs (tokens per wave tile, waves per
// workgroup) and the compiled resident-workgroups-per-CU of each variant.
int split_tile_tokens(int kernel, int head_dim, int kv_dtype);
int split_waves_per_wg(int kernel);
int valu_group_template(int g);                 // 1, 2 or 4; 0 if unsupported
int default_wgs_per_cu(int kernel, int head_dim, int kv_dtype, int group_tpl, int layout);

// The pure host planner (no HIP calls). opts must be fully resolved:
// num_cus > 0 and wgs_per_cu > 0. balanced_wgs_per_cu: workgroups per CU of
// the balanced grid (the caller's wgs_per_cu if it set one, else every
// workgroup the kernel can keep resident).
int plan_core(const fd_problem* prob, const fd_plan_opts* opts, int balanced_wgs_per_cu, fd_plan_t* out);
int validate_problem(const fd_problem* prob);
int choose_kernel(const fd_problem* prob, int requested);
uint64_t plan_checksum(const fd_plan_t* plan);

// fd_decode_fused in two steps (api.cpp): every check and the launch
// parameters, then the launch. The no-allocation entry point (noalloc.hip)
// runs both with its static scratch as workspace and counters.
int fused_params(const fd_plan_t* plan, const fd_args* args, float* ws_o, size_t ws_o_bytes, float* ws_stats,
                 size_t ws_stats_bytes, uint32_t* counters, size_t counters_bytes, float* out, float* lse,
                 SplitParams* p);
int launch_fused(const fd_plan_t* plan, const SplitParams& p, void* stream);
// The stamp records for a launch of `workgroups` workgroups (stamps.hip):
// null unless the library is the per-workgroup stamp build and they fit.
uint64_t* wg_stamp_records_for(int64_t workgroups);
int check_fused_plan(const fd_plan_t* plan);       // FD_OK or the status fd_decode_fused would return
int record_hip_error(int err, const char* where);  // keeps the text for fd_last_hip_error; FD_ERR_HIP

// Element size of an fd_dtype, 0 if invalid.
inline int dtype_size(int dt) {
  return dt == FD_DTYPE_F32 ? 4 : (dt == FD_DTYPE_F16 || dt == FD_DTYPE_BF16) ? 2 : 0;
}

}  // namespace fd
