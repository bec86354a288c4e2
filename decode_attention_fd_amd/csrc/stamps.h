// Per-workgroup stamps of the split kernels, compiled in only by the
// measurement build (FD_WG_STAMPS; build.py --wg-stamps): for each workgroup,
// its start and end on the device's 100 MHz constant clock, the K/V tokens it
// streamed, the pieces it ran, the XCD it ran on and its place inside the
// XCD (shader engine, shader array, CU). Read back with
// fd_wg_stamps. In the release build every hook below is empty.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {

#ifdef FD_WG_STAMPS
struct WgStamp {
  uint64_t t0 = 0;
  int64_t tokens = 0;
  int pieces = 0;
};
__device__ __forceinline__ void stamp_begin(const SplitParams& p, WgStamp& s) {
  if (p.stamps) s.t0 = wall_clock64();
}
__device__ __forceinline__ void stamp_piece(WgStamp& s, int tokens) {
  s.tokens += tokens;
  s.pieces += 1;
}
// Every thread of the workgroup calls it, after all of the workgroup's work.
__device__ __forceinline__ void stamp_end(const SplitParams& p, const WgStamp& s) {
  if (!p.stamps) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t w = blockIdx.x + (uint64_t)gridDim.x * (blockIdx.y + (uint64_t)gridDim.y * blockIdx.z);
    const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 0xfu;   // HW_REG_XCC_ID
    // HW_REG_HW_ID bits 8..15: CU id (4 bits), shader array (1), shader engine (3)
    const unsigned place = __builtin_amdgcn_s_getreg(4 | (8 << 6) | (7 << 11)) & 0xffu;
    uint64_t* rec = p.stamps + 4 * w;
    rec[0] = s.t0;
    rec[1] = wall_clock64();
    rec[2] = (uint64_t)s.tokens;
    rec[3] = (uint64_t)s.pieces | ((uint64_t)xcc << 32) | ((uint64_t)place << 40);
  }
}
#else
struct WgStamp {};
__device__ __forceinline__ void stamp_begin(const SplitParams&, WgStamp&) {}
__device__ __forceinline__ void stamp_piece(WgStamp&, int) {}
__device__ __forceinline__ void stamp_end(const SplitParams&, const WgStamp&) {}
#endif

}  // namespace fd
