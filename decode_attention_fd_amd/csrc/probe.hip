// Streaming-read probe: the HBM read rate a plain kernel reaches on this
// device with the load form the split kernels use (16-byte nontemporal
// loads, four in flight per lane, every workgroup on its own contiguous
// region). It is a measurement aid that bench.py reports beside the nominal
// peak, not part of the attention path.
#include <hip/hip_runtime.h>

#include "fd_internal.h"

namespace fd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int PT = 256;     // threads per workgroup
constexpr int DEPTH = 4;    // loads in flight per lane

__global__ __launch_bounds__(PT) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)PT * DEPTH) {
    u32x4 r[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t j = i + (int64_t)PT * d;
      r[d] = j < hi ? __builtin_nontemporal_load(buf + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= r[d];
  }
  // one digest word per thread keeps every load live
  sink[(int64_t)blockIdx.x * PT + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

int launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int grid, void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(PT), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // namespace fd
