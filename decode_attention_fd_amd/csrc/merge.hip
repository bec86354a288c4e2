// Merge kernel: one wave per (sequence, query head) combines the S split
// states exactly by rescaling them to their common maximum
// ("Flash-Decoding: Split-KV Attention for Long-Context Decode", kanthi.in,
// §2 stable form and §4 kernel 2; xuujii KB "Decode 专项 Attention" §04):
//   UML : M = max_s m_s, w_s = e^{m_s - M}, O = sum w_s u_s / sum w_s l_s,
//         LSE = M + ln(sum w_s l_s)
//   OLSE: M = max_s lse_s, w_s = e^{lse_s - M}, O = sum w_s o_s / sum w_s,
//         LSE = M + ln(sum w_s)
// A split whose m (lse) is -inf is skipped (weight exactly 0); a row whose
// splits are all empty writes O = 0 and LSE = -inf. Splits are accumulated in
// index order, so the result is bitwise reproducible for a fixed plan.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fd_internal.h"

namespace fd {
namespace {

constexpr int WPB = 4;   // waves (rows) per workgroup

template <int D>
__global__ __launch_bounds__(WPB * 64) void merge_kernel(MergeParams p) {
  constexpr int PER = D / 64;            // output floats per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * WPB + (threadIdx.x >> 6);
  if (row >= p.BH) return;               // whole wave exits; no barrier below
  const int S = p.S;
  const bool uml = p.ws_format == FD_WS_UML;
  const int sstride = uml ? 2 : 1;
  const float* stats = p.ws_stats + (int64_t)row * S * sstride;
  const float* ws = p.ws_o + (int64_t)row * S * D;

  // common maximum over the splits, lanes striding over s
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, stats[s * sstride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float den = 0.f;
  if (M != -INFINITY) {
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      float w[4], x[4][PER];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float mj = stats[(s + j) * sstride];
        w[j] = mj == -INFINITY ? 0.f : expf(mj - M);
#pragma unroll
        for (int i = 0; i < PER; ++i) x[j][i] = ws[(int64_t)(s + j) * D + lane * PER + i];
        den += uml ? w[j] * stats[(s + j) * sstride + 1] : w[j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(w[j], x[j][i], acc[i]);
    }
    for (; s < S; ++s) {
      const float mj = stats[s * sstride];
      const float w = mj == -INFINITY ? 0.f : expf(mj - M);
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, ws[(int64_t)s * D + lane * PER + i], acc[i]);
      den += uml ? w * stats[s * sstride + 1] : w;
    }
  }
  const bool empty = !(den > 0.f);
  const float inv = empty ? 0.f : 1.f / den;
#pragma unroll
  for (int i = 0; i < PER; ++i) p.out[(int64_t)row * D + lane * PER + i] = empty ? 0.f : acc[i] * inv;
  if (p.lse && lane == 0) p.lse[row] = empty ? -INFINITY : M + logf(den);
}

}  // namespace

int launch_merge(const MergeParams& p, int head_dim, void* stream) {
  dim3 grid((p.BH + WPB - 1) / WPB);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(WPB * 64), 0, st, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(WPB * 64), 0, st, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace fd
