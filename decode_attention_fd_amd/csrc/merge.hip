// Merge kernel: combines the S split states of each (sequence, query head)
// exactly by rescaling them to their common maximum ("Flash-Decoding:
// Split-KV Attention for Long-Context Decode", kanthi.in, §2 stable form and
// §4 kernel 2; xuujii KB "Decode 专项 Attention" §04):
//   UML : M = max_s m_s, w_s = e^{m_s - M}, O = sum w_s u_s / sum w_s l_s,
//         LSE = M + ln(sum w_s l_s)
//   OLSE: M = max_s lse_s, w_s = e^{lse_s - M}, O = sum w_s o_s / sum w_s,
//         LSE = M + ln(sum w_s)
//
// A row of D floats is read by D/4 lanes, 16 bytes each. SG groups of such
// lanes split the S splits among themselves (split s goes to group s % SG),
// so a row uses 32*SG (D = 128) threads and all of a row's loads are
// independent. Each thread folds its splits in one pass, rebasing its running
// sums whenever a larger maximum arrives (the same merge applied one split at
// a time); the SG partial states are then merged the same way through LDS.
// A split whose m (lse) is -inf weighs exactly 0; a row whose splits are all
// empty writes O = 0 and LSE = -inf. The order of every sum is fixed, so the
// result is bitwise reproducible for a fixed plan.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fd_internal.h"

namespace fd {
namespace {

constexpr int NT = 256;   // threads per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(NT) void merge_kernel(MergeParams p, int sg_log2) {
  constexpr int LPR = D / 4;                 // lanes per row (16 bytes each)
  const int SG = 1 << sg_log2;               // split groups per row
  const int tpr = LPR * SG;                  // threads per row
  const int rpw = NT / tpr;                  // rows per workgroup
  const int rl = threadIdx.x / tpr;
  const int t = threadIdx.x - rl * tpr;
  const int grp = t / LPR;
  const int dl = t - grp * LPR;
  const int row = blockIdx.x * rpw + rl;
  const bool active = row < p.BH;
  const int S = p.S;
  const bool uml = p.ws_format == FD_WS_UML;
  const int sstride = uml ? 2 : 1;

  __shared__ f32x4 part[NT];
  __shared__ float part_m[NT];
  __shared__ float part_d[NT];

  float M = -INFINITY, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const float* stats = p.ws_stats + (int64_t)row * S * sstride;
    const float* ws = p.ws_o + (int64_t)row * S * D + dl * 4;
#pragma unroll 4
    for (int s = grp; s < S; s += SG) {
      const float ms = stats[s * sstride];
      const float ls = uml ? stats[s * sstride + 1] : 1.f;
      const f32x4 u = *reinterpret_cast<const f32x4*>(ws + (int64_t)s * D);
      const bool valid = ms != -INFINITY;
      const float mn = valid ? fmaxf(M, ms) : M;
      const float a = M == -INFINITY ? 0.f : expf(M - mn);
      const float w = valid ? expf(ms - mn) : 0.f;
      acc = acc * a + u * w;
      den = den * a + ls * w;
      M = mn;
    }
  }
  part[threadIdx.x] = acc;
  part_m[threadIdx.x] = M;
  part_d[threadIdx.x] = den;
  __syncthreads();

  if (!active || grp != 0) return;
  const int base = rl * tpr + dl;
  float Mr = -INFINITY;
  for (int g = 0; g < SG; ++g) Mr = fmaxf(Mr, part_m[base + g * LPR]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float dr = 0.f;
  if (Mr != -INFINITY) {
    for (int g = 0; g < SG; ++g) {
      const float mg = part_m[base + g * LPR];
      const float a = mg == -INFINITY ? 0.f : expf(mg - Mr);
      o += part[base + g * LPR] * a;
      dr += part_d[base + g * LPR] * a;
    }
  }
  const bool empty = !(dr > 0.f);
  const float inv = empty ? 0.f : 1.f / dr;
  *reinterpret_cast<f32x4*>(p.out + (int64_t)row * D + dl * 4) = o * inv;
  if (p.lse && dl == 0) p.lse[row] = empty ? -INFINITY : Mr + logf(dr);
}

}  // namespace

int launch_merge(const MergeParams& p, int head_dim, void* stream) {
  const int lpr = head_dim / 4;
  int sg_log2 = 0;
  while ((1 << sg_log2) < p.S && (lpr << (sg_log2 + 1)) <= NT) ++sg_log2;
  const int rows_per_wg = NT / (lpr << sg_log2);
  dim3 grid((p.BH + rows_per_wg - 1) / rows_per_wg);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(NT), 0, st, p, sg_log2);
  else if (head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(NT), 0, st, p, sg_log2);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace fd
