// Merge kernel: combines the S split states of each (sequence, query head)
// exactly by rescaling them to their common maximum ("Flash-Decoding:
// Split-KV Attention for Long-Context Decode", kanthi.in, §2 stable form and
// §4 kernel 2; xuujii KB "Decode 专项 Attention" §04):
//   UML : M = max_s m_s, w_s = e^{m_s - M}, O = sum w_s u_s / sum w_s l_s,
//         LSE = M + ln(sum w_s l_s)
//   OLSE: M = max_s lse_s, w_s = e^{lse_s - M}, O = sum w_s o_s / sum w_s,
//         LSE = M + ln(sum w_s)
// Each row gets 32*SG threads (D = 128; 16*SG for D = 64) so all of a row's
// loads are independent; see merge_rows.h for the per-lane fold and the
// combination of the SG partial states.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fd_internal.h"
#include "merge_rows.h"

namespace fd {
namespace {

constexpr int NT = 256;   // threads per workgroup

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
  const bool uml = p.ws_format == FD_WS_UML;

  __shared__ mf32x4 part[NT];
  __shared__ float part_m[NT];
  __shared__ float part_d[NT];

  RowState st = {mf32x4{0.f, 0.f, 0.f, 0.f}, -INFINITY, 0.f};
  if (active)
    st = fold_splits<D>(p.ws_o + (int64_t)row * p.S * D + dl * 4, p.ws_stats + (int64_t)row * p.S * (uml ? 2 : 1),
                        p.S, uml, grp, SG);
  part[threadIdx.x] = st.acc;
  part_m[threadIdx.x] = st.m;
  part_d[threadIdx.x] = st.den;
  __syncthreads();
  if (!active || grp != 0) return;
  finish_row(part, part_m, part_d, rl * tpr + dl, LPR, SG, p.out + (int64_t)row * D, dl,
             p.lse ? p.lse + row : nullptr);
}

}  // namespace

int launch_merge(const MergeParams& p, int head_dim, void* stream) {
  const int lpr = head_dim / 4;
  const int sg_log2 = split_groups_log2(p.S, lpr, 1, NT);
  const int rows_per_wg = NT / (lpr << sg_log2);
  dim3 grid((unsigned)(((int64_t)p.BH + rows_per_wg - 1) / rows_per_wg));
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
