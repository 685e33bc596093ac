// Exact per-row top-k over the causal indexer scores (sa_topk_select).
//
// One 256-thread workgroup (4 wavefronts) per row, rows issued longest first; the
// two-pass radix selection over the row is topk_row in topk_common.h.
#include "sa_launch.h"
#include "topk_common.h"

namespace sa {

__global__ __launch_bounds__(kTkThreads) void topk_rows(const float* __restrict__ scores,
                                                        int64_t ld, int T, int row_begin,
                                                        int row_end, int k,
                                                        int32_t* __restrict__ idx) {
  __shared__ TopkShared sh;
  const int R = row_end - row_begin;
  const int b = blockIdx.x / R;
  const int r = R - 1 - (int)(blockIdx.x % R);  // longest rows first
  const int t = row_begin + r;
  const int n = t + 1;
  int32_t* __restrict__ out = idx + ((int64_t)b * T + t) * k;
  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  topk_row(scores + ((int64_t)b * R + r) * ld, n, k, out, sh);
}

hipError_t launch_topk_select(const float* scores, int64_t ld, int B, int T, int row_begin,
                              int row_end, int k, int32_t* idx, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)B * (row_end - row_begin)));
  hipLaunchKernelGGL(topk_rows, grid, dim3(kTkThreads), 0, st, scores, ld, T, row_begin, row_end,
                     k, idx);
  return hipGetLastError();
}

}  // namespace sa
