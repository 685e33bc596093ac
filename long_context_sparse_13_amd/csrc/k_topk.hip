// Exact per-row top-k over the causal indexer scores.
//
// [IC] IndexCache page, body paragraph 2 (the indexer selects a small subset of the
// earlier tokens) and [HS2] HySparse2 page, "Más precisión con menos memoria" (the
// subset is made of individual tokens).  For row t the result is the min(k, t+1)
// positions s <= t with the largest scores, ties to the lower s, written ascending.
//
// One 1024-thread workgroup per row runs the workgroup radix select of select.h on
// order-preserving keys of the scores (-0.0 and +0.0 share a key).  Rows of up to
// 1024*E positions keep their keys in registers (E = 1..64, rows up to 65,536); longer
// rows re-read the scores in each pass (E = 0).  Rows are issued longest first.
#include "sa_launch.h"
#include "select.h"

namespace sa {

constexpr int kTopkThreads = 1024;

template <int E>
__global__ __launch_bounds__(kTopkThreads) void topk_rows(const float* __restrict__ scores,
                                                          int64_t ld, int T, int row_begin,
                                                          int row_end, int k,
                                                          int32_t* __restrict__ idx) {
  __shared__ SelectShared<kTopkThreads> sh;
  const int tid = threadIdx.x;
  const int R = row_end - row_begin;
  const int b = blockIdx.x / R;
  const int r = R - 1 - (int)(blockIdx.x % R);
  const int t = row_begin + r;
  const int n = t + 1;
  const float* row = scores + ((int64_t)b * R + r) * ld;
  int32_t* out = idx + ((int64_t)b * T + t) * k;

  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  wg_topk<kTopkThreads, E>(
      n, k, [&](int e) { return order_key(row[e]); }, [&](int pos, int e) { out[pos] = e; }, sh);
}

hipError_t launch_topk_select(const float* scores, int64_t ld, int B, int T, int row_begin,
                              int row_end, int k, int32_t* idx, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)B * (row_end - row_begin)));
  const dim3 block(kTopkThreads);
  const int need = (row_end + kTopkThreads - 1) / kTopkThreads;  // slots of the longest row
#define SA_TOPK(EE) \
  hipLaunchKernelGGL(topk_rows<EE>, grid, block, 0, st, scores, ld, T, row_begin, row_end, k, idx)
  if (need <= 1) SA_TOPK(1);
  else if (need <= 2) SA_TOPK(2);
  else if (need <= 4) SA_TOPK(4);
  else if (need <= 8) SA_TOPK(8);
  else if (need <= 16) SA_TOPK(16);
  else if (need <= 32) SA_TOPK(32);
  else if (need <= 64) SA_TOPK(64);
  else SA_TOPK(0);
#undef SA_TOPK
  return hipGetLastError();
}

}  // namespace sa
