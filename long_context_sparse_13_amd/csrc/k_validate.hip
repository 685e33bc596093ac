// Debug-mode check of the index contract of the sparse attention (SA_VALIDATE=1): the
// positions a query row lists must be distinct among those the attention counts.
//
// IndexCache page, body paragraph 2: each query attends to its selected subset of earlier
// tokens, a set.  The forward and backward count a listed position s of row t when
// 0 <= s <= t - window (the window's own positions and anything outside [0, t] are
// skipped), so a repeated s in that range would be counted twice.  Only this check runs
// in debug mode; it synchronises the stream to hand its result back to the host.
#include <hip/hip_runtime.h>

#include <climits>

#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kValThreads = 256;
constexpr int kValLds = 8192;  // entries sorted in LDS per row (32 KB)

// Flat row index b * T + t of the first offending row found, ~0 when none.
__device__ unsigned long long g_first_dup_row;

__device__ __forceinline__ void report(int b, int T, int t) {
  atomicMin(&g_first_dup_row, (unsigned long long)b * (unsigned long long)T + (unsigned)t);
}

// One workgroup per row: the counted entries (others as INT_MAX) are sorted in LDS by a
// bitonic network over n2 (a power of two >= topk) slots, then equal neighbours are looked
// for.
__global__ __launch_bounds__(kValThreads) void idx_unique_sorted(const int32_t* __restrict__ idx,
                                                                 int T, int topk, int window,
                                                                 int row_begin, int n2) {
  __shared__ int s[kValLds];
  const int t = row_begin + (int)blockIdx.x;
  const int b = (int)blockIdx.y;
  const int32_t* row = idx + ((int64_t)b * T + t) * topk;
  const int lim = t - window;
  for (int i = threadIdx.x; i < n2; i += kValThreads) {
    int v = INT_MAX;
    if (i < topk) {
      const int x = row[i];
      if (x >= 0 && x <= lim) v = x;
    }
    s[i] = v;
  }
  __syncthreads();
  for (int kk = 2; kk <= n2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += kValThreads) {
        const int p = i ^ j;
        if (p > i) {
          const int a = s[i], c = s[p];
          if ((a > c) == ((i & kk) == 0)) {
            s[i] = c;
            s[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  bool dup = false;
  for (int i = threadIdx.x; i + 1 < n2; i += kValThreads)
    dup |= s[i] != INT_MAX && s[i] == s[i + 1];
  if (dup) report(b, T, t);
}

// Rows longer than the LDS sort holds: every counted entry is compared with the entries
// after it (quadratic, debug mode only).
__global__ __launch_bounds__(kValThreads) void idx_unique_pairs(const int32_t* __restrict__ idx,
                                                                int T, int topk, int window,
                                                                int row_begin) {
  const int t = row_begin + (int)blockIdx.x;
  const int b = (int)blockIdx.y;
  const int32_t* row = idx + ((int64_t)b * T + t) * topk;
  const int lim = t - window;
  bool dup = false;
  for (int i = threadIdx.x; i < topk; i += kValThreads) {
    const int x = row[i];
    if (x < 0 || x > lim) continue;
    for (int j = i + 1; j < topk; ++j) dup |= row[j] == x;
  }
  if (dup) report(b, T, t);
}

}  // namespace

hipError_t validate_idx_unique(const int32_t* idx, int B, int T, int topk, int window,
                               int row_begin, int row_end, long long* bad_row, hipStream_t st) {
  *bad_row = -1;
  if (!idx || topk <= 0 || row_end <= row_begin) return hipSuccess;
  const unsigned long long none = ~0ull;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_first_dup_row), &none, sizeof(none), 0,
                                        hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(row_end - row_begin), (unsigned)B);
  if (topk <= kValLds) {
    int n2 = 2;
    while (n2 < topk) n2 <<= 1;
    hipLaunchKernelGGL(idx_unique_sorted, grid, dim3(kValThreads), 0, st, idx, T, topk, window,
                       row_begin, n2);
  } else {
    hipLaunchKernelGGL(idx_unique_pairs, grid, dim3(kValThreads), 0, st, idx, T, topk, window,
                       row_begin);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long found = none;
  e = hipMemcpyFromSymbolAsync(&found, HIP_SYMBOL(g_first_dup_row), sizeof(found), 0,
                               hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  if (found != none) *bad_row = (long long)found;
  return hipSuccess;
}

}  // namespace sa
