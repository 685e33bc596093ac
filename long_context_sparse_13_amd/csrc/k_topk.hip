// Exact per-row top-k over the causal indexer scores.
//
// [IC] IndexCache page, body paragraph 2 (the indexer selects a small subset of the
// earlier tokens) and [HS2] HySparse2 page, "Más precisión con menos memoria" (the
// subset is made of individual tokens).  For row t the result is the min(k, t+1)
// positions s <= t with the largest scores, ties to the lower s, written ascending.
//
// One 512-thread workgroup (8 wavefronts) per row; scores become order-preserving
// 32-bit keys (-0.0 and +0.0 share a key).  Each wavefront owns one contiguous segment
// of the row.
//  pass 1 (reads the row from HBM): every wavefront builds its own histogram of the top
//         11 key bits (16-bit counters, two per LDS word).  Summed over wavefronts they
//         give the digit d* holding the k-th largest key and kk1, how many keys of that
//         digit are kept; each wavefront's own counts above and at d* give it the offsets
//         of its positions in two LDS lists.
//  pass 2 (reads the row again, now cache-resident): positions with a digit above d* are
//         kept for sure and appended, in position order, to the "sure" list; positions at
//         d* go with their keys to the candidate list.  Order is kept with ballots and
//         mbcnt, so both lists are ascending without any sort.
//  resolve (LDS only): two more radix digits (11 + 10 bits) over the candidates find the
//         exact k-th key a; candidates above a, and the first ones equal to a (lower
//         positions first, i.e. the tie rule), are appended ascending after the sure list.
//  merge: the two ascending lists are merged by binary search into the output row.
// Rows whose candidate digit holds more than kCap positions (massive exact ties) fall
// back to the multi-pass workgroup select of select.h reading the row from memory.
// Rows are issued longest first.
#include "sa_launch.h"
#include "select.h"

namespace sa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kD1Bins = 2048;  // first digit: key bits [31:21]
constexpr int kCap = 4096;     // candidate capacity
constexpr int kKMax = 4096;    // largest k
constexpr int kUnroll = 32;    // loads in flight per lane while streaming

struct TopkShared {
  union {
    uint32_t whist[kTkWaves][kD1Bins / 2];  // pass 1: per-wave 16-bit counters
    struct {
      uint32_t key[kCap];
      int pos[kCap];
    } cand;                                 // pass 2 / resolve: candidate list
    SelectShared<kTkThreads> fallback;      // rows with too many candidates
  } u;
  int sel[kKMax];        // sure list, then the chosen candidates
  uint32_t hist2[2048];  // resolve histograms
  int run_gt[kCap / 64 + 1];
  int run_eq[kCap / 64 + 1];
  int wsure[kTkWaves], wcand[kTkWaves];
  int wsum[2][kTkWaves];
  int misc[8];
};

__device__ __forceinline__ uint32_t get16(const uint32_t* h, int d) {
  return (h[d >> 1] >> ((d & 1) << 4)) & 0xffffu;
}

// Finds, over nb bins (counts from cnt(d)), the digit holding the kk-th largest element:
// writes misc[o] = digit, misc[o+1] = kk - (count above it), misc[o+2] = 1 if that is the
// digit's whole count.  Bins are owned from the top down, bpt per thread.
template <typename Cnt>
__device__ __forceinline__ void find_digit(int nb, int kk, Cnt&& cnt, TopkShared& sh, int o) {
  const int tid = threadIdx.x;
  const int bpt = (nb + kTkThreads - 1) / kTkThreads;
  const int top = nb - 1 - bpt * tid;
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < bpt && top - i >= 0) {
      c[i] = cnt(top - i);
      local += (int)c[i];
    }
  }
  int above = wg_excl_scan<kTkThreads>(local, sh.wsum[0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < bpt && top - i >= 0) {
      if (above < kk && kk <= above + (int)c[i]) {
        sh.misc[o] = top - i;
        sh.misc[o + 1] = kk - above;
        sh.misc[o + 2] = (kk - above) == (int)c[i];
      }
      above += (int)c[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTkThreads) void topk_rows(const float* __restrict__ scores,
                                                        int64_t ld, int T, int row_begin,
                                                        int row_end, int k,
                                                        int32_t* __restrict__ idx) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = row_end - row_begin;
  const int b = blockIdx.x / R;
  const int r = R - 1 - (int)(blockIdx.x % R);  // longest rows first
  const int t = row_begin + r;
  const int n = t + 1;
  const float* __restrict__ row = scores + ((int64_t)b * R + r) * ld;
  int32_t* __restrict__ out = idx + ((int64_t)b * T + t) * k;

  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }

  // ---- pass 1: per-wave histograms of the top 11 key bits
  const int seg = ((n + kTkThreads - 1) / kTkThreads) * 64;
  const int lo = min(n, w * seg), hi = min(n, lo + seg);
  for (int i = tid; i < kTkWaves * kD1Bins / 2; i += kTkThreads) (&sh.u.whist[0][0])[i] = 0u;
  __syncthreads();
  uint32_t* wh = sh.u.whist[w];
  for (int e0 = lo; e0 < hi; e0 += 64 * kUnroll) {
    float v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e0 + u * 64 + lane;
      v[u] = e < hi ? row[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e0 + u * 64 + lane;
      if (e < hi) {
        const uint32_t d = order_key(v[u]) >> 21;
        atomicAdd(&wh[d >> 1], 1u << ((d & 1u) << 4));
      }
    }
  }
  __syncthreads();

  // ---- digit of the k-th largest key; per-wave counts above / at it
  find_digit(kD1Bins, k, [&](int d) {
    uint32_t s = 0;
#pragma unroll
    for (int ww = 0; ww < kTkWaves; ++ww) s += get16(sh.u.whist[ww], d);
    return s;
  }, sh, 0);
  const int dstar = sh.misc[0];
  const int kk1 = sh.misc[1];
  {
    int above = 0;
    for (int d = dstar + 1 + lane; d < kD1Bins; d += 64) above += (int)get16(wh, d);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) above += __shfl_xor(above, m, 64);
    if (lane == 0) {
      sh.wsure[w] = above;
      sh.wcand[w] = (int)get16(wh, dstar);
    }
  }
  __syncthreads();
  int sure_off = 0, cand_off = 0, n_cand = 0;
#pragma unroll
  for (int ww = 0; ww < kTkWaves; ++ww) {
    sure_off += ww < w ? sh.wsure[ww] : 0;
    cand_off += ww < w ? sh.wcand[ww] : 0;
    n_cand += sh.wcand[ww];
  }
  const int n_sure = k - kk1;
  __syncthreads();  // the histogram region becomes the candidate list

  if (n_cand > kCap) {
    wg_topk<kTkThreads, 0>(
        n, k, [&](int e) { return order_key(row[e]); }, [&](int pos, int e) { out[pos] = e; },
        sh.u.fallback);
    return;
  }

  // ---- pass 2: sure positions and candidates, in position order
  for (int e0 = lo; e0 < hi; e0 += 64 * kUnroll) {
    float v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e0 + u * 64 + lane;
      v[u] = e < hi ? row[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e0 + u * 64 + lane;
      const uint32_t key = order_key(v[u]);
      const int d = (int)(key >> 21);
      const bool in = e < hi;
      const bool sure = in && d > dstar;
      const bool cand = in && d == dstar;
      const uint64_t ms = ballot(sure), mc = ballot(cand);
      if (sure) sh.sel[sure_off + lanes_below(ms)] = e;
      if (cand) {
        const int p = cand_off + lanes_below(mc);
        sh.u.cand.key[p] = key;
        sh.u.cand.pos[p] = e;
      }
      sure_off += __popcll(ms);
      cand_off += __popcll(mc);
    }
  }
  __syncthreads();

  // ---- resolve the candidates: keep kk1 of them (largest keys, lower positions on ties)
  uint32_t thr_gt, thr_eq;
  int take_eq;
  if (kk1 == n_cand) {  // every candidate is kept
    thr_gt = 0u;
    thr_eq = 0u;
    take_eq = 0;
  } else {
    for (int i = tid; i < 2048; i += kTkThreads) sh.hist2[i] = 0u;
    __syncthreads();
    for (int e = tid; e < n_cand; e += kTkThreads)
      atomicAdd(&sh.hist2[(sh.u.cand.key[e] >> 10) & 2047u], 1u);
    __syncthreads();
    find_digit(2048, kk1, [&](int d) { return sh.hist2[d]; }, sh, 3);
    const uint32_t d2 = (uint32_t)sh.misc[3];
    const int kk2 = sh.misc[4];
    const uint32_t pre2 = ((uint32_t)dstar << 21) | (d2 << 10);
    if (sh.misc[5]) {
      thr_gt = pre2;
      thr_eq = 0u;
      take_eq = 0;
    } else {
      __syncthreads();
      for (int i = tid; i < 1024; i += kTkThreads) sh.hist2[i] = 0u;
      __syncthreads();
      for (int e = tid; e < n_cand; e += kTkThreads) {
        const uint32_t key = sh.u.cand.key[e];
        if ((key >> 10) == (pre2 >> 10)) atomicAdd(&sh.hist2[key & 1023u], 1u);
      }
      __syncthreads();
      find_digit(1024, kk2, [&](int d) { return sh.hist2[d]; }, sh, 5);  // misc[5..7]
      const uint32_t a = pre2 | (uint32_t)sh.misc[5];
      thr_gt = a + 1u;
      thr_eq = a;
      take_eq = sh.misc[6];
    }
  }
  // order-preserving compaction of the chosen candidates after the sure list
  const int runs = (n_cand + 63) / 64;
  const int slots = (n_cand + kTkThreads - 1) / kTkThreads;
  for (int j = 0; j < slots; ++j) {
    const int e = j * kTkThreads + tid;
    const uint32_t key = e < n_cand ? sh.u.cand.key[e] : 0u;
    const bool in = e < n_cand;
    const bool gt = in && key >= thr_gt;
    const bool eq = in && !gt && take_eq > 0 && key == thr_eq;
    const uint64_t mg = ballot(gt), me = ballot(eq);
    const int run = e >> 6;
    if (lane == 0 && run < runs) {
      sh.run_gt[run] = __popcll(mg);
      sh.run_eq[run] = __popcll(me);
    }
  }
  __syncthreads();
  if (w == 0) {  // exclusive scan of the (few) runs by one wavefront
    int gsum = 0, esum = 0;
    for (int r0 = 0; r0 < runs; r0 += 64) {
      const int ri = r0 + lane;
      const int g0 = ri < runs ? sh.run_gt[ri] : 0, e0 = ri < runs ? sh.run_eq[ri] : 0;
      int gx = g0, ex = e0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int gy = __shfl_up(gx, o, 64), ey = __shfl_up(ex, o, 64);
        if (lane >= o) {
          gx += gy;
          ex += ey;
        }
      }
      if (ri < runs) {
        sh.run_gt[ri] = gsum + gx - g0;
        sh.run_eq[ri] = esum + ex - e0;
      }
      gsum += __shfl(gx, 63, 64);
      esum += __shfl(ex, 63, 64);
    }
  }
  __syncthreads();
  for (int j = 0; j < slots; ++j) {
    const int e = j * kTkThreads + tid;
    const bool in = e < n_cand;
    const uint32_t key = in ? sh.u.cand.key[e] : 0u;
    const bool gt = in && key >= thr_gt;
    const bool eq = in && !gt && take_eq > 0 && key == thr_eq;
    const uint64_t mg = ballot(gt), me = ballot(eq);
    const int run = e >> 6;
    if (in) {
      const int gb = sh.run_gt[run] + lanes_below(mg);
      const int eb = sh.run_eq[run] + lanes_below(me);
      if (gt) sh.sel[n_sure + gb + min(eb, take_eq)] = sh.u.cand.pos[e];
      else if (eq && eb < take_eq) sh.sel[n_sure + gb + eb] = sh.u.cand.pos[e];
    }
  }
  __syncthreads();

  // ---- merge the two ascending lists sel[0, n_sure) and sel[n_sure, k)
  const int nc = k - n_sure;
  for (int i = tid; i < k; i += kTkThreads) {
    const int v = sh.sel[i];
    const int* other = i < n_sure ? sh.sel + n_sure : sh.sel;
    int lo2 = 0, hi2 = i < n_sure ? nc : n_sure;  // count of entries of the other list < v
    while (lo2 < hi2) {
      const int mid = (lo2 + hi2) >> 1;
      if (other[mid] < v) lo2 = mid + 1;
      else hi2 = mid;
    }
    out[(i < n_sure ? i : i - n_sure) + lo2] = v;
  }
}

hipError_t launch_topk_select(const float* scores, int64_t ld, int B, int T, int row_begin,
                              int row_end, int k, int32_t* idx, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)B * (row_end - row_begin)));
  hipLaunchKernelGGL(topk_rows, grid, dim3(kTkThreads), 0, st, scores, ld, T, row_begin, row_end,
                     k, idx);
  return hipGetLastError();
}

}  // namespace sa
