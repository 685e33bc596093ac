// Exact per-row top-k building blocks shared by the top-k kernels: order-preserving
// digits, LDS digit search, row streaming, and the final selection over a hit list
// held in LDS in position order.
//
// [IC] IndexCache page, body paragraph 2 (the indexer selects a small subset of the
// earlier tokens) and [HS2] HySparse2 page, "Más precisión con menos memoria" (the
// subset is made of individual tokens): for row t the result is the min(k, t+1)
// positions s <= t with the largest scores, ties to the lower s, written ascending.
#pragma once

#include "select.h"

namespace sa {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kD1Bins = 2048;   // first digit: key bits [31:21]
constexpr int kHitCap = 8192;   // hit list capacity
constexpr int kLoads = 8;                // 16-byte loads per lane in flight while streaming
constexpr int kChunk = 64 * 4 * kLoads;  // positions a wavefront streams per step

struct TopkShared {
  union {
    uint32_t whist[kTkWaves][kD1Bins];  // pass 1: per-wave counters
    struct {
      uint32_t key[kHitCap];
      int pos[kHitCap];
    } hit;                              // pass 2 / resolve: the hit list
    SelectShared<kTkThreads> fallback;  // rows with too many hits
  } u;
  uint32_t hist2[2048];  // resolve histograms
  int run_gt[kHitCap / 64];
  int run_eq[kHitCap / 64];
  int whits[kTkWaves];
  int wsum[2][kTkWaves];
  int misc[8];
};

// Digit (top 11 bits of the order-preserving key) of a float, -0.0 counted as +0.0:
// positive u -> (u >> 21) | 0x400, negative u -> ~(u >> 21) & 0x7ff.
__device__ __forceinline__ uint32_t digit11(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t s = (uint32_t)((int32_t)u >> 31);
  return (u >> 21) ^ ((s & 0x3ffu) | 0x400u);
}

// Finds, over nb bins (counts from cnt(d)), the digit holding the kk-th largest element:
// writes misc[o] = digit, misc[o+1] = kk - (count above it), misc[o+2] = 1 if that is the
// digit's whole count.  Bins are owned from the top down, bpt per thread.
template <typename Cnt>
__device__ __forceinline__ void find_digit(int nb, int kk, Cnt&& cnt, TopkShared& sh, int o) {
  const int tid = threadIdx.x;
  const int bpt = (nb + kTkThreads - 1) / kTkThreads;
  const int top = nb - 1 - bpt * tid;
  uint32_t c[8];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = (i < bpt && top - i >= 0) ? cnt(top - i) : 0u;
    local += (int)c[i];
  }
  int above = wg_excl_scan<kTkThreads>(local, sh.wsum[0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
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

// Streams positions [lo, hi) of the row (lo a multiple of 4, the row 16-byte aligned) in
// groups of 4 consecutive positions per lane: f(e, x[4], valid[4]) with e the first
// position of the group.  A wavefront's call order covers its positions in increasing
// order, 256 per call round (lane-major inside a round); kLoads loads per lane are in
// flight, and full chunks run without per-position guards.
template <typename F>
__device__ __forceinline__ void stream_segment(const float* __restrict__ row, int lo, int hi,
                                               int lane, F&& f) {
  int e0 = lo;
  for (; e0 + kChunk <= hi; e0 += kChunk) {
    f32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(row + e0 + u * 256 + lane * 4);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const bool ok[4] = {true, true, true, true};
      const float x[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
      f(e0 + u * 256 + lane * 4, x, ok);
    }
  }
  if (e0 < hi) {  // the last, partial chunk: 16-byte loads where the group is whole
    f32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = e0 + u * 256 + lane * 4;
      if (e + 3 < hi) {
        v[u] = *reinterpret_cast<const f32x4*>(row + e);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[u][c] = e + c < hi ? row[e + c] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = e0 + u * 256 + lane * 4;
      const bool ok[4] = {e < hi, e + 1 < hi, e + 2 < hi, e + 3 < hi};
      const float x[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
      f(e, x, ok);
    }
  }
}


// Keeps, from the hit list sh.u.hit (n_hits keys and positions, in increasing position
// order), every key of digit > dstar and the kk1 largest keys of digit dstar (lower
// positions first among equal keys), and writes the kept positions ascending to out.
// whole: kk1 is the whole count of digit dstar.  The list may also hold keys of digits
// below dstar; they are never kept.  All threads of the workgroup call it.
__device__ inline void resolve_emit(TopkShared& sh, int n_hits, uint32_t dstar, int kk1,
                                    bool whole, int32_t* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t dlo = dstar << 21;   // smallest key of digit d*
  const uint32_t dhi = dlo + (1u << 21);
  uint32_t thr_gt = dlo;              // keys >= thr_gt are kept
  uint32_t thr_eq = 0u;               // keys == thr_eq are kept while fewer than take_eq precede
  int take_eq = 0;
  if (!whole) {
    for (int i = tid; i < 2048; i += kTkThreads) sh.hist2[i] = 0u;
    __syncthreads();
    for (int e = tid; e < n_hits; e += kTkThreads) {
      const uint32_t key = sh.u.hit.key[e];
      if (key >= dlo && key < dhi) atomicAdd(&sh.hist2[(key >> 10) & 2047u], 1u);
    }
    __syncthreads();
    find_digit(2048, kk1, [&](int d) { return sh.hist2[d]; }, sh, 3);
    const uint32_t pre2 = dlo | ((uint32_t)sh.misc[3] << 10);
    const int kk2 = sh.misc[4];
    if (sh.misc[5]) {
      thr_gt = pre2;
    } else {
      __syncthreads();
      for (int i = tid; i < 1024; i += kTkThreads) sh.hist2[i] = 0u;
      __syncthreads();
      for (int e = tid; e < n_hits; e += kTkThreads) {
        const uint32_t key = sh.u.hit.key[e];
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

  // ---- output: order-preserving compaction of the kept hits
  const int runs = (n_hits + 63) / 64;
  const int slots = (n_hits + kTkThreads - 1) / kTkThreads;
  for (int j = 0; j < slots; ++j) {
    const int e = j * kTkThreads + tid;
    const bool in = e < n_hits;
    const uint32_t key = in ? sh.u.hit.key[e] : 0u;
    const bool gt = in && key >= thr_gt;
    const bool eq = in && !gt && take_eq > 0 && key == thr_eq;
    const uint64_t mg = ballot(gt), me = ballot(eq);
    if (lane == 0 && (e >> 6) < runs) {
      sh.run_gt[e >> 6] = __popcll(mg);
      sh.run_eq[e >> 6] = __popcll(me);
    }
  }
  __syncthreads();
  if (w == 0) {  // exclusive scan of the runs by one wavefront
    int gsum = 0, esum = 0;
    for (int r0 = 0; r0 < runs; r0 += 64) {
      const int ri = r0 + lane;
      const int g0 = ri < runs ? sh.run_gt[ri] : 0, e0 = ri < runs ? sh.run_eq[ri] : 0;
      const int gx = wave_incl_scan(g0, 0, [](int a, int b) { return a + b; });
      const int ex = wave_incl_scan(e0, 0, [](int a, int b) { return a + b; });
      if (ri < runs) {
        sh.run_gt[ri] = gsum + gx - g0;
        sh.run_eq[ri] = esum + ex - e0;
      }
      gsum += __builtin_amdgcn_readlane(gx, 63);
      esum += __builtin_amdgcn_readlane(ex, 63);
    }
  }
  __syncthreads();
  for (int j = 0; j < slots; ++j) {
    const int e = j * kTkThreads + tid;
    const bool in = e < n_hits;
    const uint32_t key = in ? sh.u.hit.key[e] : 0u;
    const bool gt = in && key >= thr_gt;
    const bool eq = in && !gt && take_eq > 0 && key == thr_eq;
    const uint64_t mg = ballot(gt), me = ballot(eq);
    if (in) {
      const int gb = sh.run_gt[e >> 6] + lanes_below(mg);
      const int eb = sh.run_eq[e >> 6] + lanes_below(me);
      if (gt) out[gb + min(eb, take_eq)] = sh.u.hit.pos[e];
      else if (eq && eb < take_eq) out[gb + eb] = sh.u.hit.pos[e];
    }
  }
}

// The top-k of one row of n > k float scores (16-byte aligned, readable by this
// workgroup), written ascending to out[0..k).
//  pass 1 (reads the row from HBM): every wavefront counts the top 11 key bits (the
//         digit) of its own contiguous segment into its own LDS histogram.  Summed, the
//         histograms give the digit d* holding the k-th largest key and kk1, how many
//         keys of digit d* are kept; each wavefront's count of digits >= d* gives its
//         offset in the hit list.
//  pass 2 (reads the row again, now cache-resident): positions with digit >= d* ("hits")
//         go with their keys to the hit list, in position order (ballot + mbcnt).
//  resolve (LDS only): two more radix digits (11 + 10 bits) among the hits at d* find
//         the exact k-th key; one order-preserving compaction writes the answer.
// Rows with more hits than kHitCap (massive exact ties) fall back to the multi-pass
// workgroup select of select.h reading the row from memory.
__device__ inline void topk_row(const float* __restrict__ row, int n, int k,
                                int32_t* __restrict__ out, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // ---- pass 1: per-wave digit histograms
  const int seg = ((n + kTkThreads - 1) / kTkThreads) * 64;
  const int lo = min(n, w * seg), hi = min(n, lo + seg);
  for (int i = tid; i < kTkWaves * kD1Bins; i += kTkThreads) (&sh.u.whist[0][0])[i] = 0u;
  __syncthreads();
  uint32_t* wh = sh.u.whist[w];
  stream_segment(row, lo, hi, lane, [&](int, const float* x, const bool* ok) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (ok[c]) atomicAdd(&wh[digit11(x[c])], 1u);
  });
  __syncthreads();

  // ---- digit of the k-th largest key; per-wave counts of hits (digit >= d*)
  find_digit(kD1Bins, k, [&](int d) {
    uint32_t s = 0;
#pragma unroll
    for (int ww = 0; ww < kTkWaves; ++ww) s += sh.u.whist[ww][d];
    return s;
  }, sh, 0);
  const uint32_t dstar = (uint32_t)sh.misc[0];
  const int kk1 = sh.misc[1];
  {
    int cnt = 0;
    for (int d = (int)dstar + lane; d < kD1Bins; d += 64) cnt += (int)wh[d];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, 64);
    if (lane == 0) sh.whits[w] = cnt;
  }
  __syncthreads();
  int hit_off = 0, n_hits = 0;
#pragma unroll
  for (int ww = 0; ww < kTkWaves; ++ww) {
    hit_off += ww < w ? sh.whits[ww] : 0;
    n_hits += sh.whits[ww];
  }
  const int n_sure = k - kk1;  // hits above d*
  const bool whole = kk1 == n_hits - n_sure;
  __syncthreads();  // the histogram region becomes the hit list

  if (n_hits > kHitCap) {
    wg_topk<kTkThreads, 0>(
        n, k, [&](int e) { return order_key(row[e]); }, [&](int pos, int e) { out[pos] = e; },
        sh.u.fallback);
    return;
  }

  // ---- pass 2: the hit list, in position order
  stream_segment(row, lo, hi, lane, [&](int e, const float* x, const bool* ok) {
    bool hit[4];
    uint64_t m[4];
    int before = 0;  // hits of the lower lanes in this round (lane-major order)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      hit[c] = ok[c] && digit11(x[c]) >= dstar;
      m[c] = ballot(hit[c]);
      before += lanes_below(m[c]);
    }
    if ((m[0] | m[1] | m[2] | m[3]) != 0ull) {
      int p = hit_off + before;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (hit[c]) {
          sh.u.hit.key[p] = order_key(x[c]);
          sh.u.hit.pos[p] = e + c;
          ++p;
        }
      }
      hit_off += __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
    }
  });
  __syncthreads();

  resolve_emit(sh, n_hits, dstar, kk1, whole, out);
}

}  // namespace sa
