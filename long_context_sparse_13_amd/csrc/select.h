// Exact workgroup-wide top-k on order-preserving 32-bit keys, ties to the lower
// position, output in ascending position order.
//
// Element e of the row is held by thread e % NT at slot e / NT (keys in registers
// when E > 0; re-read through load_key in every pass when E == 0).  A radix select with
// digits of 12, 12 and 8 bits (LDS histograms) finds the k-th largest key a and the
// number kk of keys equal to a that are kept.  The ascending output needs no sort:
// 64 consecutive positions (one slot of one wavefront) form a run; ballots give each
// run's count of keys > a and == a, one workgroup scan over the runs gives their output
// offsets, and mbcnt gives each lane its place inside the run.  A key equal to a is kept
// iff fewer than kk equal keys precede it — the lower-position tie rule.
#pragma once

#include "sa_device.h"

namespace sa {

template <int NT>
struct SelectShared {
  static constexpr int W = NT / 64;
  static constexpr int MAX_RUNS = 4096;
  uint32_t hist[4096];
  int run_gt[MAX_RUNS];
  int run_eq[MAX_RUNS];
  int wsum[2][W];
  uint32_t sel_digit;
  int sel_kk;
  int done;
};

// Exclusive scan of one int per thread across an NT-thread workgroup.
template <int NT>
__device__ __forceinline__ int wg_excl_scan(int v, int* wsum) {
  constexpr int W = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int x = wave_incl_scan(v, 0, [](int a, int b) { return a + b; });
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) base += (i < w) ? wsum[i] : 0;
  return base + x - v;
}

// Calls f(j) for every slot j; fully unrolled (so register arrays stay in registers)
// when E > 0.
template <int E, typename F>
__device__ __forceinline__ void for_slots(int slots, F&& f) {
  if constexpr (E > 0) {
#pragma unroll
    for (int j = 0; j < E; ++j) f(j);
  } else {
    for (int j = 0; j < slots; ++j) f(j);
  }
}

// Requires n > k >= 1 and n <= NT * slots.  load_key(e) returns the key of position e
// (only called for e < n).  emit(pos, e) is called once for each kept position e, with
// pos = its rank among the kept positions in ascending order (0 .. k-1).
// All NT threads must call it; it contains workgroup barriers.
template <int NT, int E, typename LoadKey, typename Emit>
__device__ __forceinline__ void wg_topk(int n, int k, LoadKey&& load_key, Emit&& emit,
                                        SelectShared<NT>& sh) {
  constexpr int W = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slots = E > 0 ? E : (n + NT - 1) / NT;

  uint32_t reg[E > 0 ? E : 1];
  auto key_at = [&](int j) -> uint32_t {
    const int e = j * NT + tid;
    if constexpr (E > 0) {
      (void)e;
      return reg[j];
    } else {
      return e < n ? load_key(e) : 0u;
    }
  };
  if constexpr (E > 0) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = j * NT + tid;
      reg[j] = e < n ? load_key(e) : 0u;  // key 0 sorts below every finite value
    }
  }

  uint32_t prefix = 0, pmask = 0;
  int kk = k;
  bool early = false;
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int sft = p == 0 ? 20 : (p == 1 ? 8 : 0);
    const int nb = p == 2 ? 256 : 4096;
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    for_slots<E>(slots, [&](int j) {
      const uint32_t key = key_at(j);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> sft) & dmask], 1u);
    });
    __syncthreads();
    // this thread's bins, from the top digit down: [hi - BPT, hi)
    constexpr int BPT = 4096 / NT;
    const int bpt = nb / NT > 0 ? nb / NT : 1;  // bins per thread this pass
    const int hi = nb - bpt * tid;
    uint32_t c[BPT];
    int local = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      c[i] = (i < bpt && hi - 1 - i >= 0) ? sh.hist[hi - 1 - i] : 0u;
      local += (int)c[i];
    }
    int above = wg_excl_scan<NT>(local, sh.wsum[0]);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (i < bpt && hi - 1 - i >= 0) {
        if (above < kk && kk <= above + (int)c[i]) {
          sh.sel_digit = (uint32_t)(hi - 1 - i);
          sh.sel_kk = kk - above;
          sh.done = (kk - above) == (int)c[i];
        }
        above += (int)c[i];
      }
    }
    __syncthreads();
    prefix |= sh.sel_digit << sft;
    pmask |= dmask << sft;
    kk = sh.sel_kk;
    early = sh.done != 0;
    __syncthreads();
    if (early) break;
  }
  const uint32_t thr_gt = early ? prefix : prefix + 1u;
  const uint32_t thr_eq = prefix;
  const int take_eq = early ? 0 : kk;

  const int runs = slots * W;
  for_slots<E>(slots, [&](int j) {
    const uint32_t key = key_at(j);
    const bool gt = key >= thr_gt;
    const uint64_t mg = ballot(gt);
    const uint64_t me = ballot(key == thr_eq && !gt);
    if (lane == 0) {
      sh.run_gt[j * W + w] = __popcll(mg);
      sh.run_eq[j * W + w] = __popcll(me);
    }
  });
  __syncthreads();
  const int per = (runs + NT - 1) / NT;
  int sg = 0, se = 0;
  for (int i = 0; i < per; ++i) {
    const int ri = tid * per + i;
    if (ri < runs) {
      sg += sh.run_gt[ri];
      se += sh.run_eq[ri];
    }
  }
  int bg = wg_excl_scan<NT>(sg, sh.wsum[0]);
  int be = wg_excl_scan<NT>(se, sh.wsum[1]);
  for (int i = 0; i < per; ++i) {
    const int ri = tid * per + i;
    if (ri < runs) {
      const int g0 = sh.run_gt[ri], e0 = sh.run_eq[ri];
      sh.run_gt[ri] = bg;
      sh.run_eq[ri] = be;
      bg += g0;
      be += e0;
    }
  }
  __syncthreads();
  for_slots<E>(slots, [&](int j) {
    const uint32_t key = key_at(j);
    const bool gt = key >= thr_gt;
    const bool eq = key == thr_eq && !gt;
    const uint64_t mg = ballot(gt);
    const uint64_t me = ballot(eq);
    const int gb = sh.run_gt[j * W + w] + lanes_below(mg);
    const int eb = sh.run_eq[j * W + w] + lanes_below(me);
    const int e = j * NT + tid;
    if (gt) emit(gb + min(eb, take_eq), e);
    else if (eq && eb < take_eq) emit(gb + eb, e);
  });
  __syncthreads();  // sh may be reused by the caller
}

}  // namespace sa
