// Gathered causal sparse attention forward over S_t = listed indices U window.
//
// [IC] IndexCache page, body paragraph 2: each query attends only to its selected
// subset.  [HS2] HySparse2 page, "Dos niveles para compartir la caché": the most
// recent tokens are forced into the selected set.  [NSA] Native Sparse Attention page,
// "Análisis Profundo": group-centric loading, one K/V fetch shared by the query heads
// of a KV group.
//
// Two kernels:
//  * sparse_attn_mfma<D, OFS32>: bf16, up to 16 query heads per KV head.  One wavefront
//    per (batch, token, KV head); keys are streamed 32 at a time through GroupAttn (MFMA
//    over the grouped heads, online softmax).  Held to 3 wavefronts per SIMD (<= 168
//    registers).  The kernel is bound by how many gathered rows the memory pipeline keeps
//    in flight against the L2 / Infinity Cache latency (with every gathered row an L2 hit
//    it runs ~15 % faster; halving its VALU instructions, or cutting the K loads'
//    addresser work by staging them through LDS or loading them quad-contiguous and
//    permuting lanes, gains nothing), so more resident wavefronts beat a second tile of
//    registers per wavefront; within one tile's registers the next tile's rows are
//    requested as soon as the current tile's K and V have been consumed, and OFS32 (one KV head's rows of a
//    batch within 4 GB) addresses rows as a uniform base plus a 32-bit offset.  Items are
//    taken in ranges of about 8,192, last rows first, each range dealt to the XCDs in
//    contiguous pieces (xcd_item_phased): fewer bytes past L2 and ~12 % less time than one
//    range over the whole sequence.  Q and the index row are read
//    with non-temporal loads so they do not evict gathered K/V rows (O is written with
//    ordinary stores, which L2 combines into whole lines).  The listed indices are visited first
//    (positions inside the window or outside [0, t] are masked out, so each key is
//    counted once), then the window [t-W+1, t].
//  * sparse_attn_valu<D, BF16>: any dtype, up to 64 heads per group (G*D <= 4096); plain
//    float32 vector arithmetic, one wavefront per (batch, token, KV head), 64 keys per
//    step with one key per lane for the logits and lanes over (head, d) for P.V.
#include "attn_tile.h"
#include "sa_launch.h"

namespace sa {

template <int D, bool OFS32>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void sparse_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, int B, int T, int Hq,
    int Hkv, int topk, int window, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int r0, int nrows, int phases) {
  using GA = GroupAttn<D, OFS32>;
  __shared__ __attribute__((aligned(16))) unsigned char vl[GA::LDS_BYTES];

  const int lane = threadIdx.x;
  const int n = lane & 15, grp = lane >> 4;
  const int64_t item = xcd_item_phased(blockIdx.x, (int64_t)B * nrows * Hkv, phases);
  if (item < 0) return;
  const int g = (int)(item % Hkv);
  const int t = r0 + (int)((item / Hkv) % nrows);
  const int b = (int)(item / ((int64_t)Hkv * nrows));
  const int G = Hq / Hkv;
  const int h = g * G + n;
  const bool hv = n < G;

  GA ga;
  ga.init(hv ? q + (((int64_t)b * T + t) * Hq + h) * D : nullptr, grp);

  const int64_t stride = (int64_t)Hkv * D;
  const uint16_t* kbase = k + ((int64_t)b * T * Hkv + g) * D;
  const uint16_t* vbase = v + ((int64_t)b * T * Hkv + g) * D;
  const int32_t* irow = idx ? idx + ((int64_t)b * T + t) * topk : nullptr;

  const int n_idx = (topk + 31) / 32;
  const int n_win = (window + 31) / 32;
  const int slot = lane & 31;
  const int last_listed = t - window;  // listed keys must satisfy 0 <= s <= t - window
  const int wlo = t - window + 1;
  auto fetch = [&](int tile) -> int {
    if (tile < n_idx) {
      const int e = tile * 32 + slot;
      return e < topk ? ld_nt(irow + e) : -1;
    }
    return wlo + (tile - n_idx) * 32 + slot;
  };
  auto finish = [&](int tile, int raw, int& key, uint32_t& vm) {
    const bool ok = tile < n_idx ? (raw >= 0 && raw <= last_listed) : (raw >= 0 && raw <= t);
    vm = (uint32_t)ballot(ok);
    key = ok ? raw : 0;
  };
  ga.run(n_idx + n_win, fetch, finish, kbase, vbase, stride, vl, scale_log2, lane);

  const float l = ga.total_l();
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (hv) {
    uint16_t* orow = out + (((int64_t)b * T + t) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < GA::DT; ++dt) {
      const f32x4 a = ga.acc[dt] * inv;
      const u32x2 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
      st8(orow + dt * 16 + grp * 4, w);
    }
    if (lse && grp == 0)
      lse[((int64_t)b * Hq + h) * T + t] = l > 0.f ? (ga.m_run + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------------------------
template <bool BF>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <int D, bool BF>
__global__ __launch_bounds__(64) void sparse_attn_valu(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ idx, int B, int T, int Hq, int Hkv, int topk, int window,
    float scale_log2, void* __restrict__ out, float* __restrict__ lse, int r0, int nrows) {
  constexpr int MAXE = 4096;              // G * D
  __shared__ float qs[MAXE];               // scaled queries of the group, [G][D]
  __shared__ float os[MAXE];               // output accumulators, [G][D]
  __shared__ float ps[64 * 65];            // probabilities of the step, [key][G] (G <= 64)
  __shared__ float ms[64], ls[64], al[64]; // per-head running max, sum, rescale
  __shared__ int keys[64];

  const int lane = threadIdx.x;
  const int64_t item = xcd_item(blockIdx.x, (int64_t)B * nrows * Hkv);
  if (item < 0) return;
  const int g = (int)(item % Hkv);
  const int t = r0 + (int)((item / Hkv) % nrows);
  const int b = (int)(item / ((int64_t)Hkv * nrows));
  const int G = Hq / Hkv;
  const int GD = G * D;

  const int64_t qoff = (((int64_t)b * T + t) * Hq + (int64_t)g * G) * D;
  for (int e = lane; e < GD; e += 64) {
    qs[e] = load_elem<BF>(q, qoff + e) * scale_log2;
    os[e] = 0.f;
  }
  for (int hh = lane; hh < G; hh += 64) {
    ms[hh] = -INFINITY;
    ls[hh] = 0.f;
  }
  __syncthreads();

  const int64_t stride = (int64_t)Hkv * D;
  const int64_t kvoff = ((int64_t)b * T * Hkv + g) * D;
  const int32_t* irow = idx ? idx + ((int64_t)b * T + t) * topk : nullptr;
  const int n_idx = (topk + 63) / 64;
  const int n_win = (window + 63) / 64;
  const int wlo = t - window + 1;

  for (int tile = 0; tile < n_idx + n_win; ++tile) {
    int key;
    bool ok;
    if (tile < n_idx) {
      const int e = tile * 64 + lane;
      key = e < topk ? irow[e] : -1;
      ok = key >= 0 && key <= t - window;
    } else {
      key = wlo + (tile - n_idx) * 64 + lane;
      ok = key >= 0 && key <= t;
    }
    if (ballot(ok) == 0ull) continue;
    keys[lane] = ok ? key : -1;

    // logits of this lane's key for every head of the group
    for (int hh = 0; hh < G; ++hh) ps[lane * 65 + hh] = -INFINITY;
    if (ok) {
      const int64_t kr = kvoff + (int64_t)key * stride;
      for (int hh = 0; hh < G; ++hh) {
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += qs[hh * D + d] * load_elem<BF>(k, kr + d);
        ps[lane * 65 + hh] = acc;
      }
    }
    __syncthreads();
    // per-head max and rescale (one lane per head)
    for (int hh = lane; hh < G; hh += 64) {
      float mt = -INFINITY;
      for (int j = 0; j < 64; ++j) mt = fmaxf(mt, ps[j * 65 + hh]);
      const float mn = fmaxf(ms[hh], mt);
      al[hh] = exp2f(ms[hh] - mn);
      float sum = 0.f;
      for (int j = 0; j < 64; ++j) {
        const float p = exp2f(ps[j * 65 + hh] - mn);
        ps[j * 65 + hh] = p;
        sum += p;
      }
      ls[hh] = ls[hh] * al[hh] + sum;
      ms[hh] = mn;
    }
    __syncthreads();
    // P.V, lanes over (head, d)
    for (int e = lane; e < GD; e += 64) {
      const int hh = e / D, d = e - hh * D;
      float acc = os[e] * al[hh];
      for (int j = 0; j < 64; ++j) {
        const int kk = keys[j];
        if (kk >= 0) acc += ps[j * 65 + hh] * load_elem<BF>(v, kvoff + (int64_t)kk * stride + d);
      }
      os[e] = acc;
    }
    __syncthreads();
  }

  for (int e = lane; e < GD; e += 64) {
    const int hh = e / D;
    const float l = ls[hh];
    const float o = l > 0.f ? os[e] / l : 0.f;
    if constexpr (BF) reinterpret_cast<uint16_t*>(out)[qoff + e] = (uint16_t)f32_to_bf16_bits(o);
    else reinterpret_cast<float*>(out)[qoff + e] = o;
  }
  if (lse)
    for (int hh = lane; hh < G; hh += 64) {
      const float l = ls[hh];
      lse[((int64_t)b * Hq + (int64_t)g * G + hh) * T + t] =
          l > 0.f ? (ms[hh] + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// Ranges of about 8,192 (token, KV head) items, taken last rows first (xcd_item_phased):
// at 64K tokens this takes the forward from 5.8 to 5.1 ms against one range dealt to the
// XCDs in 8,192-token pieces (first rows first: 5.7 ms; ranges of 2,048 items or fewer:
// no gain), the gathers then running mostly within one 8K-row band of the sequence.
static int attn_phases(int64_t items) {
  const int64_t p = (items + 8191) / 8192;
  return (int)(p < 1 ? 1 : p > 64 ? 64 : p);
}

hipError_t launch_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx,
                                  int B, int T, int Hq, int Hkv, int D, int topk, int window,
                                  float scale, bool bf16, void* out, float* lse, int row_begin,
                                  int row_end, hipStream_t st) {
  const int G = Hq / Hkv;
  const float sl2 = scale * kLog2e;
  const int nrows = row_end - row_begin;
  if (nrows <= 0) return hipSuccess;
  // no listed keys: a plain sliding window, whose K/V rows neighbouring tokens share
  if ((!idx || topk == 0) && bf16 && G <= 16 && (D == 64 || D == 128) && window >= 1)
    return launch_window_attn(q, k, v, B, T, Hq, Hkv, D, window, scale, out, lse, row_begin,
                              row_end, st);
  const dim3 grid((unsigned)xcd_grid((int64_t)B * nrows * Hkv));
  const dim3 block(64);
  if (bf16 && G <= 16) {
    // 32-bit row offsets when one KV head's rows of a batch span less than 4 GB
    const bool ofs32 = (int64_t)T * Hkv * D * 2 < (int64_t)UINT32_MAX;
    const int64_t items = (int64_t)B * nrows * Hkv;
    const int phases = attn_phases(items);
    const dim3 pgrid((unsigned)xcd_grid_phased(items, phases));
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, pgrid, block, 0, st, (const uint16_t*)q, (const uint16_t*)k,
                         (const uint16_t*)v, idx, B, T, Hq, Hkv, topk, window, sl2,
                         (uint16_t*)out, lse, row_begin, nrows, phases);
    };
    if (D == 128) ofs32 ? go(sparse_attn_mfma<128, true>) : go(sparse_attn_mfma<128, false>);
    else ofs32 ? go(sparse_attn_mfma<64, true>) : go(sparse_attn_mfma<64, false>);
  } else if (bf16) {
    if (D == 128)
      hipLaunchKernelGGL((sparse_attn_valu<128, true>), grid, block, 0, st, q, k, v, idx, B, T, Hq,
                         Hkv, topk, window, sl2, out, lse, row_begin, nrows);
    else
      hipLaunchKernelGGL((sparse_attn_valu<64, true>), grid, block, 0, st, q, k, v, idx, B, T, Hq,
                         Hkv, topk, window, sl2, out, lse, row_begin, nrows);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((sparse_attn_valu<128, false>), grid, block, 0, st, q, k, v, idx, B, T,
                         Hq, Hkv, topk, window, sl2, out, lse, row_begin, nrows);
    else
      hipLaunchKernelGGL((sparse_attn_valu<64, false>), grid, block, 0, st, q, k, v, idx, B, T, Hq,
                         Hkv, topk, window, sl2, out, lse, row_begin, nrows);
  }
  return hipGetLastError();
}

}  // namespace sa
