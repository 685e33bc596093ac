// Gathered causal sparse attention backward: dQ, dK, dV for the forward over
// S_t = listed indices U window (the same key order and masks as the forward).
//
// [NSA] Native Sparse Attention page, "Puntos Clave": the backward pass of sparse attention
// (6x at 64K there) beside the forward; "Análisis Profundo": one K/V fetch per GQA group.
//
// sparse_attn_bwd_mfma<D, PART>: bf16, up to 16 query heads per KV head.  One wavefront
// per (batch, token, KV head), 32 gathered keys per step, the 16 query heads as the MFMA N
// dimension (as in the forward):
//   S^T  = K . Q^T        A = K rows (16 B per lane, also staged in LDS), B = Q
//   dP^T = V . dO^T       A = V rows, B = dO
//   P = exp2(S * scale * log2 e - lse2),  dS = P (dP - delta),  delta = dO . O
//   dQ^T += K^T . dS^T    A = K^T read transposed from LDS, B = dS^T (bf16)
//   dV    = P^T . dO      16x16x16: A = P^T through LDS, B = dO (registers, once per
//   dK    = dS^T . Q      wavefront)
// dQ is written once per (token, head).  A key is selected by many queries, so its dK and
// dV rows are sums over (query, key) pairs.  Two ways to form them:
//  * PART = false (no workspace): float atomics into float32 rows that the launch clears
//    first; each atomic instruction covers 16 consecutive floats of 4 rows.  Float atomics
//    run at a fixed rate (~3.3e11 adds/s on MI355X whatever the locality), so at 64K
//    (139 M pairs, 256 adds each) they take ~95% of the time.
//  * PART = true (workspace): every pair's dK and dV contributions are written as one
//    bf16 row [dK | dV] of the pair-major partial buffer (slot = listed position, or
//    topk + window offset, of the query's row), with plain non-temporal stores: the
//    product's B operand holds d = n*DT + dt in column n of d-tile dt, so a lane owns DT
//    consecutive values of a key row.  Then, per chunk of query rows:
//      bwd_count    LDS histogram of each 32-row block's keys over 64-key buckets, added
//                   to per-bucket totals
//      bwd_totscan  bucket starts (exclusive scan), cursors, totals cleared again
//      bwd_scatter  the same histogram, one global reservation per (block, bucket), then
//                   (key, partial row) entries written in bucket order
//      bwd_reduce   16384 entries per workgroup: each wavefront owns an eighth of a
//                   bucket's keys and sums their rows in registers, then adds them to
//                   dK / dV with float atomics (a few per key and bucket piece)
//    The partial rows are read once: 2 x 4D bytes of traffic per pair in place of 2D
//    float atomics.
#include "attn_tile.h"
#include "sa_launch.h"

#include <algorithm>

namespace sa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void clear_f32(float* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) *reinterpret_cast<f32x4*>(p + 4 * i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Partial-path geometry: keys per bucket, rows per count/scatter block, entries per
// reduce workgroup.
constexpr int kBwdR = 64;
constexpr int kBwdRB = 32;
constexpr int kBwdSlice = 16384;
constexpr int kBwdMaxT = 1 << 20;  // bucket histograms of at most 16384 counters in LDS

template <int D, bool PART>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_bwd_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ o, const float* __restrict__ lse,
    const uint16_t* __restrict__ dout, int B, int T, int Hq, int Hkv, int topk, int window,
    float scale, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    int r0, int nrows, int C, uint16_t* __restrict__ part) {
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int LROW = D * 2 + 16;  // padded LDS row of a staged K row
  __shared__ __attribute__((aligned(16))) unsigned char kl[32 * LROW];
  __shared__ __attribute__((aligned(16))) uint16_t pl[32][16];  // P as [key][head] (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t sl[32][16];  // dS as [key][head]
  // the S / dP B operands (Q and dO rows of the group's heads), parked in LDS between
  // tiles so that the registers hold the next tile's K and V rows instead; each lane
  // reads back only what it wrote
  __shared__ __attribute__((aligned(16))) unsigned char qsl[16 * LROW];
  __shared__ __attribute__((aligned(16))) unsigned char dsl[16 * LROW];

  const int lane = threadIdx.x;
  const int n = lane & 15, grp = lane >> 4;
  const int64_t item = xcd_item(blockIdx.x, (int64_t)B * nrows * Hkv);
  if (item < 0) return;
  const int g = (int)(item % Hkv);
  const int tl = (int)((item / Hkv) % nrows);
  const int t = r0 + tl;
  const int b = (int)(item / ((int64_t)Hkv * nrows));
  const int G = Hq / Hkv;
  const int h = g * G + n;
  const bool hv = n < G;
  const float scale_log2 = scale * 1.4426950408889634f;

  // ---- per (token, head): Q and dO as B operands; delta = dO . O; the log2-domain lse
  const int64_t hrow = ((int64_t)b * T + t) * Hq + h;
  float delta = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 wq = {0u, 0u, 0u, 0u}, wd = wq, wo = wq;
    if (hv) {
      wq = ld16(q + hrow * D + ks * 32 + grp * 8);
      wd = ld16(dout + hrow * D + ks * 32 + grp * 8);
      wo = ld16(o + hrow * D + ks * 32 + grp * 8);
    }
    st16(qsl + n * LROW + (ks * 32 + grp * 8) * 2, wq);
    st16(dsl + n * LROW + (ks * 32 + grp * 8) * 2, wd);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      delta += bf16_lo(wd[c]) * bf16_lo(wo[c]) + bf16_hi(wd[c]) * bf16_hi(wo[c]);
  }
  delta += shfl_xor_f(delta, 16);
  delta += shfl_xor_f(delta, 32);
  const float lse2 = hv ? lse[((int64_t)b * Hq + h) * T + t] * 1.4426950408889634f : 0.f;

  // ---- B operands of the 16x16x16 products: dO and Q, heads grp*4 + j; column n of
  // d-tile dt is d = dt*16 + n (atomics: 16 consecutive floats per row and instruction)
  // or d = n*DT + dt (partial rows: a lane owns DT consecutive values of a key row)
  s16x4 aDO[DT], aQ[DT];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = grp * 4 + j;
    const bool ok = hh < G;
    const int64_t r = (((int64_t)b * T + t) * Hq + g * G + hh) * D;
    if constexpr (PART) {
      uint32_t wd[DT / 2], wq[DT / 2];
      if (ok) {
        if constexpr (DT == 8) {
          const u32x4 a = ld16(dout + r + n * DT), c = ld16(q + r + n * DT);
#pragma unroll
          for (int u = 0; u < 4; ++u) { wd[u] = a[u]; wq[u] = c[u]; }
        } else {
          const u32x2 a = ld8(dout + r + n * DT), c = ld8(q + r + n * DT);
#pragma unroll
          for (int u = 0; u < 2; ++u) { wd[u] = a[u]; wq[u] = c[u]; }
        }
      } else {
#pragma unroll
        for (int u = 0; u < DT / 2; ++u) { wd[u] = 0u; wq[u] = 0u; }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        aDO[dt][j] = (short)(wd[dt / 2] >> (16 * (dt % 2)));
        aQ[dt][j] = (short)(wq[dt / 2] >> (16 * (dt % 2)));
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        aDO[dt][j] = ok ? (short)dout[r + dt * 16 + n] : (short)0;
        aQ[dt][j] = ok ? (short)q[r + dt * 16 + n] : (short)0;
      }
    }
  }

  f32x4 acc[DT];  // dQ^T: lane holds d = dt*16 + grp*4 + i of head n
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t stride = (int64_t)Hkv * D;
  const uint16_t* kbase = k + ((int64_t)b * T * Hkv + g) * D;
  const uint16_t* vbase = v + ((int64_t)b * T * Hkv + g) * D;
  float* dkbase = dk + ((int64_t)b * T * Hkv + g) * D;
  float* dvbase = dv + ((int64_t)b * T * Hkv + g) * D;
  const int32_t* irow = idx ? idx + ((int64_t)b * T + t) * topk : nullptr;
  // partial rows of this (token, KV head): [slot][dK (D) | dV (D)] bf16
  const int slots = topk + window;
  uint16_t* prow = PART ? part + ((((int64_t)b * Hkv + g) * C + tl) * slots) * (4 * D / 2) : nullptr;
  const int n_idx = (topk + 31) / 32;
  const int n_win = (window + 31) / 32;
  const int slot = lane & 31;
  const int last_listed = t - window;
  const int wlo = t - window + 1;

  // The tiles' keys, as in the forward: listed positions outside [0, t - window] and window
  // positions outside [0, t] are masked out, so each key counts once; tiles with no key
  // are skipped.  next_tile() advances a cursor to the next non-empty tile (the listed
  // positions one tile ahead are always in flight), and its K and V rows are requested
  // while the current tile is still being worked on.
  auto listed = [&](int tile) {
    const int e = tile * 32 + slot;
    return (tile < n_idx && e < topk) ? irow[e] : -1;
  };
  const int ntiles = n_idx + n_win;
  int cursor = 0;
  int raw_next = listed(0);
  auto next_tile = [&](int& tile_out, uint32_t& vm_out, int& key_out) {
    while (cursor < ntiles) {
      const int tile = cursor++;
      int raw;
      bool ok;
      if (tile < n_idx) {
        raw = raw_next;
        raw_next = listed(tile + 1);
        ok = raw >= 0 && raw <= last_listed;
      } else {
        raw = wlo + (tile - n_idx) * 32 + slot;
        ok = raw >= 0 && raw <= t;
      }
      const uint32_t vm_ = (uint32_t)ballot(ok);
      if (vm_ != 0u) {
        tile_out = tile;
        vm_out = vm_;
        key_out = ok ? raw : 0;
        return;
      }
    }
    tile_out = ntiles;
    vm_out = 0u;
    key_out = 0;
  };
  // K and V rows of a tile's two 16-key halves as A operands
  u32x4 kA[2][KS], vA[2][KS];
  auto fetch_kv = [&](uint32_t vm_, int key_) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int sl_ = c2 * 16 + n;
      const int kr = shfl_i(key_, sl_);
      const bool okr = (vm_ >> sl_) & 1u;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 wk = {0u, 0u, 0u, 0u}, wv = wk;
        if (okr) {
          wk = ld16(kbase + (int64_t)kr * stride + ks * 32 + grp * 8);
          wv = ld16(vbase + (int64_t)kr * stride + ks * 32 + grp * 8);
        }
        kA[c2][ks] = wk;
        vA[c2][ks] = wv;
      }
    }
  };

  int tile, key;
  uint32_t vm;
  next_tile(tile, vm, key);
  if (tile < ntiles) fetch_kv(vm, key);
  while (tile < ntiles) {
    f32x4 s[2], dp[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      s[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[c2] = s[c2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qB = as_bf16x8(ld16(qsl + n * LROW + (ks * 32 + grp * 8) * 2));
        const bf16x8 dB = as_bf16x8(ld16(dsl + n * LROW + (ks * 32 + grp * 8) * 2));
        s[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kA[c2][ks]), qB, s[c2], 0, 0, 0);
        dp[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vA[c2][ks]), dB, dp[c2], 0, 0, 0);
      }
      // stage the K rows (key c2*16 + n, features ks*32 + grp*8) for the K^T reads
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st16(kl + (c2 * 16 + n) * LROW + (ks * 32 + grp * 8) * 2, kA[c2][ks]);
    }

    // the next non-empty tile; its K and V rows are in flight from here on
    int tile_n, key_n;
    uint32_t vm_n;
    next_tile(tile_n, vm_n, key_n);
    if (tile_n < ntiles) fetch_kv(vm_n, key_n);

    // P and dS: lane (n, grp) holds keys c2*16 + grp*4 + i of head n
    float pv[8], dsv[8];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sk = c2 * 16 + grp * 4 + i;
        const bool on = hv && ((vm >> sk) & 1u);
        const float p = on ? exp2_hw(s[c2][i] * scale_log2 - lse2) : 0.f;
        pv[c2 * 4 + i] = p;
        dsv[c2 * 4 + i] = p * (dp[c2][i] - delta);
        pl[sk][n] = (uint16_t)f32_to_bf16_bits(p);
        sl[sk][n] = (uint16_t)f32_to_bf16_bits(dsv[c2 * 4 + i]);
      }
    wave_lds_sync();

    // ---- dQ^T += K^T . dS^T (the reduction slot (grp, j) is the key the lane holds)
    const u32x4 dsw = {pack_bf16x2(dsv[0], dsv[1]), pack_bf16x2(dsv[2], dsv[3]),
                       pack_bf16x2(dsv[4], dsv[5]), pack_bf16x2(dsv[6], dsv[7])};
    const unsigned char* krow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (j < 4) ? grp * 4 + j : 16 + grp * 4 + (j - 4);
      krow[j] = kl + r * LROW + n * 2;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint32_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(krow[2 * j] + dt * 32);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(krow[2 * j + 1] + dt * 32);
        a[j] = lo | (hi << 16);
      }
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{a[0], a[1], a[2], a[3]}),
                                                        as_bf16x8(dsw), acc[dt], 0, 0, 0);
    }

    // ---- dV[key, d] = P^T . dO and dK[key, d] = scale dS^T . Q on the 16x16x16 MFMA:
    // A = [key][head] from LDS (lane: key c2*16 + n, heads grp*4 .. +3), B = the dO / Q
    // registers; C: keys c2*16 + grp*4 + i, column n
    const int slot_base = tile < n_idx ? tile * 32 : topk + (tile - n_idx) * 32;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const s16x4 aP = *reinterpret_cast<const s16x4*>(&pl[c2 * 16 + n][grp * 4]);
      const s16x4 aS = *reinterpret_cast<const s16x4*>(&sl[c2 * 16 + n][grp * 4]);
      if constexpr (PART) {
        // dV rows (bf16, d = n*DT .. +DT-1 per lane) at +D, then dK rows at +0
#pragma unroll
        for (int part_k = 0; part_k < 2; ++part_k) {
          f32x4 c[DT];
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            c[dt] = part_k ? __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aS, aQ[dt], z, 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aP, aDO[dt], z, 0, 0, 0);
          const float m = part_k ? scale : 1.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sk = c2 * 16 + grp * 4 + i;
            if ((vm >> sk) & 1u) {
              uint16_t* pr = prow + (int64_t)(slot_base + sk) * (2 * D) + (part_k ? 0 : D) + n * DT;
              if constexpr (DT == 8) {
                const u32x4 wv = {pack_bf16x2(c[0][i] * m, c[1][i] * m), pack_bf16x2(c[2][i] * m, c[3][i] * m),
                                  pack_bf16x2(c[4][i] * m, c[5][i] * m), pack_bf16x2(c[6][i] * m, c[7][i] * m)};
                __builtin_nontemporal_store(wv, reinterpret_cast<u32x4*>(pr));
              } else {
                const u32x2 wv = {pack_bf16x2(c[0][i] * m, c[1][i] * m), pack_bf16x2(c[2][i] * m, c[3][i] * m)};
                __builtin_nontemporal_store(wv, reinterpret_cast<u32x2*>(pr));
              }
            }
          }
        }
      } else {
        int kr[4];
        bool okr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sk = c2 * 16 + grp * 4 + i;
          kr[i] = shfl_i(key, sk);
          okr[i] = (vm >> sk) & 1u;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const f32x4 cv = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aP, aDO[dt], z, 0, 0, 0);
          const f32x4 ck = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aS, aQ[dt], z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (okr[i]) {
              atomicAdd(dvbase + (int64_t)kr[i] * stride + dt * 16 + n, cv[i]);
              atomicAdd(dkbase + (int64_t)kr[i] * stride + dt * 16 + n, ck[i] * scale);
            }
          }
        }
      }
    }
    wave_lds_sync();  // the staging areas are rewritten by the next tile
    tile = tile_n;
    vm = vm_n;
    key = key_n;
  }

  if (hv) {
    float* qr = dq + hrow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(qr + dt * 16 + grp * 4) = acc[dt] * scale;
  }
}

// ---------------------------------------------------------------- partial-path passes
// A (query, key) pair of rows [r0, r0 + nrows): listed position e < topk with key
// idx[b, t, e] in [0, t - window], or window offset w < window with key t - window + 1 + w
// >= 0 (the main kernel's masks).  Its partial row within the chunk is
// w0 = (t - r0) * slots + slot.

template <typename Visit>
__device__ __forceinline__ void for_each_pair(const int32_t* __restrict__ idx, int T, int topk,
                                              int window, int b, int t0, int t1, Visit&& visit) {
  const int slots = topk + window;
  for (int t = t0; t < t1; ++t) {
    const int32_t* irow = idx ? idx + ((int64_t)b * T + t) * topk : nullptr;
    for (int s = threadIdx.x; s < slots; s += blockDim.x) {
      int key;
      bool ok;
      if (s < topk) {
        key = irow[s];
        ok = key >= 0 && key <= t - window;
      } else {
        key = t - window + 1 + (s - topk);
        ok = key >= 0;
      }
      if (ok) visit(t, s, key);
    }
  }
}

__global__ __launch_bounds__(256) void bwd_count(const int32_t* __restrict__ idx, int T, int topk,
                                                 int window, int r0, int nrows, int NR,
                                                 uint32_t* __restrict__ tot) {
  extern __shared__ uint32_t hist[];
  const int b = blockIdx.y;
  const int t0 = r0 + blockIdx.x * kBwdRB, t1 = min(t0 + kBwdRB, r0 + nrows);
  for (int r = threadIdx.x; r < NR; r += blockDim.x) hist[r] = 0u;
  __syncthreads();
  for_each_pair(idx, T, topk, window, b, t0, t1,
                [&](int, int, int key) { atomicAdd(&hist[key / kBwdR], 1u); });
  __syncthreads();
  for (int r = threadIdx.x; r < NR; r += blockDim.x)
    if (hist[r]) atomicAdd(&tot[(int64_t)b * NR + r], hist[r]);
}

// One workgroup: bucket starts = exclusive scan of the totals (B * NR of them), cursor =
// start, totals cleared for the next chunk; start[B * NR] = number of entries.
__global__ __launch_bounds__(1024) void bwd_totscan(uint32_t* __restrict__ tot,
                                                    uint32_t* __restrict__ start,
                                                    uint32_t* __restrict__ cursor, int n) {
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t carry;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0u;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const uint32_t x = i < n ? tot[i] : 0u;
    int wt;
    const uint32_t ex = (uint32_t)wave_excl_sum((int)x, wt);
    if (lane == 0) wsum[w] = (uint32_t)wt;
    __syncthreads();
    uint32_t before = carry;
    for (int u = 0; u < w; ++u) before += wsum[u];
    if (i < n) {
      start[i] = before + ex;
      cursor[i] = before + ex;
      tot[i] = 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t all = 0u;
      for (int u = 0; u < 16; ++u) all += wsum[u];
      carry += all;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) start[n] = carry;
}

__global__ __launch_bounds__(256) void bwd_scatter(const int32_t* __restrict__ idx, int T,
                                                   int topk, int window, int r0, int nrows,
                                                   int NR, uint32_t* __restrict__ cursor,
                                                   u32x2* __restrict__ ent) {
  extern __shared__ uint32_t hist[];
  const int b = blockIdx.y;
  const int slots = topk + window;
  const int t0 = r0 + blockIdx.x * kBwdRB, t1 = min(t0 + kBwdRB, r0 + nrows);
  for (int r = threadIdx.x; r < NR; r += blockDim.x) hist[r] = 0u;
  __syncthreads();
  for_each_pair(idx, T, topk, window, b, t0, t1,
                [&](int, int, int key) { atomicAdd(&hist[key / kBwdR], 1u); });
  __syncthreads();
  // this block's range in each bucket
  for (int r = threadIdx.x; r < NR; r += blockDim.x)
    if (hist[r]) hist[r] = atomicAdd(&cursor[(int64_t)b * NR + r], hist[r]);
  __syncthreads();
  for_each_pair(idx, T, topk, window, b, t0, t1, [&](int t, int s, int key) {
    const uint32_t pos = atomicAdd(&hist[key / kBwdR], 1u);
    ent[pos] = u32x2{(uint32_t)key, (uint32_t)((t - r0) * slots + s)};
  });
}

// Entries [slice * kBwdSlice, +kBwdSlice) for KV head blockIdx.y.  Float atomics in LDS
// run far below the LDS bandwidth, so nothing is shared: wavefront w of the 8 owns the keys
// base + 8s + w (s < 8) of each bucket piece and keeps their [dK | dV] sums in registers
// (lane l: elements l*EPL .. +EPL-1 of each of its 8 key rows, the key picked by a uniform
// switch).  Every wavefront scans the piece's entries (8 B each, cached; the next 256 are
// requested before the current ones are used), keeps its own (about an eighth) and
// gathers their partial rows 16 at a time, then adds its 8 rows to dK / dV with float
// atomics (other workgroups may hold the same keys).
template <int D>
__global__ __launch_bounds__(512) void bwd_reduce(const u32x2* __restrict__ ent,
                                                  const uint32_t* __restrict__ start,
                                                  const uint16_t* __restrict__ part, int T,
                                                  int Hkv, int NR, int C, int slots, int nB,
                                                  float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int EPL = D / 32;  // bf16 elements of a [dK | dV] row per lane
  constexpr int ROW = 2 * D;   // elements per partial row
  constexpr int U = 16;        // gathered rows in flight per wavefront
  constexpr int NW = 8;        // wavefronts; key ownership by (key - base) % NW
  constexpr int NK = kBwdR / NW;  // keys owned per wavefront and bucket
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const uint32_t total = start[nB * NR];
  const uint32_t begin = (uint32_t)blockIdx.x * kBwdSlice;
  if (begin >= total) return;
  const uint32_t end = min(begin + (uint32_t)kBwdSlice, total);

  // first bucket: the last one whose start is <= begin (uniform scalar search)
  int lo = 0, hi = nB * NR - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= begin) lo = mid; else hi = mid - 1;
  }
  const int64_t gstride = (int64_t)Hkv * D;

  for (int bb = lo; bb < nB * NR; ++bb) {
    const uint32_t p0 = max(begin, start[bb]), p1 = min(end, start[bb + 1]);
    if (p0 >= end) break;
    if (p0 >= p1) continue;
    const int b = bb / NR, kbase = (bb % NR) * kBwdR;
    const uint16_t* pbase = part + (((int64_t)b * Hkv + g) * C) * slots * (int64_t)ROW + lane * EPL;
    float r[NK][EPL];
#pragma unroll
    for (int s = 0; s < NK; ++s)
#pragma unroll
      for (int qq = 0; qq < EPL; ++qq) r[s][qq] = 0.f;

    auto fetch = [&](uint32_t e0, u32x2 (&m)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t e = e0 + (uint32_t)(c * 64 + lane);
        m[c] = e < p1 ? ent[e] : u32x2{0xffffffffu, 0u};
      }
    };
    u32x2 cur[4], nxt[4];
    fetch(p0, cur);
    for (uint32_t e0 = p0; e0 < p1; e0 += 256) {
      // this wavefront's entries among the 256 (entries past p1 have key 0xffffffff)
      uint64_t mask[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        mask[c] = ballot(cur[c][0] != 0xffffffffu && (((int)cur[c][0] - kbase) & (NW - 1)) == w);
      fetch(e0 + 256, nxt);
      while (mask[0] | mask[1] | mask[2] | mask[3]) {
        int sl[U];
        uint32_t val[U][EPL / 2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint32_t key = 0xffffffffu, w0 = 0u;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (key == 0xffffffffu && mask[c]) {
              const int j = __builtin_ctzll(mask[c]);
              mask[c] &= mask[c] - 1;
              key = (uint32_t)__builtin_amdgcn_readlane((int)cur[c][0], j);
              w0 = (uint32_t)__builtin_amdgcn_readlane((int)cur[c][1], j);
            }
          }
          sl[u] = key == 0xffffffffu ? -1 : (((int)key - kbase) >> 3);
          if (sl[u] >= 0) {
            const uint16_t* src = pbase + (int64_t)w0 * ROW;
            if constexpr (EPL == 4) {
              const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
              val[u][0] = x[0];
              val[u][1] = x[1];
            } else {
              val[u][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float x[EPL];
#pragma unroll
          for (int qq = 0; qq < EPL; ++qq)
            x[qq] = (qq & 1) ? bf16_hi(val[u][qq / 2]) : bf16_lo(val[u][qq / 2]);
          switch (sl[u]) {
#define SA_BWD_ADD(S) \
  case S:                                                \
    _Pragma("unroll") for (int qq = 0; qq < EPL; ++qq) r[S][qq] += x[qq]; \
    break;
            SA_BWD_ADD(0) SA_BWD_ADD(1) SA_BWD_ADD(2) SA_BWD_ADD(3)
            SA_BWD_ADD(4) SA_BWD_ADD(5) SA_BWD_ADD(6) SA_BWD_ADD(7)
#undef SA_BWD_ADD
            default: break;
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) cur[c] = nxt[c];
    }
    // add the 8 owned rows: lanes below D / EPL hold dK elements, the rest dV
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int key = kbase + s * NW + w;
      if (key < T) {
        const int e = lane * EPL;
        float* dst = (e < D ? dk + e : dv + (e - D)) + ((int64_t)b * T + key) * gstride + (int64_t)g * D;
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq)
          if (r[s][qq] != 0.f) atomicAdd(dst + qq, r[s][qq]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

namespace {
struct BwdWs {
  int slots, NR;
  size_t part, ent, tot, start, cursor, total;
};
size_t al256(size_t x) { return (x + 255) / 256 * 256; }
BwdWs bwd_layout(int B, int T, int Hkv, int D, int topk, int window, int C) {
  BwdWs w;
  w.slots = topk + window;
  w.NR = (T + kBwdR - 1) / kBwdR;
  const size_t nb = (size_t)B * w.NR;
  w.part = 0;
  w.ent = al256((size_t)B * Hkv * C * w.slots * 4 * D);
  w.tot = w.ent + al256((size_t)B * C * w.slots * 8);
  w.start = w.tot + al256(nb * 4);
  w.cursor = w.start + al256((nb + 1) * 4);
  w.total = w.cursor + al256(nb * 4);
  return w;
}
}  // namespace

bool sparse_attn_bwd_partial_ok(int B, int T, int topk, int window) {
  return T <= kBwdMaxT && (int64_t)B * T * (topk + window) < ((int64_t)1 << 31);
}

size_t sparse_attn_bwd_workspace_bytes(int B, int T, int Hkv, int D, int topk, int window,
                                       int rows) {
  const int C = (rows <= 0 || rows > T) ? T : rows;
  return bwd_layout(B, T, Hkv, D, topk, window, C).total;
}

int sparse_attn_bwd_chunk_rows(int B, int T, int Hkv, int D, int topk, int window,
                               size_t ws_bytes) {
  if (sparse_attn_bwd_workspace_bytes(B, T, Hkv, D, topk, window, T) <= ws_bytes) return T;
  int lo = 0, hi = T;  // largest C with bytes(C) <= ws_bytes (bytes grow with C)
  while (lo < hi) {
    const int mid = (int)(((int64_t)lo + hi + 1) / 2);
    if (sparse_attn_bwd_workspace_bytes(B, T, Hkv, D, topk, window, mid) <= ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

hipError_t launch_sparse_attn_bwd(const void* q, const void* k, const void* v, const int32_t* idx,
                                  int B, int T, int Hq, int Hkv, int D, int topk, int window,
                                  float scale, const void* out, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv,
                                  void* workspace, size_t ws_bytes, hipStream_t st) {
  const int64_t n4 = (int64_t)B * T * Hkv * D / 4;
  const dim3 gc((unsigned)((n4 + 255) / 256));
  hipLaunchKernelGGL(clear_f32, gc, dim3(256), 0, st, dk, n4);
  hipLaunchKernelGGL(clear_f32, gc, dim3(256), 0, st, dv, n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint16_t *q16 = (const uint16_t*)q, *k16 = (const uint16_t*)k, *v16 = (const uint16_t*)v,
                 *o16 = (const uint16_t*)out, *d16 = (const uint16_t*)dout;

  if (!workspace) {
    const dim3 grid((unsigned)xcd_grid((int64_t)B * T * Hkv));
    if (D == 128)
      hipLaunchKernelGGL((sparse_attn_bwd_mfma<128, false>), grid, dim3(64), 0, st, q16, k16, v16,
                         idx, o16, lse, d16, B, T, Hq, Hkv, topk, window, scale, dq, dk, dv, 0, T,
                         T, (uint16_t*)nullptr);
    else
      hipLaunchKernelGGL((sparse_attn_bwd_mfma<64, false>), grid, dim3(64), 0, st, q16, k16, v16,
                         idx, o16, lse, d16, B, T, Hq, Hkv, topk, window, scale, dq, dk, dv, 0, T,
                         T, (uint16_t*)nullptr);
    return hipGetLastError();
  }

  const int C = sparse_attn_bwd_chunk_rows(B, T, Hkv, D, topk, window, ws_bytes);
  if (C < 1) return hipErrorInvalidValue;
  const BwdWs L = bwd_layout(B, T, Hkv, D, topk, window, C);
  char* ws = static_cast<char*>(workspace);
  uint16_t* part = reinterpret_cast<uint16_t*>(ws + L.part);
  u32x2* ent = reinterpret_cast<u32x2*>(ws + L.ent);
  uint32_t* tot = reinterpret_cast<uint32_t*>(ws + L.tot);
  uint32_t* start = reinterpret_cast<uint32_t*>(ws + L.start);
  uint32_t* cursor = reinterpret_cast<uint32_t*>(ws + L.cursor);
  const int64_t nb = (int64_t)B * L.NR;
  hipLaunchKernelGGL(fill_u32, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, tot, nb, 0u);
  const size_t hist_bytes = (size_t)L.NR * 4;
  for (int r0 = 0; r0 < T; r0 += C) {
    const int nrows = std::min(C, T - r0);
    const dim3 grid((unsigned)xcd_grid((int64_t)B * nrows * Hkv));
    if (D == 128)
      hipLaunchKernelGGL((sparse_attn_bwd_mfma<128, true>), grid, dim3(64), 0, st, q16, k16, v16,
                         idx, o16, lse, d16, B, T, Hq, Hkv, topk, window, scale, dq, dk, dv, r0,
                         nrows, C, part);
    else
      hipLaunchKernelGGL((sparse_attn_bwd_mfma<64, true>), grid, dim3(64), 0, st, q16, k16, v16,
                         idx, o16, lse, d16, B, T, Hq, Hkv, topk, window, scale, dq, dk, dv, r0,
                         nrows, C, part);
    const dim3 gb((unsigned)((nrows + kBwdRB - 1) / kBwdRB), (unsigned)B);
    hipLaunchKernelGGL(bwd_count, gb, dim3(256), hist_bytes, st, idx, T, topk, window, r0, nrows,
                       L.NR, tot);
    hipLaunchKernelGGL(bwd_totscan, dim3(1), dim3(1024), 0, st, tot, start, cursor, (int)nb);
    hipLaunchKernelGGL(bwd_scatter, gb, dim3(256), hist_bytes, st, idx, T, topk, window, r0,
                       nrows, L.NR, cursor, ent);
    const int64_t max_ent = (int64_t)B * nrows * L.slots;
    const dim3 gr((unsigned)((max_ent + kBwdSlice - 1) / kBwdSlice), (unsigned)Hkv);
    if (D == 128)
      hipLaunchKernelGGL(bwd_reduce<128>, gr, dim3(512), 0, st, ent, start, part, T, Hkv, L.NR, C,
                         L.slots, B, dk, dv);
    else
      hipLaunchKernelGGL(bwd_reduce<64>, gr, dim3(512), 0, st, ent, start, part, T, Hkv, L.NR, C,
                         L.slots, B, dk, dv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sa
