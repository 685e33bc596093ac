// The indexer contraction on the 16x16x32 bf16 MFMA, shared by every indexer kernel so
// that all of them produce bit-identical float32 scores.
//
// [IC] IndexCache page, body paragraphs 2-3: score(t, s) = sum_h w[h] * ReLU(qi[t, h, :]
// . ki[s, :]).  M = (token, head) pairs, N = keys, K = the indexer feature dimension.
// The 16 M rows of a tile are 16/H consecutive tokens times their H heads; in the MFMA
// C layout a lane holds four consecutive rows, i.e. all heads of 4/H tokens, so ReLU,
// the head weights and the head sum stay inside the lane.
#pragma once

#include "sa_device.h"

namespace sa {

// Work split of the MFMA indexer kernels: a workgroup of kIdxWaves wavefronts owns a
// strip of kIdxStrip rows; the key range is cut into chunks of kIdxChunk handed
// round-robin to kIdxGroups workgroups per strip.
constexpr int kIdxWaves = 4;
constexpr int kIdxStrip = 32 * kIdxWaves;  // 128 rows per workgroup
constexpr int kIdxChunk = 256;             // keys per chunk
constexpr int kIdxGroups = 64;             // workgroups per row strip

// max(0, x) for a finite float as one integer max on its bits (negative floats, -0.0
// included, are negative integers; the result is +0.0 for them).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Score of one (token, key) pair from the head dot products acc[u*H .. u*H+H-1] held
// by a lane: heads summed in increasing order.
template <int H>
__device__ __forceinline__ float index_score(const f32x4& acc, int u, const float (&w)[H]) {
  float sc = 0.f;
#pragma unroll
  for (int hh = 0; hh < H; ++hh) sc += w[hh] * relu_bits(acc[u * H + hh]);
  return sc;
}

// One wavefront's query side: 32 consecutive tokens (TM M tiles) held as MFMA A
// operands in registers.  A 16-key tile is scored with TM*KS MFMAs into TM independent
// accumulators.  Lane (n = lane % 16, grp = lane / 16) receives the scores of key n of
// the tile for the NSC tokens token(i, grp), i < NSC.
template <int H, int DI>
struct IdxWave {
  static constexpr int KS = DI / 32;     // MFMA steps over the feature dimension
  static constexpr int TPT = 16 / H;     // tokens per 16-row M tile
  static constexpr int ROWS = 32;        // tokens per wavefront
  static constexpr int TM = ROWS / TPT;  // M tiles
  static constexpr int TPL = 4 / H;      // tokens per lane in the C layout
  static constexpr int NSC = TM * TPL;   // scores per lane per key tile
  u32x4 a[TM][KS];
  float w[H];

  __device__ static int token(int i, int grp) { return (i / TPL) * TPT + grp * TPL + i % TPL; }

  // Tokens t0 .. t0+31 of qib ([T, H, DI] of one batch); tokens >= row_end read as 0.
  __device__ void load(const uint16_t* __restrict__ qib, int t0, int row_end,
                       const float* __restrict__ wgt, int n, int grp) {
#pragma unroll
    for (int i = 0; i < H; ++i) w[i] = wgt[i];
#pragma unroll
    for (int m = 0; m < TM; ++m) {
      const int row = m * 16 + n;  // (token, head) row inside the wave
      const int tt = t0 + row / H;
      const bool ok = tt < row_end;
      const uint16_t* p = qib + ((int64_t)(ok ? tt : t0) * H + row % H) * DI + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = ld16(p + ks * 32);
        a[m][ks] = v;
      }
    }
  }

  // Token t in every token slot of M tile 0 (the single-row path of score_single).
  __device__ void load_single(const uint16_t* __restrict__ qib, int t,
                              const float* __restrict__ wgt, int n, int grp) {
#pragma unroll
    for (int i = 0; i < H; ++i) w[i] = wgt[i];
    const uint16_t* p = qib + ((int64_t)t * H + n % H) * DI + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[0][ks] = ld16(p + ks * 32);
  }

  // B operand for this lane: key row s of kib ([T, DI] of one batch).
  __device__ static void load_keys(const uint16_t* __restrict__ kib, int s, int grp,
                                   u32x4 (&bk)[KS]) {
    const uint16_t* kp = kib + (int64_t)s * DI + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bk[ks] = ld16(kp + ks * 32);
  }

  __device__ void scores(const u32x4 (&bk)[KS], float (&sc)[NSC]) const {
    f32x4 acc[TM];
#pragma unroll
    for (int m = 0; m < TM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int m = 0; m < TM; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m][ks]), as_bf16x8(bk[ks]),
                                                         acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int u = 0; u < TPL; ++u) sc[m * TPL + u] = index_score<H>(acc[m], u, w);
  }

  // After load_single: the score of the loaded token against key n of the tile (every
  // lane group gets the same value).  Same MFMA operands and order as scores().
  __device__ float score_single(const u32x4 (&bk)[KS]) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[0][ks]), as_bf16x8(bk[ks]), acc,
                                                    0, 0, 0);
    return index_score<H>(acc, 0, w);
  }
};

}  // namespace sa
