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

#include <type_traits>

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

// Eight E4M3 codes (two dwords, lowest byte first) widened to eight bf16 values in MFMA
// operand order.  The widening is exact: every E4M3 value is a bf16 value.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t d0, uint32_t d1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
  return r;
}

// One wavefront's query side: 32 consecutive tokens (TM M tiles) held as bf16 MFMA A
// operands in registers.  A 16-key tile is scored with TM*KS MFMAs into TM independent
// accumulators.  Lane (n = lane % 16, grp = lane / 16) receives the scores of key n of
// the tile for the NSC tokens token(i, grp), i < NSC.
//
// F8: qi and ki hold E4M3 codes (one byte per element).  Key tiles stay as codes in
// registers (half the bytes of bf16) and are widened to bf16 right before their MFMAs;
// the queries are widened once, when loaded.  The MFMA k index of (lane group grp, step
// ks, element j) is feature dim grp*8 + ks*32 + j for bf16, and for E4M3
// (ks/2)*64 + grp*16 + (ks%2)*8 + j, so that a lane's bytes of a key are contiguous
// (one 16-byte load per two steps).  A and B use the same map, so the dot products are
// unchanged.
template <int H, int DI, bool F8 = false>
struct IdxWave {
  static constexpr int KS = DI / 32;     // MFMA steps over the feature dimension
  static constexpr int EB = F8 ? 1 : 2;  // bytes per stored element
  static constexpr int KV = F8 ? (KS + 1) / 2 : KS;  // 16-byte key registers per lane
  static constexpr int TPT = 16 / H;     // tokens per 16-row M tile
  static constexpr int ROWS = 32;        // tokens per wavefront
  static constexpr int TM = ROWS / TPT;  // M tiles
  static constexpr int TPL = 4 / H;      // tokens per lane in the C layout
  static constexpr int NSC = TM * TPL;   // scores per lane per key tile
  struct Keys {
    u32x4 v[KV];
  };
  u32x4 a[TM][KS];
  float w[H];

  __device__ static int token(int i, int grp) { return (i / TPL) * TPT + grp * TPL + i % TPL; }

  // Byte offset, inside one stored row of DI elements, of the data of register c of lane
  // group grp (16 bytes; 8 for E4M3 with KS == 1).
  __device__ static int row_off(int c, int grp) {
    if constexpr (F8) return KS == 1 ? grp * 8 : c * 64 + grp * 16;
    else return (grp * 8 + c * 32) * 2;
  }
  __device__ static u32x4 ld_reg(const uint8_t* p) {
    if constexpr (F8 && KS == 1) {
      const u32x2 v = ld8(p);
      return u32x4{v[0], v[1], 0u, 0u};
    } else {
      return ld16(p);
    }
  }
  // bf16 operand of step ks from the loaded registers r.
  __device__ static u32x4 operand(const u32x4* r, int ks) {
    if constexpr (F8) {
      const u32x4 x = r[ks / 2];
      return (ks % 2) ? e4m3x8_to_bf16x8(x[2], x[3]) : e4m3x8_to_bf16x8(x[0], x[1]);
    } else {
      return r[ks];
    }
  }

  // Tokens t0 .. t0+31 of qib ([T, H, DI] of one batch); tokens >= row_end read as 0.
  __device__ void load(const void* __restrict__ qib, int t0, int row_end,
                       const float* __restrict__ wgt, int n, int grp) {
#pragma unroll
    for (int i = 0; i < H; ++i) w[i] = wgt[i];
#pragma unroll
    for (int m = 0; m < TM; ++m) {
      const int row = m * 16 + n;  // (token, head) row inside the wave
      const int tt = t0 + row / H;
      const bool ok = tt < row_end;
      const uint8_t* p = reinterpret_cast<const uint8_t*>(qib) +
                         ((int64_t)(ok ? tt : t0) * H + row % H) * DI * EB;
      u32x4 r[KV];
#pragma unroll
      for (int c = 0; c < KV; ++c) r[c] = ok ? ld_reg(p + row_off(c, grp)) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[m][ks] = operand(r, ks);
    }
  }

  // Token t in every token slot of M tile 0 (the single-row path of score_single).
  __device__ void load_single(const void* __restrict__ qib, int t,
                              const float* __restrict__ wgt, int n, int grp) {
#pragma unroll
    for (int i = 0; i < H; ++i) w[i] = wgt[i];
    const uint8_t* p = reinterpret_cast<const uint8_t*>(qib) + ((int64_t)t * H + n % H) * DI * EB;
    u32x4 r[KV];
#pragma unroll
    for (int c = 0; c < KV; ++c) r[c] = ld_reg(p + row_off(c, grp));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[0][ks] = operand(r, ks);
  }

  // B operand registers for this lane: key row s of kib ([T, DI] of one batch).
  __device__ static void load_keys(const void* __restrict__ kib, int s, int grp, Keys& bk) {
    const uint8_t* kp = reinterpret_cast<const uint8_t*>(kib) + (int64_t)s * DI * EB;
#pragma unroll
    for (int c = 0; c < KV; ++c) bk.v[c] = ld_reg(kp + row_off(c, grp));
  }

  // A block of consecutive key rows staged in LDS: row kk at kk * RB bytes, its 16-byte
  // pieces XOR-swizzled by the row (piece p at p ^ (kk & SWM)), so that the row-wise
  // writes of the cooperative load and the 16 rows read by each lane group's B operands
  // land on distinct banks.
  static constexpr int RB = DI * EB;                      // bytes per key row
  static constexpr int SWM = (RB / 16 >= 8 ? 8 : RB / 16) - 1;
  __device__ static int lds_off(int kk, int off) {
    return kk * RB + (((off >> 4) ^ (kk & SWM)) << 4) + (off & 15);
  }
  // B operand registers for this lane from row kk of a staged block.
  __device__ static void lds_keys(const unsigned char* blk, int kk, int grp, Keys& bk) {
#pragma unroll
    for (int c = 0; c < KV; ++c) bk.v[c] = ld_reg(blk + lds_off(kk, row_off(c, grp)));
  }

  __device__ void scores(const Keys& bk, float (&sc)[NSC]) const {
    f32x4 acc[TM];
#pragma unroll
    for (int m = 0; m < TM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 b = operand(bk.v, ks);
#pragma unroll
      for (int m = 0; m < TM; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m][ks]), as_bf16x8(b),
                                                         acc[m], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int u = 0; u < TPL; ++u) sc[m * TPL + u] = index_score<H>(acc[m], u, w);
  }

  // After load_single: the score of the loaded token against key n of the tile (every
  // lane group gets the same value).  Same MFMA operands and order as scores().
  __device__ float score_single(const Keys& bk) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[0][ks]),
                                                    as_bf16x8(operand(bk.v, ks)), acc, 0, 0, 0);
    return index_score<H>(acc, 0, w);
  }
};

// Host side: calls f(integral_constant H, integral_constant DI, bool_constant F8) for an
// MFMA indexer configuration (H_I in {1, 2, 4}, D_I in {32, 64, 128}; callers check).
template <typename F>
inline hipError_t dispatch_indexer(int H_I, int D_I, bool f8, F&& f) {
  auto by_f8 = [&](auto h, auto d) {
    return f8 ? f(h, d, std::true_type{}) : f(h, d, std::false_type{});
  };
  auto by_d = [&](auto h) {
    if (D_I == 32) return by_f8(h, std::integral_constant<int, 32>{});
    if (D_I == 64) return by_f8(h, std::integral_constant<int, 64>{});
    return by_f8(h, std::integral_constant<int, 128>{});
  };
  if (H_I == 4) return by_d(std::integral_constant<int, 4>{});
  if (H_I == 2) return by_d(std::integral_constant<int, 2>{});
  return by_d(std::integral_constant<int, 1>{});
}

}  // namespace sa
