// Indexer scores S[t, s] = sum_h w[h] * ReLU(qi[t, h, :] . ki[s, :]) for s <= t.
//
// [IC] IndexCache page, body paragraphs 2-3: the DSA indexer is a light module that
// scores every earlier token for every query; its cost is quadratic in the context.
//
// indexer_mfma<H, DI>: bf16, H indexer heads in {1, 2, 4}, DI % 32 == 0.  The product
// is a dense contraction with M = (token, head) pairs, N = keys and K = DI, so it runs on
// the 16x16x32 bf16 MFMA.  The M rows of a 16-row tile are 16/H consecutive tokens times
// their H heads; in the MFMA C layout a lane holds four consecutive rows, i.e. all the
// heads of one token (H = 4), so ReLU, the head weights and the head sum are lane-local.
// A workgroup of 4 wavefronts owns 128 consecutive rows (32 per wavefront); its
// wavefronts walk the same key range, so the key rows they load are shared in cache.
// Each wavefront computes 32 rows x 64 keys of scores into LDS and writes them back as
// 16-byte-per-lane stores of whole 256-byte row pieces.
// Key ranges are cut into chunks of 256 and handed round-robin to 64 workgroups per
// row strip, which balances the triangular (causal) work.
//
// indexer_valu<BF>: any dtype, H * DI <= 4096; float32 FMAs, one thread per key and 4
// query rows per workgroup.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kIdxRowsPerWave = 32;
constexpr int kIdxWaves = 4;
constexpr int kIdxStrip = kIdxRowsPerWave * kIdxWaves;  // 128 rows per workgroup
constexpr int kIdxChunk = 256;                           // keys per chunk
constexpr int kIdxGroups = 64;                           // workgroups per row strip

template <int H, int DI>
__global__ __launch_bounds__(256) void indexer_mfma(const uint16_t* __restrict__ qi,
                                                     const uint16_t* __restrict__ ki,
                                                     const float* __restrict__ wgt, int T,
                                                     int row_begin, int row_end,
                                                     float* __restrict__ scores, int64_t ld) {
  constexpr int KS = DI / 32;
  constexpr int TPT = 16 / H;                        // tokens per 16-row M tile
  constexpr int TM = kIdxRowsPerWave / TPT;          // M tiles per wavefront
  constexpr int TPL = 4 / H;                         // tokens per lane in the C layout
  constexpr int SB = 64;                             // keys per staged block
  constexpr int SROW = SB + 4;                       // padded LDS row (floats)
  __shared__ __attribute__((aligned(16))) float stage[kIdxWaves][kIdxRowsPerWave * SROW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int R = row_end - row_begin;
  const int strips = (R + kIdxStrip - 1) / kIdxStrip;
  const int strip = strips - 1 - (int)(blockIdx.x / kIdxGroups);  // longest strips first
  const int group = (int)(blockIdx.x % kIdxGroups);
  const int b = blockIdx.y;
  const int t0 = row_begin + strip * kIdxStrip + wv * kIdxRowsPerWave;  // this wave's rows
  if (t0 >= row_end) return;
  const int t_last = min(t0 + kIdxRowsPerWave, row_end) - 1;
  const int wave_chunks = t_last / kIdxChunk + 1;  // chunks that meet this wave's rows
  float* st = stage[wv];

  float w[H];
#pragma unroll
  for (int i = 0; i < H; ++i) w[i] = wgt[i];

  // A operands: the wave's 32 rows (x H heads), loaded once
  u32x4 a[TM][KS];
#pragma unroll
  for (int m = 0; m < TM; ++m) {
    const int row = m * 16 + n;                      // (token, head) row inside the wave
    const int tt = t0 + row / H;
    const bool ok = tt < row_end;
    const uint16_t* p = qi + (((int64_t)b * T + (ok ? tt : t0)) * H + row % H) * DI + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = ld16(p + ks * 32);
      a[m][ks] = v;
    }
  }
  const uint16_t* kib = ki + (int64_t)b * T * DI;
  float* sb = scores + (int64_t)b * R * ld;

  for (int c = group; c < wave_chunks; c += kIdxGroups) {
    const int s_lo = c * kIdxChunk;
    const int s_hi = min(s_lo + kIdxChunk, t_last + 1);
    for (int s0 = s_lo; s0 < s_hi; s0 += SB) {
      // ---- 32 rows x 64 keys of scores into this wave's LDS stage
#pragma unroll
      for (int nt = 0; nt < SB / 16; ++nt) {
        const int s = min(s0 + nt * 16 + n, T - 1);
        u32x4 bk[KS];
        const uint16_t* kp = kib + (int64_t)s * DI + grp * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bk[ks] = ld16(kp + ks * 32);
#pragma unroll
        for (int m = 0; m < TM; ++m) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m][ks]), as_bf16x8(bk[ks]),
                                                          acc, 0, 0, 0);
#pragma unroll
          for (int u = 0; u < TPL; ++u) {
            float sc = 0.f;
#pragma unroll
            for (int hh = 0; hh < H; ++hh) sc += w[hh] * fmaxf(acc[u * H + hh], 0.f);
            st[(m * TPT + grp * TPL + u) * SROW + nt * 16 + n] = sc;
          }
        }
      }
      wave_lds_sync();
      // ---- 16 B per lane: 4 rows x 64 keys per instruction
      const bool full = s0 + SB - 1 <= t0;  // every key of the block precedes every row
#pragma unroll
      for (int i = 0; i < kIdxRowsPerWave / 4; ++i) {
        const int rr = i * 4 + (lane >> 4);
        const int tt = t0 + rr;
        const int sc0 = s0 + (lane & 15) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + rr * SROW + (lane & 15) * 4);
        float* dst = sb + (int64_t)(tt - row_begin) * ld + sc0;
        if (full && tt < row_end) {
          *reinterpret_cast<f32x4*>(dst) = v;
        } else if (tt < row_end) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (sc0 + j <= tt && sc0 + j < s_hi) dst[j] = v[j];
        }
      }
      wave_lds_sync();
    }
  }
}

template <bool BF>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  if constexpr (BF) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <bool BF>
__global__ __launch_bounds__(256) void indexer_valu(const void* __restrict__ qi,
                                                     const void* __restrict__ ki,
                                                     const float* __restrict__ wgt, int T, int H,
                                                     int DI, int row_begin, int row_end,
                                                     float* __restrict__ scores, int64_t ld) {
  constexpr int RT = 4;
  __shared__ float qs[RT * 4096];
  const int R = row_end - row_begin;
  const int tb = row_begin + blockIdx.x * RT;
  const int s = blockIdx.y * 256 + threadIdx.x;
  const int b = blockIdx.z;
  const int t_hi = min(tb + RT, row_end) - 1;
  if ((int)(blockIdx.y * 256) > t_hi) return;
  const int HD = H * DI;
  for (int e = threadIdx.x; e < RT * HD; e += 256) {
    const int r = e / HD;
    const int tt = min(tb + r, row_end - 1);
    qs[e] = ld_elem<BF>(qi, ((int64_t)b * T + tt) * HD + (e - r * HD));
  }
  __syncthreads();
  if (s > t_hi) return;
  float sc[RT] = {0.f, 0.f, 0.f, 0.f};
  const int64_t kr = ((int64_t)b * T + s) * DI;
  for (int hh = 0; hh < H; ++hh) {
    float acc[RT] = {0.f, 0.f, 0.f, 0.f};
    for (int d = 0; d < DI; ++d) {
      const float kv = ld_elem<BF>(ki, kr + d);
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r] += qs[r * HD + hh * DI + d] * kv;
    }
    const float wh = wgt[hh];
#pragma unroll
    for (int r = 0; r < RT; ++r) sc[r] += wh * fmaxf(acc[r], 0.f);
  }
  float* sb = scores + (int64_t)b * R * ld;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int tt = tb + r;
    if (tt < row_end && s <= tt) sb[(int64_t)(tt - row_begin) * ld + s] = sc[r];
  }
}

hipError_t launch_indexer_scores(const void* qi, const void* ki, const float* w, int B, int T,
                                 int H_I, int D_I, bool bf16, int row_begin, int row_end,
                                 float* scores, int64_t ld, hipStream_t st) {
  const int R = row_end - row_begin;
  if (bf16 && (H_I == 1 || H_I == 2 || H_I == 4) && (D_I == 32 || D_I == 64 || D_I == 128)) {
    const int strips = (R + kIdxStrip - 1) / kIdxStrip;
    const dim3 grid((unsigned)(strips * kIdxGroups), (unsigned)B);
#define SA_IDX(HH, DD)                                                                        \
  hipLaunchKernelGGL((indexer_mfma<HH, DD>), grid, dim3(256), 0, st, (const uint16_t*)qi,     \
                     (const uint16_t*)ki, w, T, row_begin, row_end, scores, ld)
    if (H_I == 4) {
      if (D_I == 32) SA_IDX(4, 32); else if (D_I == 64) SA_IDX(4, 64); else SA_IDX(4, 128);
    } else if (H_I == 2) {
      if (D_I == 32) SA_IDX(2, 32); else if (D_I == 64) SA_IDX(2, 64); else SA_IDX(2, 128);
    } else {
      if (D_I == 32) SA_IDX(1, 32); else if (D_I == 64) SA_IDX(1, 64); else SA_IDX(1, 128);
    }
#undef SA_IDX
  } else {
    const dim3 grid((unsigned)((R + 3) / 4), (unsigned)((row_end + 255) / 256), (unsigned)B);
    if (bf16)
      hipLaunchKernelGGL(indexer_valu<true>, grid, dim3(256), 0, st, qi, ki, w, T, H_I, D_I,
                         row_begin, row_end, scores, ld);
    else
      hipLaunchKernelGGL(indexer_valu<false>, grid, dim3(256), 0, st, qi, ki, w, T, H_I, D_I,
                         row_begin, row_end, scores, ld);
  }
  return hipGetLastError();
}

}  // namespace sa
