// Indexer scores S[t, s] = sum_h w[h] * ReLU(qi[t, h, :] . ki[s, :]) for s <= t.
//
// [IC] IndexCache page, body paragraphs 2-3: the DSA indexer is a light module that
// scores every earlier token for every query; its cost is quadratic in the context.
//
// indexer_mfma<H, DI>: bf16, H indexer heads in {1, 2, 4}, DI in {32, 64, 128}.  The
// contraction runs on the 16x16x32 bf16 MFMA through IdxWave (indexer_tile.h).  A
// workgroup of 4 wavefronts owns 128 consecutive rows (32 per wavefront); its
// wavefronts walk the same key range, whose 64-key blocks are staged once per workgroup
// in LDS.  Each wavefront scores 16-key tiles, stages 32 rows x 64 keys of scores in LDS
// and writes them back as 16-byte-per-lane stores of whole 256-byte row pieces.  Key ranges are cut into chunks of 256 and handed round-robin to
// 64 workgroups per row strip, which balances the triangular (causal) work.
//
// indexer_valu<BF>: any dtype, H * DI <= 4096; float32 FMAs, one thread per key and 4
// query rows per workgroup.
#include "indexer_tile.h"
#include "sa_launch.h"

namespace sa {

// Scores of the key slots j = 0, 1, ... at positions j << sshift (sshift = 0: every key;
// sshift > 0: the strided sample used by the fused selection) into scores[row, j] for the
// slots with j << sshift <= t.  Slots are cut into chunks of `chunk` (a multiple of 64).
// The four wavefronts of a workgroup (128 rows of one strip) walk the same slot blocks,
// so each block of 64 key rows is loaded once per workgroup, with consecutive lanes on
// consecutive 16-byte pieces of a row, into one of two LDS buffers (the next block in
// flight meanwhile); the MFMA B operands are read from there.
template <int H, int DI, bool F8>
__global__ __launch_bounds__(256) void indexer_mfma(const uint8_t* __restrict__ qi,
                                                     const uint8_t* __restrict__ ki,
                                                     const float* __restrict__ wgt, int T,
                                                     int row_begin, int row_end, int sshift,
                                                     int chunk, float* __restrict__ scores,
                                                     int64_t ld) {
  using IW = IdxWave<H, DI, F8>;
  constexpr int SB = 64;        // key slots per staged block (4 tiles)
  constexpr int SROW = SB + 4;  // padded LDS row (floats)
  constexpr int BLK = SB * IW::RB;                   // bytes of one key block
  constexpr int NPT = (BLK / 16 + 255) / 256;        // 16-byte pieces per thread
  __shared__ __attribute__((aligned(16))) float stage[kIdxWaves][IW::ROWS * SROW];
  __shared__ __attribute__((aligned(16))) unsigned char keys_s[2][BLK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int R = row_end - row_begin;
  const int strips = (R + kIdxStrip - 1) / kIdxStrip;
  const int strip = strips - 1 - (int)(blockIdx.x / kIdxGroups);  // longest strips first
  const int group = (int)(blockIdx.x % kIdxGroups);
  const int b = blockIdx.y;
  const int ts = row_begin + strip * kIdxStrip;           // first row of the strip
  const int t_last_wg = min(ts + kIdxStrip, row_end) - 1;
  const int j_last_wg = t_last_wg >> sshift;              // last slot any row reads
  const int wg_chunks = j_last_wg / chunk + 1;
  if (group >= wg_chunks) return;                         // (uniform over the workgroup)
  const int t0 = ts + wv * IW::ROWS;                       // this wave's rows
  const bool wave_ok = __builtin_amdgcn_readfirstlane((int)(t0 < row_end)) != 0;
  const int t_last = min(t0 + IW::ROWS, row_end) - 1;
  const int j_last = t_last >> sshift;
  float* st = stage[wv];

  IW iw;
  if (wave_ok) iw.load(qi + (int64_t)b * T * H * DI * IW::EB, t0, row_end, wgt, n, grp);
  const uint8_t* kib = ki + (int64_t)b * T * DI * IW::EB;
  float* sb = scores + (int64_t)b * R * ld;

  // cooperative block load: piece pi = tid + 256 u is 16 bytes of the key of slot
  // j0 + pi / (RB / 16) (positions past T - 1 repeat the last key; no row keeps them)
  u32x4 pf[NPT];
  auto fetch_block = [&](int j0) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pi = tid + 256 * u;
      if (pi < BLK / 16) {
        const int kk = pi / (IW::RB / 16), pc = pi % (IW::RB / 16);
        const int pos = min((j0 + kk) << sshift, T - 1);
        pf[u] = ld16(kib + (int64_t)pos * IW::RB + pc * 16);
      }
    }
  };
  auto store_block = [&](unsigned char* dst) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pi = tid + 256 * u;
      if (pi < BLK / 16) {
        const int kk = pi / (IW::RB / 16), pc = pi % (IW::RB / 16);
        st16(dst + IW::lds_off(kk, pc * 16), pf[u]);
      }
    }
  };
  auto next_j0 = [&](int c, int j0) -> int {
    if (j0 + SB < min(c * chunk + chunk, j_last_wg + 1)) return j0 + SB;
    return c + kIdxGroups < wg_chunks ? (c + kIdxGroups) * chunk : -1;
  };

  fetch_block(group * chunk);
  store_block(keys_s[0]);
  __syncthreads();
  int buf = 0;
  for (int c = group; c < wg_chunks; c += kIdxGroups) {
    const int j_lo = c * chunk;
    const int j_hi_wg = min(j_lo + chunk, j_last_wg + 1);
    const int j_hi = min(j_lo + chunk, j_last + 1);
    for (int j0 = j_lo; j0 < j_hi_wg; j0 += SB) {
      const int jn = next_j0(c, j0);
      if (jn >= 0) fetch_block(jn);
      const unsigned char* blk = keys_s[buf];
      if (wave_ok && j0 < j_hi) {
        // ---- 32 rows x 64 slots of scores into this wave's LDS stage
#pragma unroll
        for (int nt = 0; nt < SB / 16; ++nt) {
          typename IW::Keys bk;
          IW::lds_keys(blk, nt * 16 + n, grp, bk);
          float sc[IW::NSC];
          iw.scores(bk, sc);
#pragma unroll
          for (int i = 0; i < IW::NSC; ++i) st[IW::token(i, grp) * SROW + nt * 16 + n] = sc[i];
        }
        wave_lds_sync();
        // ---- 16 B per lane: 4 rows x 64 slots per instruction
        const bool full = j0 + SB - 1 <= (t0 >> sshift);  // every slot precedes every row
#pragma unroll
        for (int i = 0; i < IW::ROWS / 4; ++i) {
          const int rr = i * 4 + (lane >> 4);
          const int tt = t0 + rr;
          const int jc = j0 + (lane & 15) * 4;
          const f32x4 v = *reinterpret_cast<const f32x4*>(st + rr * SROW + (lane & 15) * 4);
          float* dst = sb + (int64_t)(tt - row_begin) * ld + jc;
          if (full && tt < row_end) {
            *reinterpret_cast<f32x4*>(dst) = v;
          } else if (tt < row_end) {
            const int lim = tt >> sshift;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              if (jc + jj <= lim && jc + jj < j_hi) dst[jj] = v[jj];
          }
        }
        wave_lds_sync();
      }
      if (jn >= 0) store_block(keys_s[buf ^ 1]);
      __syncthreads();  // the next block is staged; this one may be overwritten next
      buf ^= 1;
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

hipError_t launch_indexer_mfma(const void* qi, const void* ki, const float* w, int B, int T,
                               int H_I, int D_I, bool f8, int row_begin, int row_end, int sshift,
                               int chunk, float* scores, int64_t ld, hipStream_t st) {
  const int R = row_end - row_begin;
  const int strips = (R + kIdxStrip - 1) / kIdxStrip;
  const dim3 grid((unsigned)(strips * kIdxGroups), (unsigned)B);
  return dispatch_indexer(H_I, D_I, f8, [&](auto h, auto d, auto f) {
    hipLaunchKernelGGL((indexer_mfma<decltype(h)::value, decltype(d)::value, decltype(f)::value>),
                       grid, dim3(256), 0, st, (const uint8_t*)qi, (const uint8_t*)ki, w, T,
                       row_begin, row_end, sshift, chunk, scores, ld);
    return hipGetLastError();
  });
}

bool indexer_has_mfma(int elem, int H_I, int D_I) {
  return (elem == kBF16 || elem == kE4M3) && (H_I == 1 || H_I == 2 || H_I == 4) &&
         (D_I == 32 || D_I == 64 || D_I == 128);
}

hipError_t launch_indexer_scores(const void* qi, const void* ki, const float* w, int B, int T,
                                 int H_I, int D_I, int elem, int row_begin, int row_end,
                                 float* scores, int64_t ld, hipStream_t st) {
  const int R = row_end - row_begin;
  if (indexer_has_mfma(elem, H_I, D_I)) {
    return launch_indexer_mfma(qi, ki, w, B, T, H_I, D_I, elem == kE4M3, row_begin, row_end, 0,
                               kIdxChunk, scores, ld, st);
  } else {
    const dim3 grid((unsigned)((R + 3) / 4), (unsigned)((row_end + 255) / 256), (unsigned)B);
    if (elem == kBF16)
      hipLaunchKernelGGL(indexer_valu<true>, grid, dim3(256), 0, st, qi, ki, w, T, H_I, D_I,
                         row_begin, row_end, scores, ld);
    else
      hipLaunchKernelGGL(indexer_valu<false>, grid, dim3(256), 0, st, qi, ki, w, T, H_I, D_I,
                         row_begin, row_end, scores, ld);
  }
  return hipGetLastError();
}

}  // namespace sa
