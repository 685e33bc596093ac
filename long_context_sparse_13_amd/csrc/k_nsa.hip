// NSA's compressed and selected branches for prefill, and the gated combine of the three
// branches.
//
// [NSA] Native Sparse Attention page, "Puntos Clave": a hierarchical sparse strategy of
// coarse token compression (global context with fewer tokens), fine-grained selection
// (the most important details, chosen in blocks) and a sliding window (local
// dependencies); "Análisis Profundo": compression and selection combined, one K/V fetch
// shared by the query heads of a GQA group.
//
//  * round_bf16: the float32 block means (sa_block_meanpool of K and of V) rounded once
//    per call to bf16 rows for the MFMA tiles.
//  * band_attn_tile<D, WIN>: the compressed branch (WIN = false) and sliding-window
//    attention without listed keys (WIN = true: the window branch, taken by
//    sa_sparse_attn_fwd when no index list is given).  One workgroup per (batch, 8
//    tokens, KV head), one wavefront per token with GroupAttn's arithmetic over its key
//    rows (compressed keys j < (t+1)/block, or tokens [t - W + 1, t]); the 32-row K/V
//    tiles are loaded once per workgroup into LDS and shared by its 8 tokens.
//  * head_sum + block_scores: score[t, j] = sum_h q[t,h] . kbar[j, g(h)] in float32 for the
//    complete blocks of each row (the queries of each KV group summed first); a workgroup
//    owns 64 rows x 64 blocks with the summed queries and the pooled keys staged in LDS,
//    each wavefront 16 rows on the fp32 MFMA (16x16x4; float32 products and sums, as the
//    vector-ALU form it replaced: 0.56 -> 0.48 ms for the whole 64K selection).
//  * block_topk_expand: one wavefront per row picks the top_blocks blocks (ties to the lower
//    block; every block when fewer are complete), sorts them and writes their tokens as
//    the row's index list for sa_sparse_attn_fwd, the blocks interleaved (token e of the
//    i-th block at e * top_blocks + i; -1 for blocks that do not exist).
//  * nsa_decode_range<D>: decode attention of each sequence's query over one contiguous
//    row range of a bf16 cache: the window of the token cache, or the complete blocks of
//    the pooled cache (the compressed branch); per (sequence, KV head) n_splits workgroups
//    of 8 wavefronts, each taking a share of the range's 32-row tiles, merged by
//    log-sum-exp in LDS; with several splits each publishes its partial with agent-scope
//    stores and the last one (a counter) merges them.  One launch can run both range
//    branches (the compressed one's workgroups, then the window's).  The selected branch
//    of decode is sa_sparse_decode with window 0.
//  * nsa_combine: O = g0 * O_cmp + g1 * O_slc + g2 * O_win, 8 elements per thread.
#include "attn_tile.h"
#include "sa_launch.h"

#include <climits>

namespace sa {

__global__ __launch_bounds__(256) void round_bf16(const float* __restrict__ src,
                                                  uint16_t* __restrict__ dst, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * i);
  st8(dst + 4 * i, u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
}

// One workgroup of 8 wavefronts per (batch, 8 consecutive tokens 8 tg .. 8 tg + 7, KV
// head); wavefront w takes token 8 tg + w.  The K and V rows the 8 tokens attend to are
// streamed in 32-row tiles that the whole workgroup loads once into LDS (the next tile's
// rows in flight in registers while the current one is used), so each row leaves L2
// once per 8 tokens instead of once per token.  Per token the arithmetic is GroupAttn's
// (attn_tile.h): S^T = K . Q^T with the group's heads as the MFMA N dimension, an online
// softmax in the log2 domain, O^T += V^T . P^T with V^T read from LDS.  The keys of token t:
//   WIN = false (NSA's compressed branch): the compressed rows j < (t + 1) / block of the
//     bf16 block means (nkv = T / block rows per batch); token groups longest first;
//   WIN = true (a sliding window, the window branch): the token rows [t - window + 1, t]
//     of the K / V caches (nkv = T).
// Tiles start at multiples of 32 rows, so a token's keys fall into the same tiles
// whichever tokens share its workgroup or row range: a row's result does not depend on
// the range it was computed in.  Tokens outside [r0, r0 + nrows) are skipped.
template <int D, bool WIN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void band_attn_tile(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, int B, int T, int Hq, int Hkv, int nkv, int block,
    int window, int r0, int nrows, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int KS = D / 32, DT = D / 16, CH = D * 2 / 16;  // 16-byte chunks per row
  constexpr int LROW = D * 2 + 16;                          // padded LDS row of K (bytes)
  constexpr int VP = 72;  // bytes per V^T row (32 keys of one feature, 8 bytes of pad)
  constexpr int TPG = 8;                                    // tokens per workgroup
  __shared__ __attribute__((aligned(16))) unsigned char kt[32 * LROW];
  __shared__ __attribute__((aligned(16))) unsigned char vt[D * VP];  // V^T [d][key]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int tg0 = r0 / TPG;                             // first token group of the range
  const int ntg = (r0 + nrows + TPG - 1) / TPG - tg0;
  const int64_t items = (int64_t)B * ntg * Hkv;
  if ((int64_t)blockIdx.x >= items) return;
  const int64_t item = items - 1 - (int64_t)blockIdx.x;  // last (longest) token groups first
  const int g = (int)(item % Hkv);
  const int b = (int)((item / Hkv) % B);
  const int tg = tg0 + (int)(item / ((int64_t)Hkv * B));
  const int t = tg * TPG + w;
  const bool tok = t >= r0 && t < r0 + nrows;
  const int G = Hq / Hkv;
  const int h = g * G + n;
  const bool hv = tok && n < G;

  bf16x8 qB[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (hv) x = ld16_nt(q + (((int64_t)b * T + t) * Hq + h) * D + ks * 32 + grp * 8);
    qB[ks] = as_bf16x8(x);
  }
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // key rows [lo_w, hi_w] of this token (empty when hi_w < lo_w) and [lo, hi] of the
  // workgroup's tokens in the range
  const int t_first = max(tg * TPG, r0), t_last = min(tg * TPG + TPG - 1, r0 + nrows - 1);
  int lo_w, hi_w, lo, hi;
  if constexpr (WIN) {
    lo_w = max(0, t - window + 1);
    hi_w = tok ? t : -1;
    lo = max(0, t_first - window + 1);
    hi = t_last;
  } else {
    lo_w = 0;
    hi_w = tok ? (t + 1) / block - 1 : -1;
    lo = 0;
    hi = (t_last + 1) / block - 1;
  }
  const int tbase = lo & ~31;  // tiles start at multiples of 32 rows
  const int ntiles = hi >= lo ? (hi - tbase) / 32 + 1 : 0;
  const int64_t stride = (int64_t)Hkv * D;
  const uint16_t* kbase = kb + ((int64_t)b * nkv * Hkv + g) * D;
  const uint16_t* vbase = vb + ((int64_t)b * nkv * Hkv + g) * D;
  // tile loads: thread tid < 32 * CH takes row tid / CH, 16-byte chunk tid % CH
  const bool ldr = tid < 32 * CH;
  const int r_ld = tid / CH, c_ld = tid % CH;
  u32x4 kr = {0u, 0u, 0u, 0u}, vr = kr;
  auto ldtile = [&](int tile) {
    const int j = tbase + tile * 32 + r_ld;
    kr = u32x4{0u, 0u, 0u, 0u};
    vr = kr;
    if (ldr && j >= lo && j <= hi) {
      kr = ld16(kbase + (int64_t)j * stride + c_ld * 8);
      vr = ld16(vbase + (int64_t)j * stride + c_ld * 8);
    }
  };
  if (ntiles > 0) ldtile(0);

  for (int tile = 0; tile < ntiles; ++tile) {
    if (ldr) {
      st16(kt + r_ld * LROW + c_ld * 16, kr);
      // V transposed: value q of this thread's chunk is feature 8 c + q of key r; the order
      // is rotated by the chunk so that a wavefront's lanes write distinct LDS banks
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int qv = (k + c_ld) & 7;
        const uint32_t w01 = (qv & 2) ? vr[1] : vr[0];
        const uint32_t w23 = (qv & 2) ? vr[3] : vr[2];
        const uint32_t wv = (qv & 4) ? w23 : w01;
        *reinterpret_cast<uint16_t*>(vt + (c_ld * 8 + qv) * VP + r_ld * 2) =
            (uint16_t)((qv & 1) ? (wv >> 16) : (wv & 0xffffu));
      }
    }
    __syncthreads();
    if (tile + 1 < ntiles) ldtile(tile + 1);  // in flight while this tile is used
    // this token's keys in the tile: slots [a, e] (a contiguous run)
    const int base = tbase + tile * 32;
    const int a = max(lo_w - base, 0), e = min(hi_w - base, 31);
    if (a <= e) {
      const uint32_t vm = (e == 31 ? 0xffffffffu : ((1u << (e + 1)) - 1u)) & ~((1u << a) - 1u);
      // ---- S^T = K . Q^T for the two 16-key halves (K rows from LDS)
      f32x4 s[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        s[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kA = ld16(kt + (c2 * 16 + n) * LROW + (ks * 32 + grp * 8) * 2);
          s[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kA), qB[ks], s[c2], 0, 0, 0);
        }
      }
      // ---- online softmax (log2 domain); head n's max over the 4 lane groups
      float x[8];
      float mt = -INFINITY;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = c2 * 16 + grp * 4 + i;
          const float v = ((vm >> slot) & 1u) ? s[c2][i] * scale_log2 : -INFINITY;
          x[c2 * 4 + i] = v;
          mt = fmaxf(mt, v);
        }
      mt = rows4_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2_hw(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = exp2_hw(x[j] - m_new);
        psum += x[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (ballot(alpha != 1.f) != 0ull) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      }
      const u32x4 pw = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                        pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      const bf16x8 pB = as_bf16x8(pw);
      // ---- O^T += V^T . P^T: the lane's reduction slots (grp, j) are keys grp*4 + j and
      // 16 + grp*4 + j - 4, two runs of 4 keys of feature row dt*16 + n of V^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const unsigned char* vrow = vt + (dt * 16 + n) * VP;
        const u32x2 a0 = ld8(vrow + grp * 8);
        const u32x2 a1 = ld8(vrow + 32 + grp * 8);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]}), pB, acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();  // the tile's LDS rows are rewritten next
  }

  const float l = rows4_sum(l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (hv) {
    uint16_t* orow = out + (((int64_t)b * T + t) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 a = acc[dt] * inv;
      st8(orow + dt * 16 + grp * 4, u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
    }
    if (lse && grp == 0)
      lse[((int64_t)b * Hq + h) * T + t] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- block selection
constexpr int kBsRows = 64;    // rows per workgroup
constexpr int kBsBlks = 64;    // blocks per workgroup
constexpr int kBsDim = 128;    // feature slice staged at a time
constexpr int kBsPad = kBsDim + 4;

// qs[b, r, g*D + d] = sum over the query heads h of KV group g of q[b, t, h, d] (float32,
// heads in increasing order), t = row_begin + r; W (4 or 8, dividing D) features per
// thread, read 16 bytes at a time when W = 8 and the input is bf16.
template <bool BF, int W>
__global__ __launch_bounds__(256) void head_sum(const void* __restrict__ q, int T, int Hq,
                                                int Hkv, int D, int row_begin, int row_end,
                                                int B, float* __restrict__ qs) {
  const int E = Hkv * D, G = Hq / Hkv, R = row_end - row_begin;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // W features each
  if (i * W >= (int64_t)B * R * E) return;
  const int64_t f = i * W;
  const int64_t br = f / E;
  const int e = (int)(f % E);
  const int b = (int)(br / R), r = (int)(br % R);
  const int g = e / D, d = e % D;
  const int64_t base = (((int64_t)b * T + row_begin + r) * Hq + g * G) * D + d;
  f32x4 s[W / 4];
#pragma unroll
  for (int u = 0; u < W / 4; ++u) s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int hh = 0; hh < G; ++hh) {
    if constexpr (BF && W == 8) {
      const u32x4 w = ld16(reinterpret_cast<const uint16_t*>(q) + base + (int64_t)hh * D);
      s[0] += f32x4{bf16_to_f32((uint16_t)w[0]), bf16_hi(w[0]), bf16_to_f32((uint16_t)w[1]), bf16_hi(w[1])};
      s[1] += f32x4{bf16_to_f32((uint16_t)w[2]), bf16_hi(w[2]), bf16_to_f32((uint16_t)w[3]), bf16_hi(w[3])};
    } else if constexpr (BF) {
      const u32x2 w = ld8(reinterpret_cast<const uint16_t*>(q) + base + (int64_t)hh * D);
      s[0] += f32x4{bf16_to_f32((uint16_t)w[0]), bf16_hi(w[0]), bf16_to_f32((uint16_t)w[1]), bf16_hi(w[1])};
    } else {
#pragma unroll
      for (int u = 0; u < W / 4; ++u)
        s[u] += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(q) + base +
                                                (int64_t)hh * D + 4 * u);
    }
  }
#pragma unroll
  for (int u = 0; u < W / 4; ++u) *reinterpret_cast<f32x4*>(qs + f + 4 * u) = s[u];
}

// sc[b, r, j] = qs[b, r, :] . kbar[b, j, :] (float32) for rows t = row_begin + r and
// complete blocks j < (t+1)/block; other entries untouched.
__global__ __launch_bounds__(256) void block_scores(const float* __restrict__ qsum,
                                                    const float* __restrict__ kbar, int E,
                                                    int nb, int block, int row_begin,
                                                    int row_end, float* __restrict__ sc,
                                                    int64_t ldsc) {
  __shared__ __attribute__((aligned(16))) float qs[kBsRows][kBsPad];
  __shared__ __attribute__((aligned(16))) float ks[kBsBlks][kBsPad];
  const int tid = threadIdx.x;
  const int R = row_end - row_begin;
  const int r0 = blockIdx.x * kBsRows;
  const int j0 = blockIdx.y * kBsBlks;
  const int b = blockIdx.z;
  const int t_hi = row_begin + min(r0 + kBsRows, R) - 1;
  if (j0 >= (t_hi + 1) / block) return;  // every block of the tile is past every row
  // wavefront w: rows 16 w .. 16 w + 15 of the tile against its 64 blocks, four 16x16
  // tiles on the fp32 MFMA (16x16x4).  Step s of a slice takes dims s, 32 + s, 64 + s,
  // 96 + s (lane group g = lane / 16 supplies dim 32 g + s), so each lane reads its 32
  // dims of a row as eight 16-byte LDS reads.
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int e0 = 0; e0 < E; e0 += kBsDim) {
    for (int i = tid; i < kBsRows * kBsDim / 4; i += 256) {
      const int rr = i / (kBsDim / 4), c = (i % (kBsDim / 4)) * 4;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (r0 + rr < R && e0 + c < E)
        x = *reinterpret_cast<const f32x4*>(qsum + ((int64_t)b * R + r0 + rr) * E + e0 + c);
      *reinterpret_cast<f32x4*>(&qs[rr][c]) = x;
    }
    for (int i = tid; i < kBsBlks * kBsDim / 4; i += 256) {
      const int jj = i / (kBsDim / 4), c = (i % (kBsDim / 4)) * 4;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (j0 + jj < nb && e0 + c < E)
        x = *reinterpret_cast<const f32x4*>(kbar + ((int64_t)b * nb + j0 + jj) * E + e0 + c);
      *reinterpret_cast<f32x4*>(&ks[jj][c]) = x;
    }
    __syncthreads();
    f32x4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = *reinterpret_cast<const f32x4*>(&qs[16 * w + n][32 * g + 4 * u]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 kb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kb[u] = *reinterpret_cast<const f32x4*>(&ks[16 * ct + n][32 * g + 4 * u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][v], kb[u][v], acc[ct], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane (n, g) holds rows 4 g .. 4 g + 3 of column n of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 16 * w + 4 * g + i;
    if (r >= R) continue;
    const int nfull = (row_begin + r + 1) / block;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int j = j0 + 16 * ct + n;
      if (j < nfull) sc[((int64_t)b * R + r) * ldsc + j] = acc[ct][i];
    }
  }
}

// One wavefront per row: the top `nsel` (<= 64) complete blocks by score, ties to the
// lower block (every complete block when there are no more than nsel), ascending, written
// as their tokens to idx[b, t, 0 : nsel*block], -1 padded.  Scores in registers: lane L
// holds blocks L + 64 m, m < PER.
template <int PER>
__global__ __launch_bounds__(256) void block_topk_expand(const float* __restrict__ sc,
                                                         int64_t ldsc, int B, int T,
                                                         int row_begin, int row_end, int block,
                                                         int nsel, int32_t* __restrict__ idx) {
  __shared__ int sorted_s[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int R = row_end - row_begin;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= (int64_t)B * R) return;
  const int b = (int)(item / R), r = (int)(item % R);
  const int t = row_begin + r;
  const int nfull = (t + 1) / block;
  const float* row = sc + ((int64_t)b * R + r) * ldsc;
  int32_t* out = idx + ((int64_t)b * T + t) * ((int64_t)nsel * block);
  const int take = min(nsel, nfull);
  int mine = INT_MAX;  // lane i: the block chosen in round i
  if (take == nfull) {
    mine = lane < nfull ? lane : INT_MAX;
  } else {
    // order keys (-0 as +0); 0, below every float's key, marks a block that does not exist
    // or was already chosen
    uint32_t key[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m)
      key[m] = lane + 64 * m < nfull ? order_key(row[lane + 64 * m]) : 0u;
    for (int i = 0; i < take; ++i) {
      // this lane's largest key, its lowest block among equal keys (blocks ascend with m)
      uint32_t bk = 0u;
      int bj = INT_MAX;
#pragma unroll
      for (int m = 0; m < PER; ++m)
        if (key[m] > bk) {
          bk = key[m];
          bj = lane + 64 * m;
        }
      // the largest key over the wavefront, then the lowest block holding it (DPP scans,
      // no LDS round trips)
      const uint32_t mk = wave_max_u32(bk);
      const int mj = (int)wave_min_u32(bk == mk ? (uint32_t)bj : 0xffffffffu);
      if (lane == i) mine = mj;
      if ((mj & 63) == lane) {  // a chosen block drops out of later rounds
#pragma unroll
        for (int m = 0; m < PER; ++m)
          if (m == (mj >> 6)) key[m] = 0u;
      }
    }
  }
  // ascending: lane i's rank among the chosen blocks, through LDS
  int rank = 0;
  for (int i = 0; i < take; ++i) rank += __builtin_amdgcn_readlane(mine, i) < mine;
  if (lane < take) sorted_s[wv][rank] = mine;
  wave_lds_sync();
  // interleaved: entry e * nsel + i is token e of the i-th block, so each 32-entry tile of
  // the attention takes two rows from each of 16 blocks instead of 32 consecutive rows of
  // one block (the selected branch at 64K: 3.28 -> 2.73 ms)
  if ((nsel & (nsel - 1)) == 0) {  // nsel divides 64: each lane keeps one block i
    const int sh = __builtin_ctz(nsel);
    const int i = lane & (nsel - 1);
    const int blk = i < take ? sorted_s[wv][i] : -1;
    for (int p = lane, e = lane >> sh; p < nsel * block; p += 64, e += 64 >> sh)
      out[p] = blk >= 0 ? blk * block + e : -1;
  } else {
    for (int p = lane; p < nsel * block; p += 64) {
      const int i = p % nsel, e = p / nsel;
      const int blk = i < take ? sorted_s[wv][i] : -1;
      out[p] = blk >= 0 ? blk * block + e : -1;
    }
  }
}

// ---------------------------------------------------------------- decode: one row range
// One workgroup of kRangeWaves wavefronts per (sequence, KV head): the wavefronts take
// consecutive slices of the range (32-row tiles) through GroupAttn, then their partial
// softmax states are merged by log-sum-exp through LDS.  One launch serves one or two
// branches (sides): split workgroups y < s0.n_splits run side 0, the next s1.n_splits
// side 1, so the compressed and the window branch of a decode step can share a launch.
constexpr int kRangeWaves = 8;

struct RangeSide {
  const uint16_t* keys;
  const uint16_t* vals;
  uint16_t* out;
  float* lse;
  float* partials;
  uint32_t* counters;
  int Lrows, kind, n_splits;
};

template <int D>
__global__ __launch_bounds__(64 * kRangeWaves) void nsa_decode_range(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ lens, int Hq, int Hkv,
    int block, int window, float scale_log2, RangeSide s0, RangeSide s1) {
  using GA = GroupAttn<D>;
  const bool second = (int)blockIdx.y >= s0.n_splits;  // uniform
  const uint16_t* __restrict__ keys = second ? s1.keys : s0.keys;
  const uint16_t* __restrict__ vals = second ? s1.vals : s0.vals;
  uint16_t* __restrict__ out = second ? s1.out : s0.out;
  float* __restrict__ lse = second ? s1.lse : s0.lse;
  float* __restrict__ partials = second ? s1.partials : s0.partials;
  uint32_t* __restrict__ counters = second ? s1.counters : s0.counters;
  const int Lrows = second ? s1.Lrows : s0.Lrows;
  const int kind = second ? s1.kind : s0.kind;
  const int n_splits = second ? s1.n_splits : s0.n_splits;
  constexpr int PS = D + 4;  // floats per (split, head) partial: o[D], m, l, 2 pad
  __shared__ __attribute__((aligned(16))) unsigned char vl[kRangeWaves][GA::LDS_BYTES];
  __shared__ int last;
  // once the tiles are done, the staging areas hold each wavefront's unnormalised O per
  // head, then the maxima and sums (so a CU holds two of these workgroups)
  static_assert(kRangeWaves * 16 * (D + 2) * 4 <= kRangeWaves * GA::LDS_BYTES,
                "the merge area must fit the staging areas");
  float(*pacc)[16][D] = reinterpret_cast<float(*)[16][D]>(&vl[0][0]);
  float(*pm)[16] = reinterpret_cast<float(*)[16]>(&vl[0][0] + kRangeWaves * 16 * D * 4);
  float(*pl)[16] = pm + kRangeWaves;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int bg = (int)blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int split = (int)blockIdx.y - (second ? s0.n_splits : 0);
  const int G = Hq / Hkv;
  const int h = g * G + n;
  const bool hv = n < G;
  // lengths outside the cache are clamped to it: [0, Lrows] cache rows for the window
  // branch, [0, Lrows * block] tokens (Lrows complete blocks) for the compressed one
  const int64_t lcap = kind == 0 ? (int64_t)Lrows : (int64_t)Lrows * block;
  const int L = (int)min((int64_t)max(lens[b], 0), lcap);
  const int lo = kind == 0 ? max(0, L - window) : 0;
  const int hi = kind == 0 ? L : L / block;
  // tiles of the range: this split's share, then this wavefront's share of that
  const int ntiles_all = (hi - lo + 31) / 32;
  const int ps = (ntiles_all + n_splits - 1) / n_splits;
  const int sb = min(ntiles_all, split * ps), se = min(ntiles_all, sb + ps);
  const int per = (se - sb + kRangeWaves - 1) / kRangeWaves;
  const int tb = min(se, sb + wv * per), te = min(se, tb + per);

  GA ga;
  ga.init(hv ? q + ((int64_t)b * Hq + h) * D : nullptr, grp);
  const int64_t stride = (int64_t)Hkv * D;
  const uint16_t* kbase = keys + ((int64_t)b * Lrows * Hkv + g) * D;
  const uint16_t* vbase = vals + ((int64_t)b * Lrows * Hkv + g) * D;
  const int slot = lane & 31;
  auto fetch = [&](int tile) -> int { return lo + (tb + tile) * 32 + slot; };
  auto finish = [&](int, int raw, int& key, uint32_t& vm) {
    const bool ok = raw < hi;
    vm = (uint32_t)ballot(ok);
    key = ok ? raw : lo;
  };
  ga.run(te - tb, fetch, finish, kbase, vbase, stride, vl[wv], scale_log2, lane);

  const float lt = ga.total_l();
  __syncthreads();  // every wavefront is done with its staging area
  if (grp == 0) {
    pm[wv][n] = ga.m_run;
    pl[wv][n] = lt;
  }
#pragma unroll
  for (int dt = 0; dt < GA::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) pacc[wv][n][dt * 16 + grp * 4 + i] = ga.acc[dt][i];
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += 64 * kRangeWaves) {
    const int hh = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kRangeWaves; ++w) M = fmaxf(M, pm[w][hh]);
    float lsum = 0.f, o = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kRangeWaves; ++w) {
        if (pm[w][hh] > -INFINITY) {
          const float f = exp2f(pm[w][hh] - M);
          lsum += f * pl[w][hh];
          o += f * pacc[w][hh][d];
        }
      }
    }
    const int64_t oh = (int64_t)b * Hq + g * G + hh;
    if (n_splits == 1) {
      out[oh * D + d] = (uint16_t)f32_to_bf16_bits(lsum > 0.f ? o / lsum : 0.f);
      if (lse && d == 0) lse[oh] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
      continue;
    }
    // this split's partial, with agent-scope stores that go to the memory side
    float* pp = partials + (((int64_t)bg * n_splits + split) * G + hh) * PS;
    __hip_atomic_store(pp + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(pp + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pp + D + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (n_splits == 1) return;

  // ---- the last split of this (sequence, KV head) merges all splits
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&counters[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(n_splits - 1);
  __syncthreads();
  if (!last) return;
  const float* pb = partials + (int64_t)bg * n_splits * G * PS;
  auto ald = [](const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int e = threadIdx.x; e < G * D; e += 64 * kRangeWaves) {
    const int hh = e / D, d = e % D;
    float M = -INFINITY, lsum = 0.f, o = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += 8) {  // 8 splits' loads in flight, online rescale
      float ms[8], ls[8], os[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ms[u] = -INFINITY;
        ls[u] = 0.f;
        os[u] = 0.f;
        if (s0 + u < n_splits) {
          const float* ps2 = pb + ((int64_t)(s0 + u) * G + hh) * PS;
          ms[u] = ald(ps2 + D);
          ls[u] = ald(ps2 + D + 1);
          os[u] = ald(ps2 + d);
        }
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, ms[u]);
      if (Mn > -INFINITY) {
        const float a = exp2f(M - Mn);  // 0 while M is -inf
        lsum *= a;
        o *= a;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float f = exp2f(ms[u] - Mn);  // 0 for empty splits
          lsum += f * ls[u];
          o += f * os[u];
        }
        M = Mn;
      }
    }
    const int64_t oh = (int64_t)b * Hq + g * G + hh;
    out[oh * D + d] = (uint16_t)f32_to_bf16_bits(lsum > 0.f ? o / lsum : 0.f);
    if (lse && d == 0) lse[oh] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
  }
  if (threadIdx.x == 0) __hip_atomic_store(&counters[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t nsa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int n_splits) {
  const size_t G = (size_t)(Hq / Hkv);
  const size_t part = ((size_t)B * Hkv * n_splits * G * (D + 4) * 4 + 255) / 256 * 256;
  return part + ((size_t)B * Hkv * 4 + 255) / 256 * 256;
}

static RangeSide range_side(const void* keys, const void* vals, int B, int Lrows, int Hq,
                            int Hkv, int D, int kind, void* out, float* lse, int n_splits,
                            void* workspace) {
  RangeSide r{(const uint16_t*)keys, (const uint16_t*)vals, (uint16_t*)out, lse, nullptr,
              nullptr, Lrows, kind, n_splits};
  if (n_splits > 1) {
    const size_t G = (size_t)(Hq / Hkv);
    const size_t part = ((size_t)B * Hkv * n_splits * G * (D + 4) * 4 + 255) / 256 * 256;
    r.partials = static_cast<float*>(workspace);
    r.counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + part);
  }
  return r;
}

static hipError_t launch_ranges(const void* q, const int32_t* lens, int B, int Hq, int Hkv,
                                int D, int block, int window, float scale, const RangeSide& s0,
                                const RangeSide& s1, hipStream_t st) {
  const dim3 grid((unsigned)(B * Hkv), (unsigned)(s0.n_splits + s1.n_splits));
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    hipLaunchKernelGGL(nsa_decode_range<128>, grid, dim3(64 * kRangeWaves), 0, st,
                       (const uint16_t*)q, lens, Hq, Hkv, block, window, sl2, s0, s1);
  else
    hipLaunchKernelGGL(nsa_decode_range<64>, grid, dim3(64 * kRangeWaves), 0, st,
                       (const uint16_t*)q, lens, Hq, Hkv, block, window, sl2, s0, s1);
  return hipGetLastError();
}

hipError_t launch_nsa_decode_range(const void* q, const void* keys, const void* vals,
                                   const int32_t* lens, int B, int Lrows, int Hq, int Hkv, int D,
                                   int kind, int block, int window, float scale, void* out,
                                   float* lse, int n_splits, void* workspace, hipStream_t st) {
  const RangeSide s0 = range_side(keys, vals, B, Lrows, Hq, Hkv, D, kind, out, lse, n_splits,
                                  workspace);
  const RangeSide none{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
  return launch_ranges(q, lens, B, Hq, Hkv, D, block, window, scale, s0, none, st);
}

hipError_t launch_nsa_decode_cmp_win(const void* q, const void* kbar16, const void* vbar16,
                                     const void* kcache, const void* vcache, const int32_t* lens,
                                     int B, int Lmax, int Hq, int Hkv, int D, int block,
                                     int window, float scale, void* out_cmp, float* lse_cmp,
                                     void* out_win, float* lse_win, int ns_cmp, int ns_win,
                                     void* workspace, hipStream_t st) {
  const size_t ws_cmp = ns_cmp > 1 ? nsa_decode_workspace_bytes(B, Hq, Hkv, D, ns_cmp) : 0;
  const RangeSide sc = range_side(kbar16, vbar16, B, Lmax / block, Hq, Hkv, D, 1, out_cmp, lse_cmp,
                                  ns_cmp, workspace);
  const RangeSide sw = range_side(kcache, vcache, B, Lmax, Hq, Hkv, D, 0, out_win, lse_win, ns_win,
                                  static_cast<char*>(workspace) + ws_cmp);
  return launch_ranges(q, lens, B, Hq, Hkv, D, block, window, scale, sc, sw, st);
}

__global__ __launch_bounds__(256) void nsa_combine_k(const uint16_t* __restrict__ oc,
                                                     const uint16_t* __restrict__ os,
                                                     const uint16_t* __restrict__ ow,
                                                     const float* __restrict__ gates, int D,
                                                     int64_t n8, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t row = (i * 8) / D;  // (token, head)
  const float g0 = gates[row * 3], g1 = gates[row * 3 + 1], g2 = gates[row * 3 + 2];
  const u32x4 a = ld16(oc + 8 * i), s = ld16(os + 8 * i), w = ld16(ow + 8 * i);
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float lo = g0 * bf16_to_f32((uint16_t)a[c]) + g1 * bf16_to_f32((uint16_t)s[c]) +
                     g2 * bf16_to_f32((uint16_t)w[c]);
    const float hi = g0 * bf16_hi(a[c]) + g1 * bf16_hi(s[c]) + g2 * bf16_hi(w[c]);
    r[c] = pack_bf16x2(lo, hi);
  }
  st16(out + 8 * i, r);
}

// ---------------------------------------------------------------- host side
size_t cmp_attn_workspace_bytes(int B, int T, int Hkv, int D, int block) {
  const int64_t nb = T / block;
  const size_t one = ((size_t)B * nb * Hkv * D * 2 + 255) / 256 * 256;
  return 2 * one + 256;
}

hipError_t launch_cmp_attn(const void* q, const float* kbar, const float* vbar, int B, int T,
                           int Hq, int Hkv, int D, int block, float scale, void* out, float* lse,
                           void* workspace, hipStream_t st) {
  const int nb = T / block;
  const int64_t n = (int64_t)B * nb * Hkv * D;
  const size_t one = ((size_t)n * 2 + 255) / 256 * 256;
  uint16_t* kb = reinterpret_cast<uint16_t*>(workspace);
  uint16_t* vb = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + one);
  if (n > 0) {
    const unsigned g = (unsigned)((n / 4 + 255) / 256);
    hipLaunchKernelGGL(round_bf16, dim3(g), dim3(256), 0, st, kbar, kb, n / 4);
    hipLaunchKernelGGL(round_bf16, dim3(g), dim3(256), 0, st, vbar, vb, n / 4);
  }
  const int64_t items = (int64_t)B * ((T + 7) / 8) * Hkv;
  const dim3 grid((unsigned)items);
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    hipLaunchKernelGGL((band_attn_tile<128, false>), grid, dim3(512), 0, st, (const uint16_t*)q, kb,
                       vb, B, T, Hq, Hkv, nb, block, 0, 0, T, sl2, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((band_attn_tile<64, false>), grid, dim3(512), 0, st, (const uint16_t*)q, kb,
                       vb, B, T, Hq, Hkv, nb, block, 0, 0, T, sl2, (uint16_t*)out, lse);
  return hipGetLastError();
}

hipError_t launch_window_attn(const void* q, const void* k, const void* v, int B, int T, int Hq,
                              int Hkv, int D, int window, float scale, void* out, float* lse,
                              int row_begin, int row_end, hipStream_t st) {
  const int nrows = row_end - row_begin;
  if (nrows <= 0) return hipSuccess;
  const int ntg = (row_end + 7) / 8 - row_begin / 8;
  const dim3 grid((unsigned)((int64_t)B * ntg * Hkv));
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    hipLaunchKernelGGL((band_attn_tile<128, true>), grid, dim3(512), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, B, T, Hq, Hkv, T, 1, window,
                       row_begin, nrows, sl2, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((band_attn_tile<64, true>), grid, dim3(512), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, B, T, Hq, Hkv, T, 1, window,
                       row_begin, nrows, sl2, (uint16_t*)out, lse);
  return hipGetLastError();
}

size_t block_select_workspace_bytes(int B, int T, int Hkv, int D, int block, int row_begin,
                                    int row_end) {
  const int64_t ld = ((int64_t)(T / block) + 3) / 4 * 4;
  const int64_t rows = (int64_t)B * (row_end - row_begin);
  const size_t sc = ((size_t)rows * ld * sizeof(float) + 255) / 256 * 256;
  return sc + (size_t)rows * Hkv * D * sizeof(float) + 256;
}

hipError_t launch_block_select(const void* q, const float* kbar, int B, int T, int Hq, int Hkv,
                               int D, bool bf16, int block, int top_blocks, int row_begin,
                               int row_end, int32_t* idx, void* workspace, hipStream_t st) {
  const int nb = T / block;
  const int64_t ld = ((int64_t)nb + 3) / 4 * 4;
  const int R = row_end - row_begin;
  const int64_t rows = (int64_t)B * R;
  const int E = Hkv * D;
  float* sc = reinterpret_cast<float*>(workspace);
  float* qs = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       ((size_t)rows * ld * sizeof(float) + 255) / 256 * 256);
  hipError_t e;
  if (nb > 0) {
    const bool w8 = D % 8 == 0;  // 8 features per thread (else 4: D is a multiple of 4)
    const unsigned g0 = (unsigned)((rows * E / (w8 ? 8 : 4) + 255) / 256);
    if (bf16 && w8)
      hipLaunchKernelGGL((head_sum<true, 8>), dim3(g0), dim3(256), 0, st, q, T, Hq, Hkv, D,
                         row_begin, row_end, B, qs);
    else if (bf16)
      hipLaunchKernelGGL((head_sum<true, 4>), dim3(g0), dim3(256), 0, st, q, T, Hq, Hkv, D,
                         row_begin, row_end, B, qs);
    else if (w8)
      hipLaunchKernelGGL((head_sum<false, 8>), dim3(g0), dim3(256), 0, st, q, T, Hq, Hkv, D,
                         row_begin, row_end, B, qs);
    else
      hipLaunchKernelGGL((head_sum<false, 4>), dim3(g0), dim3(256), 0, st, q, T, Hq, Hkv, D,
                         row_begin, row_end, B, qs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 g1((unsigned)((R + kBsRows - 1) / kBsRows), (unsigned)((nb + kBsBlks - 1) / kBsBlks),
                  (unsigned)B);
    hipLaunchKernelGGL(block_scores, g1, dim3(256), 0, st, qs, kbar, E, nb, block, row_begin,
                       row_end, sc, ld);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 g2((unsigned)((rows + 3) / 4));
  const int per = (nb + 63) / 64;
  if (per <= 4)
    hipLaunchKernelGGL(block_topk_expand<4>, g2, dim3(256), 0, st, sc, ld, B, T, row_begin, row_end,
                       block, top_blocks, idx);
  else if (per <= 16)
    hipLaunchKernelGGL(block_topk_expand<16>, g2, dim3(256), 0, st, sc, ld, B, T, row_begin,
                       row_end, block, top_blocks, idx);
  else
    hipLaunchKernelGGL(block_topk_expand<64>, g2, dim3(256), 0, st, sc, ld, B, T, row_begin,
                       row_end, block, top_blocks, idx);
  return hipGetLastError();
}

hipError_t launch_nsa_combine(const void* oc, const void* os, const void* ow, const float* gates,
                              int B, int T, int Hq, int D, void* out, hipStream_t st) {
  const int64_t n8 = (int64_t)B * T * Hq * D / 8;
  hipLaunchKernelGGL(nsa_combine_k, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)oc, (const uint16_t*)os, (const uint16_t*)ow, gates, D, n8,
                     (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace sa
