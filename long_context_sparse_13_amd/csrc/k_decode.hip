// Block-selected sparse decode: mean-pooled block keys, top blocks, split-K attention
// and log-sum-exp merge.
//
// [NSA] Native Sparse Attention page, "Puntos Clave": coarse compression of tokens,
// blockwise fine-grained selection and a sliding window; "Análisis Profundo": one
// selection per KV group with a shared KV fetch.  [STAR] Star Attention page, body
// paragraph 3: partial attentions computed separately are combined with a distributed
// softmax — here the split-K partials (m, l, o) merged by their log-sum-exp.
//
// Kernels of one decode step (two launches):
//  1. decode_block_scores: score_j = (sum_h q_h) . kbar_j for every complete block;
//     the last workgroup of each (sequence, KV head) to finish (an atomic counter)
//     selects the top blocks with the workgroup radix select of select.h.
//  2. decode_split_attn: one wavefront per (sequence, KV head, split) attends the
//     group's query heads to its slice of U = selected blocks' tokens before the window
//     followed by the window, through GroupAttn (MFMA over the grouped heads); the last
//     wavefront of each (sequence, KV head) merges the splits.
// The counters return to zero at the end of every call.
#include "attn_tile.h"
#include "sa_launch.h"
#include "select.h"

namespace sa {

// ------------------------------------------------------------------------ mean-pool
template <bool BF>
__global__ __launch_bounds__(256) void block_meanpool_k(const void* __restrict__ kc,
                                                         const int32_t* __restrict__ lens, int B,
                                                         int Lmax, int Hkv, int D, int block,
                                                         float* __restrict__ kbar) {
  const int nb = Lmax / block;
  const int D4 = D / 4;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)B * nb * Hkv * D4;
  if (item >= total) return;
  const int dq = (int)(item % D4);
  const int g = (int)((item / D4) % Hkv);
  const int j = (int)((item / ((int64_t)D4 * Hkv)) % nb);
  const int b = (int)(item / ((int64_t)D4 * Hkv * nb));
  if (j >= min(max(lens[b], 0), Lmax) / block) return;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  const int64_t row0 = ((int64_t)b * Lmax + (int64_t)j * block) * Hkv + g;
  for (int i = 0; i < block; ++i) {
    const int64_t off = (row0 + (int64_t)i * Hkv) * D + dq * 4;
    if constexpr (BF) {
      const u32x2 w = ld8(reinterpret_cast<const uint16_t*>(kc) + off);
      s0 += bf16_lo(w[0]);
      s1 += bf16_hi(w[0]);
      s2 += bf16_lo(w[1]);
      s3 += bf16_hi(w[1]);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(kc) + off);
      s0 += a[0];
      s1 += a[1];
      s2 += a[2];
      s3 += a[3];
    }
  }
  const float inv = 1.f / (float)block;
  *reinterpret_cast<f32x4*>(kbar + (((int64_t)b * nb + j) * Hkv + g) * D + dq * 4) =
      f32x4{s0 * inv, s1 * inv, s2 * inv, s3 * inv};
}

hipError_t launch_block_meanpool(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv,
                                 int D, int block, bool bf16, float* kbar, hipStream_t st) {
  const int64_t total = (int64_t)B * (Lmax / block) * Hkv * (D / 4);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(block_meanpool_k<true>, grid, dim3(256), 0, st, kcache, lens, B, Lmax, Hkv,
                       D, block, kbar);
  else
    hipLaunchKernelGGL(block_meanpool_k<false>, grid, dim3(256), 0, st, kcache, lens, B, Lmax, Hkv,
                       D, block, kbar);
  return hipGetLastError();
}

// ------------------------------------------------------------------------ workspace
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int D, int block, int top_blocks,
                              int n_splits) {
  const size_t bh = (size_t)B * Hkv;
  const size_t nb = (size_t)(Lmax / block);
  const size_t G = (size_t)(Hq / Hkv);
  return align256(bh * nb * 4) + align256(bh * top_blocks * 4) +
         align256(bh * n_splits * G * (D + 4) * 4) + align256(bh * 2 * 4);
}

DecodeWs decode_workspace_carve(void* ws, int B, int Lmax, int Hq, int Hkv, int D, int block,
                                int top_blocks, int n_splits) {
  const size_t bh = (size_t)B * Hkv;
  const size_t nb = (size_t)(Lmax / block);
  const size_t G = (size_t)(Hq / Hkv);
  char* p = static_cast<char*>(ws);
  DecodeWs w;
  w.block_scores = reinterpret_cast<float*>(p);
  p += align256(bh * nb * 4);
  w.sel = reinterpret_cast<int32_t*>(p);
  p += align256(bh * top_blocks * 4);
  w.partials = reinterpret_cast<float*>(p);
  p += align256(bh * n_splits * G * (D + 4) * 4);
  w.counters = reinterpret_cast<uint32_t*>(p);
  return w;
}

// Largest |U|: every selected block fully before the window, plus the window.
static int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

static int decode_u_max(int Lmax, int block, int top_blocks, int window) {
  const int64_t nb = Lmax / block;
  const int64_t u = imin(top_blocks, nb) * block + imin(window, Lmax);
  return (int)imin(u, Lmax);
}

int decode_auto_splits(int B, int Lmax, int Hkv, int block, int top_blocks, int window) {
  const int64_t umax = decode_u_max(Lmax, block, top_blocks, window);
  const int64_t steps = imax(1, (umax + 31) / 32);           // 32-key steps of the whole U
  const int64_t want = (512 + (int64_t)B * Hkv - 1) / ((int64_t)B * Hkv);  // ~2 waves per CU
  return (int)imax(1, imin(imin(want, steps), 64));
}

// ------------------------------------------------------------------------ kernel 1
constexpr int kScoreThreads = 256;
constexpr int kScoreBlocksPerWG = 256;

template <int D>
__global__ __launch_bounds__(kScoreThreads) void decode_block_scores(
    const uint16_t* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ lens, int Lmax, int Hq, int Hkv, int block, int top_blocks,
    float* __restrict__ bscore, int32_t* __restrict__ sel, int32_t* __restrict__ sel_out,
    uint32_t* __restrict__ counters) {
  __shared__ SelectShared<kScoreThreads> sh;
  __shared__ int last;
  constexpr int LPR = D / 4;        // lanes per kbar row (16 bytes each)
  constexpr int RPI = 64 / LPR;     // rows per wave instruction
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bg = blockIdx.x;        // (sequence, KV head)
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int nb = Lmax / block;
  const int L = min(max(lens[b], 0), Lmax);  // lengths outside [0, Lmax] are clamped
  const int nfull = L / block;
  float* sc = bscore + (int64_t)bg * nb;

  // (sum of the group's query heads) for this lane's 4 columns
  const int d0 = (lane % LPR) * 4;
  float qb[4] = {0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < G; ++hh) {
    const u32x2 w = ld8(q + ((int64_t)b * Hq + g * G + hh) * D + d0);
    qb[0] += bf16_lo(w[0]);
    qb[1] += bf16_hi(w[0]);
    qb[2] += bf16_lo(w[1]);
    qb[3] += bf16_hi(w[1]);
  }
  const int j_lo = blockIdx.y * kScoreBlocksPerWG;
  const int j_hi = min(j_lo + kScoreBlocksPerWG, nfull);
  for (int j0 = j_lo + wv * RPI; j0 < j_hi; j0 += 4 * RPI) {
    const int j = j0 + lane / LPR;
    float part = 0.f;
    if (j < j_hi) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(kbar + (((int64_t)b * nb + j) * Hkv + g) * D + d0);
      part = a[0] * qb[0] + a[1] * qb[1] + a[2] * qb[2] + a[3] * qb[3];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
    if (j < j_hi && lane % LPR == 0) sc[j] = part;
  }

  // the last workgroup of this (sequence, KV head) selects
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(&counters[bg], 1u) == gridDim.y - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  int32_t* so = sel + (int64_t)bg * top_blocks;
  int32_t* uo = sel_out ? sel_out + (int64_t)bg * top_blocks : nullptr;
  if (nfull <= top_blocks) {
    for (int i = tid; i < top_blocks; i += kScoreThreads) {
      const int v = i < nfull ? i : -1;
      so[i] = v;
      if (uo) uo[i] = v;
    }
  } else {
    for (int i = tid; i < top_blocks; i += kScoreThreads) so[i] = -1;
    __syncthreads();
    wg_topk<kScoreThreads, 0>(
        nfull, top_blocks, [&](int e) { return order_key(__builtin_nontemporal_load(sc + e)); },
        [&](int pos, int e) {
          so[pos] = e;
          if (uo) uo[pos] = e;
        },
        sh);
  }
  if (tid == 0) counters[bg] = 0u;
}

// ------------------------------------------------------------------------ kernel 2
template <int D>
__global__ __launch_bounds__(64) void decode_split_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ lens, int Lmax, int Hq,
    int Hkv, int block, int top_blocks, int window, int n_splits, float scale_log2,
    const int32_t* __restrict__ sel, float* __restrict__ partials, uint32_t* __restrict__ counters,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  using GA = GroupAttn<D>;
  __shared__ __attribute__((aligned(16))) unsigned char vl[GA::LDS_BYTES];
  __shared__ int pre[65];   // token offsets of the selected blocks inside U
  __shared__ int blk[64];
  __shared__ int last;
  const int lane = threadIdx.x;
  const int n = lane & 15, grp = lane >> 4;
  const int bg = blockIdx.x;
  const int split = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int L = min(max(lens[b], 0), Lmax);
  const int wstart = max(0, L - window);

  // tokens each selected block contributes before the window (blocks ascending)
  {
    int j = -1, cnt = 0;
    if (lane < top_blocks) {
      j = sel[(int64_t)bg * top_blocks + lane];
      if (j >= 0) cnt = max(0, min(block, wstart - j * block));
    }
    int x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane < top_blocks) {
      pre[lane] = x - cnt;
      blk[lane] = j;
    }
    if (lane == 63) pre[64] = x;  // lanes >= top_blocks add 0
  }
  __syncthreads();
  const int nsel = pre[64];
  const int U = nsel + (L - wstart);
  const int per = ((U + n_splits - 1) / n_splits + 31) / 32 * 32;
  const int u_lo = split * per;
  const int u_hi = min(U, u_lo + per);

  const int h = g * G + n;
  const bool hv = n < G;
  GA ga;
  ga.init(hv ? q + ((int64_t)b * Hq + h) * D : nullptr, grp);
  const int64_t stride = (int64_t)Hkv * D;
  const uint16_t* kbase = kc + ((int64_t)b * Lmax * Hkv + g) * D;
  const uint16_t* vbase = vc + ((int64_t)b * Lmax * Hkv + g) * D;

  for (int u0 = u_lo; u0 < u_hi; u0 += 32) {
    const int u = u0 + (lane & 31);
    const bool ok = u < u_hi;
    int key = 0;
    if (ok) {
      if (u < nsel) {
        int i = 0;  // the selected block holding position u
        while (i + 1 < top_blocks && pre[i + 1] <= u) ++i;
        key = blk[i] * block + (u - pre[i]);
      } else {
        key = wstart + (u - nsel);
      }
    }
    const uint32_t vm = (uint32_t)ballot(ok);
    ga.step(kbase, vbase, stride, key, vm, vl, scale_log2, lane);
  }

  // partial (o unnormalised, m in log2 units, l) of this split
  const float l = ga.total_l();
  constexpr int PS = D + 4;  // floats per (split, head) partial: o[D], m, l, 2 pad
  const int64_t pbase = (((int64_t)bg * n_splits + split) * G) * PS;
  if (hv) {
    float* pp = partials + pbase + (int64_t)n * PS;
#pragma unroll
    for (int dt = 0; dt < GA::DT; ++dt)
      *reinterpret_cast<f32x4*>(pp + dt * 16 + grp * 4) = ga.acc[dt];
    if (grp == 0) {
      pp[D] = ga.m_run;
      pp[D + 1] = l;
    }
  }

  // the last split of this (sequence, KV head) merges
  __threadfence();
  __syncthreads();
  if (lane == 0) last = atomicAdd(&counters[bg], 1u) == (uint32_t)(n_splits - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  const float* pb = partials + ((int64_t)bg * n_splits) * G * PS;
  for (int hh = 0; hh < G; ++hh) {
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s)
      M = fmaxf(M, __builtin_nontemporal_load(pb + ((int64_t)s * G + hh) * PS + D));
    float lt = 0.f;
    float o[D / 64];
#pragma unroll
    for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
    if (M > -INFINITY) {
      for (int s = 0; s < n_splits; ++s) {
        const float* ps = pb + ((int64_t)s * G + hh) * PS;
        const float ms = __builtin_nontemporal_load(ps + D);
        const float f = exp2f(ms - M);  // 0 for an empty split (ms = -inf)
        lt += f * __builtin_nontemporal_load(ps + D + 1);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) o[i] += f * __builtin_nontemporal_load(ps + lane + 64 * i);
      }
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = out + ((int64_t)b * Hq + g * G + hh) * D;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) orow[lane + 64 * i] = (uint16_t)f32_to_bf16_bits(o[i] * inv);
    if (lse && lane == 0)
      lse[(int64_t)b * Hq + g * G + hh] = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
  }
  if (lane == 0) counters[bg] = 0u;
}

hipError_t launch_sparse_decode(const void* q, const void* kcache, const void* vcache,
                                const float* kbar, const int32_t* lens, int B, int Lmax, int Hq,
                                int Hkv, int D, int block, int top_blocks, int window,
                                int n_splits, float scale, void* out, float* lse,
                                int32_t* sel_out, const DecodeWs& ws, hipStream_t st) {
  const int nb = Lmax / block;
  const dim3 g1((unsigned)(B * Hkv), (unsigned)imax(1, (nb + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG));
  const dim3 g2((unsigned)(B * Hkv), (unsigned)n_splits);
  const float sl2 = scale * kLog2e;
  if (D == 128) {
    hipLaunchKernelGGL(decode_block_scores<128>, g1, dim3(kScoreThreads), 0, st, (const uint16_t*)q,
                       kbar, lens, Lmax, Hq, Hkv, block, top_blocks, ws.block_scores, ws.sel,
                       sel_out, ws.counters);
    hipLaunchKernelGGL(decode_split_attn<128>, g2, dim3(64), 0, st, (const uint16_t*)q,
                       (const uint16_t*)kcache, (const uint16_t*)vcache, lens, Lmax, Hq, Hkv, block,
                       top_blocks, window, n_splits, sl2, ws.sel, ws.partials,
                       ws.counters + B * Hkv, (uint16_t*)out, lse);
  } else {
    hipLaunchKernelGGL(decode_block_scores<64>, g1, dim3(kScoreThreads), 0, st, (const uint16_t*)q,
                       kbar, lens, Lmax, Hq, Hkv, block, top_blocks, ws.block_scores, ws.sel,
                       sel_out, ws.counters);
    hipLaunchKernelGGL(decode_split_attn<64>, g2, dim3(64), 0, st, (const uint16_t*)q,
                       (const uint16_t*)kcache, (const uint16_t*)vcache, lens, Lmax, Hq, Hkv, block,
                       top_blocks, window, n_splits, sl2, ws.sel, ws.partials,
                       ws.counters + B * Hkv, (uint16_t*)out, lse);
  }
  return hipGetLastError();
}

}  // namespace sa
