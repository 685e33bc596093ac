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
//     each workgroup hands on the exact top-16 of its blocks as candidates.
//  2. decode_split_attn: one workgroup of 8 wavefronts per (sequence, KV head, split)
//     selects the top blocks from
//     the candidates; each wavefront attends the group's query heads to its sub-slice of
//     U = selected blocks' tokens before the window followed by the window, through
//     GroupAttn (MFMA over the grouped heads); the workgroup merges its wavefronts in LDS
//     and the last workgroup of each (sequence, KV head) merges the splits.
// The kernel boundary makes the candidates visible to kernel 2.  Inside kernel 2 the
// split partials travel through 16-byte stores and loads with the cache policy of
// agent-scope atomics (sc1) and one counter per (sequence, KV head), avoiding a
// device-wide cache flush per workgroup.  Kernel 1 clears the counters (so the workspace
// needs no initialisation) and kernel 2 returns them to zero at its end.
#include "attn_tile.h"
#include "sa_launch.h"
#include "select.h"

#include <mutex>
#include <type_traits>

namespace sa {

// ------------------------------------------------------------------------ mean-pool
// OUT16: the means are written rounded to bf16 (for MFMA operands) instead of float32.
template <bool BF, bool OUT16>
__global__ __launch_bounds__(256) void block_meanpool_k(const void* __restrict__ kc,
                                                         const int32_t* __restrict__ lens, int B,
                                                         int Lmax, int Hkv, int D, int block,
                                                         void* __restrict__ kbar) {
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
  const int64_t o = (((int64_t)b * nb + j) * Hkv + g) * D + dq * 4;
  if constexpr (OUT16)
    st8(reinterpret_cast<uint16_t*>(kbar) + o,
        u32x2{pack_bf16x2(s0 * inv, s1 * inv), pack_bf16x2(s2 * inv, s3 * inv)});
  else
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(kbar) + o) =
        f32x4{s0 * inv, s1 * inv, s2 * inv, s3 * inv};
}

hipError_t launch_block_meanpool(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv,
                                 int D, int block, bool bf16, void* kbar, bool out16,
                                 hipStream_t st) {
  const int64_t total = (int64_t)B * (Lmax / block) * Hkv * (D / 4);
  const dim3 grid((unsigned)((total + 255) / 256));
  auto go = [&](auto bf, auto o16) {
    hipLaunchKernelGGL((block_meanpool_k<decltype(bf)::value, decltype(o16)::value>), grid,
                       dim3(256), 0, st, kcache, lens, B, Lmax, Hkv, D, block, kbar);
  };
  if (bf16) {
    if (out16) go(std::true_type{}, std::true_type{}); else go(std::true_type{}, std::false_type{});
  } else {
    if (out16) go(std::false_type{}, std::true_type{}); else go(std::false_type{}, std::false_type{});
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------ workspace
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

constexpr int kScoreThreads = 256;
constexpr int kScoreChunk = 256;   // blocks scored per workgroup pass (64 per wavefront)
constexpr int kCandMax = 64;       // most candidates a scoring workgroup hands on
constexpr int kMaxScoreWGs = 64;   // scoring workgroups per (sequence, KV head)
constexpr int kSplitWaves = 8;     // wavefronts per split workgroup (n_splits > 1)
constexpr int kSplitGrain = kSplitWaves * 32;  // positions of U per split: 1 tile per wave
constexpr int kWholeWaves = 8;     // wavefronts of the one workgroup per sequence (n_splits == 1)

// Scoring workgroups per (sequence, KV head) and blocks each one covers.
static void score_grid(int nb, int& nwg, int& per_wg) {
  const int chunks = (int)imax(1, (nb + kScoreChunk - 1) / kScoreChunk);
  nwg = (int)imin(chunks, kMaxScoreWGs);
  per_wg = ((chunks + nwg - 1) / nwg) * kScoreChunk;
}

size_t decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int D, int block, int top_blocks,
                              int n_splits) {
  const size_t bh = (size_t)B * Hkv;
  const size_t G = (size_t)(Hq / Hkv);
  int nwg, per;
  score_grid(Lmax / block, nwg, per);
  return align256(bh * nwg * kCandMax * 8) + align256(bh * n_splits * G * (D + 4) * 4) +
         align256(bh * 4);
}

DecodeWs decode_workspace_carve(void* ws, int B, int Lmax, int Hq, int Hkv, int D, int block,
                                int top_blocks, int n_splits) {
  const size_t bh = (size_t)B * Hkv;
  const size_t G = (size_t)(Hq / Hkv);
  int nwg, per;
  score_grid(Lmax / block, nwg, per);
  char* p = static_cast<char*>(ws);
  DecodeWs w;
  w.cand = reinterpret_cast<uint32_t*>(p);
  p += align256(bh * nwg * kCandMax * 8);
  w.partials = reinterpret_cast<float*>(p);
  p += align256(bh * n_splits * G * (D + 4) * 4);
  w.counters = reinterpret_cast<uint32_t*>(p);
  return w;
}

// Largest |U|: every selected block fully before the window, plus the window.
static int decode_u_max(int Lmax, int block, int top_blocks, int window) {
  const int64_t nb = Lmax / block;
  const int64_t u = imin(top_blocks, nb) * block + imin(window, Lmax);
  return (int)imin(u, Lmax);
}

int decode_auto_splits(int B, int Lmax, int Hkv, int block, int top_blocks, int window) {
  // one 32-key tile per wavefront of an 8-wavefront split, so each wavefront waits for
  // one round of gathers (two tiles per wavefront of 4-wavefront splits: 1 us slower per
  // step; one tile per wavefront of 4-wavefront splits, twice the splits: 4 us slower,
  // the merge costs more than it saves), up to ~8 waves per CU
  const int64_t umax = decode_u_max(Lmax, block, top_blocks, window);
  const int64_t steps = imax(1, (umax + kSplitGrain - 1) / kSplitGrain);
  const int64_t cap = imax(1, (2048 / kSplitWaves) / ((int64_t)B * Hkv));
  return (int)imax(1, imin(imin(steps, cap), 64));
}

// (order key, position) packed so that a larger value is a better entry: larger key, or
// equal key and lower position.  0 marks an empty entry.
__device__ __forceinline__ uint64_t pack_rank(uint32_t key, int pos) {
  return pos < 0 ? 0ull : ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)pos);
}
__device__ __forceinline__ int unpack_pos(uint64_t c) { return (int)(0xffffffffu - (uint32_t)c); }

// Exact top-m of n packed entries in LDS (n a multiple of 8, padded with 0; comb 16-byte
// aligned): an entry's rank is the number of entries better than it; entries with rank < m
// are handed to keep(rank, entry).  All threads read the same LDS words (broadcast), 32
// per batch so that one LDS round trip covers 32 comparisons.
template <int NT, typename Keep>
__device__ __forceinline__ void rank_select(const uint64_t* comb, int n, int m, Keep&& keep) {
  typedef __attribute__((ext_vector_type(2))) unsigned long long u64x2;
  const u64x2* c2 = reinterpret_cast<const u64x2*>(comb);
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint64_t ci = comb[i];
    int rank = 0;
    int j = 0;
    for (; j + 32 <= n; j += 32) {
      u64x2 x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = c2[j / 2 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) rank += (x[u][0] > ci) + (x[u][1] > ci);
    }
    for (; j < n; j += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) rank += comb[j + u] > ci;
    }
    if (ci != 0ull && rank < m) keep(rank, ci);
  }
}

// ------------------------------------------------------------------------ kernel 1
// score_j = (sum of the group's query heads) . kbar_j for this workgroup's blocks; the
// workgroup hands on its own exact top-cpw (cpw = top_blocks rounded up to 8) as packed
// (key, block) candidates.  Any block of the global top is in the top of its own
// workgroup, so the candidates suffice.
template <int D>
__global__ __launch_bounds__(kScoreThreads) void decode_block_scores(
    const uint16_t* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ lens, int Lmax, int Hq, int Hkv, int block, int per_wg, int cpw,
    uint32_t* __restrict__ cand, uint32_t* __restrict__ counters) {
  __shared__ __attribute__((aligned(16))) uint64_t scomb[kScoreChunk];
  // each wavefront's top cpw of the chunk, then the running candidates
  __shared__ __attribute__((aligned(16))) uint64_t wsel[(kScoreThreads / 64 + 1) * kCandMax];
  __shared__ uint64_t best[kCandMax];
  __shared__ __attribute__((aligned(16))) uint16_t qrows[16 * D];  // the group's query rows
  // a row (D floats) is read by 8 lanes, C = D/8 consecutive floats each; 8 rows per
  // group of loads, 8 groups for the wave's 64 rows; rows are reduced with DPP
  constexpr int C = D / 8;
  constexpr int NL = C / 4;         // 16-byte loads per lane per row
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bg = blockIdx.x;        // (sequence, KV head)
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const int nb = Lmax / block;
  const int d0 = (lane & 7) * C;
  const int j_begin = blockIdx.y * per_wg;
  // Issue order: the group's query rows (G x D bf16, one 16-byte piece per thread), the
  // key means of the workgroup's blocks, then the sequence's length.  The means are read
  // through a buffer resource over sequence b's rows of KV head g: rows past the cache
  // read as zero, so no load waits for the length or a branch (rows at or past the
  // sequence's last complete block are read and then left out of the ranking), and the
  // query sum below runs while the means are in flight.
  const int pieces = G * D / 8;
  const int qp = min(tid, pieces - 1);  // threads past the pieces repeat the last one
  const u32x4 qv = ld16(q + ((int64_t)b * Hq + g * G) * D + qp * 8);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(kbar) + ((int64_t)b * nb * Hkv + g) * D, 0,
      (int)(((int64_t)nb * Hkv - g) * D * 4), 0x00020000);
  f32x4 a[8][NL];
  auto load_rows = [&](int c0) {
    const int jw = c0 + wv * 64 + (lane >> 3);  // this lane's row in group 0
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {  // all of the wave's rows in flight at once
      const uint32_t o = ((uint32_t)(jw + gi * 8) * (uint32_t)(Hkv * D) + d0) * 4u;
#pragma unroll
      for (int l = 0; l < NL; ++l)
        a[gi][l] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, o + 16 * l, 0, 0));
    }
  };
  load_rows(j_begin);
  const int L = min(max(lens[b], 0), Lmax);  // lengths outside [0, Lmax] are clamped
  const int nfull = L / block;
  const int j_end = min(j_begin + per_wg, nfull);  // blocks scored
  *reinterpret_cast<u32x4*>(&qrows[qp * 8]) = qv;
  __syncthreads();
  float qb[C];
#pragma unroll
  for (int i = 0; i < C; ++i) qb[i] = 0.f;
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int c = 0; c < C / 8; ++c) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(&qrows[hh * D + d0 + c * 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qb[c * 8 + 2 * i] += bf16_lo(w[i]);
        qb[c * 8 + 2 * i + 1] += bf16_hi(w[i]);
      }
    }
  }
  if (tid < cpw) best[tid] = 0ull;
  for (int c0 = j_begin; c0 < j_end; c0 += kScoreChunk) {
    const int jw = c0 + wv * 64 + (lane >> 3);  // this lane's row in group 0
    if (c0 != j_begin) load_rows(c0);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      float part = 0.f;
#pragma unroll
      for (int l = 0; l < NL; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += a[gi][l][i] * qb[4 * l + i];
      part = sum8_dpp(part);
      const int j = jw + gi * 8;
      if ((lane & 7) == 0)
        scomb[wv * 64 + gi * 8 + (lane >> 3)] = pack_rank(order_key(part), j < j_end ? j : -1);
    }
    // each wavefront keeps the top cpw of its own 64 rows (an entry of the chunk's top cpw
    // has fewer than cpw entries above it in its wavefront too), ranked against its 64
    // entries only; the workgroup then ranks the 4 cpw survivors
    constexpr int NW = kScoreThreads / 64;
    uint64_t* ws = wsel + wv * cpw;
    if (lane < cpw) ws[lane] = 0ull;
    wave_lds_sync();  // this wavefront's scores and cleared slots are in place
    {
      typedef __attribute__((ext_vector_type(2))) unsigned long long u64x2;
      const u64x2* c2 = reinterpret_cast<const u64x2*>(scomb + wv * 64);
      const uint64_t ci = scomb[wv * 64 + lane];
      int rank = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u64x2 x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = c2[h * 16 + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) rank += (x[u][0] > ci) + (x[u][1] > ci);
      }
      if (ci != 0ull && rank < cpw) ws[rank] = ci;
    }
    // from the second chunk on, the running candidates compete with the new scores
    const bool first = c0 == j_begin;
    if (!first && tid < cpw) wsel[NW * cpw + tid] = best[tid];
    __syncthreads();
    rank_select<kScoreThreads>(wsel, NW * cpw + (first ? 0 : cpw), cpw,
                               [&](int rank, uint64_t c) { best[rank] = c; });
    __syncthreads();
  }
  if (tid < cpw)
    reinterpret_cast<uint64_t*>(cand)[((int64_t)bg * gridDim.y + blockIdx.y) * cpw + tid] = best[tid];
  // the merge counter of this (sequence, KV head) starts kernel 2 at zero (same policy as
  // kernel 2's own accesses to it)
  if (blockIdx.y == 0 && tid == 0)
    __hip_atomic_store(&counters[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------ kernel 2
// One workgroup of kSplitWaves wavefronts per (sequence, KV head, split).  It picks the
// top blocks from the scoring candidates (every split does so identically), takes its
// slice of U = selected blocks' tokens before the window followed by the window, gives one
// sub-slice to each wavefront, merges the wavefronts' partial softmaxes in LDS and
// publishes the split's partial.  The last split to finish (a counter) merges all splits
// into the output.  Partials are written and read with the agent-scope (sc1) policy:
// those accesses go straight to the memory side, so no cache flush is needed between
// workgroups.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void decode_split_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ lens, int Lmax, int Hq,
    int Hkv, int block, int top_blocks, int window, int n_splits, int n_cand, float scale_log2,
    const uint32_t* __restrict__ cand, float* __restrict__ partials,
    uint32_t* __restrict__ counters, int32_t* __restrict__ sel_out, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  using GA = GroupAttn<D>;
  constexpr int PS = D + 4;  // floats per (split, head) partial: o[D], m, l, 2 pad
  // per-wave staging area, also used for the wave's merge slot and (all of it) for the
  // candidate list
  constexpr int CAND_BYTES = kMaxScoreWGs * kCandMax * 8 + 64 * 4;
  constexpr int STAGE = GA::LDS_BYTES * W >= CAND_BYTES
                            ? GA::LDS_BYTES
                            : (CAND_BYTES + W - 1) / W;
  static_assert(16 * D * 4 + 2 * 16 * 4 <= STAGE, "merge area must fit the stage");
  __shared__ __attribute__((aligned(16))) unsigned char vl[W][(STAGE + 15) / 16 * 16];
  __shared__ int pre[65];   // token offsets of the selected blocks inside U
  __shared__ int blk[64];   // selected blocks, ascending
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int bg = blockIdx.x;
  const int split = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  const bool hv = n < G;
  // Issue order: this thread's first candidate (n_cand >= 8), the query rows (padding
  // heads read the group's last row and zero it), then the sequence's length, which is
  // needed only once the candidates are in LDS; no load waits for another.
  const uint64_t* cb = reinterpret_cast<const uint64_t*>(cand) + (int64_t)bg * n_cand;
  const uint64_t c_first = cb[min(tid, n_cand - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order
  GA ga;
  ga.init_masked(q + ((int64_t)b * Hq + g * G + (hv ? n : G - 1)) * D, hv, grp);
  __builtin_amdgcn_sched_barrier(0);
  const int L = min(max(lens[b], 0), Lmax);
  const int wstart = max(0, L - window);
  const int nfull = L / block;
  const int nsel_blocks = min(top_blocks, nfull);

  // ---- top blocks from the candidates (by score), then ascending by block
  {
    uint64_t* cc = reinterpret_cast<uint64_t*>(&vl[0][0]);
    int* rsel = reinterpret_cast<int*>(cc + n_cand);  // blocks in score order
    cc[min(tid, n_cand - 1)] = c_first;  // (threads past n_cand repeat the last entry)
    for (int i = tid + 64 * W; i < n_cand; i += 64 * W) cc[i] = cb[i];
    __syncthreads();
    rank_select<64 * W>(cc, n_cand, nsel_blocks,
                                  [&](int rank, uint64_t c) { rsel[rank] = unpack_pos(c); });
    __syncthreads();
    if (tid < nsel_blocks) {  // ascending block order
      const int v = rsel[tid];
      int r = 0;
#pragma unroll 8
      for (int j = 0; j < nsel_blocks; ++j) r += rsel[j] < v;
      blk[r] = v;
    }
    __syncthreads();
    if (wv == 0) {
      const int j = lane < nsel_blocks ? blk[lane] : -1;
      const int cnt = j >= 0 ? max(0, min(block, wstart - j * block)) : 0;
      const int x = wave_incl_scan(cnt, 0, [](int a, int b2) { return a + b2; });
      if (lane < top_blocks) pre[lane] = x - cnt;
      if (lane == 63) pre[64] = x;
      if (sel_out && split == 0 && lane < top_blocks)
        sel_out[(int64_t)bg * top_blocks + lane] = j;
    }
    __syncthreads();
  }
  const int nsel = pre[64];
  const int U = nsel + (L - wstart);
  const int per = ((U + n_splits - 1) / n_splits + 32 * W - 1) / (32 * W) * (32 * W);
  const int wper = per / W;
  const int u_lo = min(U, split * per + wv * wper);
  const int u_hi = min(U, u_lo + wper);

  const int64_t stride = (int64_t)Hkv * D;
  const uint16_t* kbase = kc + ((int64_t)b * Lmax * Hkv + g) * D;
  const uint16_t* vbase = vc + ((int64_t)b * Lmax * Hkv + g) * D;

  auto fetch = [&](int i) -> int {  // U position -> token
    const int u = u_lo + i * 32 + (lane & 31);
    if (u >= u_hi) return -1;
    if (u >= nsel) return wstart + (u - nsel);
    int lo = 0, hi = nsel_blocks - 1;  // last selected block with pre[.] <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= u) lo = mid;
      else hi = mid - 1;
    }
    return blk[lo] * block + (u - pre[lo]);
  };
  auto finish = [&](int, int raw, int& key, uint32_t& vm) {
    vm = (uint32_t)ballot(raw >= 0);
    key = raw >= 0 ? raw : 0;
  };
  __syncthreads();  // the candidate area in vl[0] is reused as staging
  ga.run((u_hi - u_lo + 31) / 32, fetch, finish, kbase, vbase, stride, vl[wv], scale_log2, lane);

  // ---- merge the wavefronts' partials in LDS (the staging areas are free now)
  const float lw = ga.total_l();
  __syncthreads();
  {
    float* mo = reinterpret_cast<float*>(vl[wv]);  // [16 heads][D] then m[16], l[16]
    if (hv) {
#pragma unroll
      for (int dt = 0; dt < GA::DT; ++dt)
        *reinterpret_cast<f32x4*>(mo + n * D + dt * 16 + grp * 4) = ga.acc[dt];
      if (grp == 0) {
        mo[16 * D + n] = ga.m_run;
        mo[16 * D + 16 + n] = lw;
      }
    }
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)bg * n_splits + split) * G * PS;
  for (int it = tid; it < G * (D / 8); it += 64 * W) {
    const int hh = it / (D / 8), dd = (it % (D / 8)) * 8;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2)
      M = fmaxf(M, reinterpret_cast<const float*>(vl[w2])[16 * D + hh]);
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < W; ++w2) {
        const float* mo = reinterpret_cast<const float*>(vl[w2]);
        const float f = exp2f(mo[16 * D + hh] - M);
        lt += f * mo[16 * D + 16 + hh];
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(mo + hh * D + dd);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(mo + hh * D + dd + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] += f * x0[i];
          o[4 + i] += f * x1[i];
        }
      }
    }
    if (n_splits == 1) {  // the whole of U was here: write the output
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = out + ((int64_t)b * Hq + g * G + hh) * D + dd;
      st16(orow, u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                       pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)});
      if (lse && dd == 0)
        lse[(int64_t)b * Hq + g * G + hh] = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
      continue;
    }
    // 16-byte stores with the cache policy of agent-scope atomic stores (sc1), so the
    // partial is visible to the other splits' workgroups on any XCD
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(partials + pbase, 0, G * PS * 4, 0x00020000);
    const uint32_t po = (uint32_t)(hh * PS + dd) * 4u;
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])},
        prs, po, 0, kSc1);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])},
        prs, po + 16u, 0, kSc1);
    if (dd == 0)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(M), __float_as_uint(lt)}, prs,
                                           (uint32_t)(hh * PS + D) * 4u, 0, kSc1);
  }

  if (n_splits == 1) return;
  // ---- the last split of this (sequence, KV head) merges all splits
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(&counters[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(n_splits - 1);
  __syncthreads();
  if (!last) return;
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      partials + (int64_t)bg * n_splits * G * PS, 0, n_splits * G * PS * 4, 0x00020000);
  for (int it = tid; it < G * (D / 4); it += 64 * W) {
    const int hh = it / (D / 4), dd = (it % (D / 4)) * 4;
    float M = -INFINITY, lt = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_splits; s0 += 8) {  // 8 splits' loads in flight
      float ms[8], ls[8], os[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ms[u] = -INFINITY;
        ls[u] = 0.f;
        os[u][0] = os[u][1] = os[u][2] = os[u][3] = 0.f;
        if (s0 + u < n_splits) {  // loads with the agent-scope cache policy (sc1)
          const uint32_t ps = (uint32_t)(((s0 + u) * G + hh) * PS) * 4u;
          const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(mrs, ps + D * 4, 0, kSc1);
          const u32x4 ov = __builtin_amdgcn_raw_buffer_load_b128(mrs, ps + dd * 4, 0, kSc1);
          ms[u] = __uint_as_float(ml[0]);
          ls[u] = __uint_as_float(ml[1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) os[u][i] = __uint_as_float(ov[i]);
        }
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, ms[u]);
      if (Mn > -INFINITY) {
        const float a = exp2f(M - Mn);  // 0 while M is -inf
        lt *= a;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= a;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float f = exp2f(ms[u] - Mn);  // 0 for empty splits
          lt += f * ls[u];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] += f * os[u][i];
        }
        M = Mn;
      }
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = out + ((int64_t)b * Hq + g * G + hh) * D + dd;
    st8(orow, u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)});
    if (lse && dd == 0)
      lse[(int64_t)b * Hq + g * G + hh] = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
  }
  if (tid == 0) __hip_atomic_store(&counters[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
static void launch_decode_d(const void* q, const void* kcache, const void* vcache,
                            const float* kbar, const int32_t* lens, int B, int Lmax, int Hq,
                            int Hkv, int block, int top_blocks, int window, int n_splits,
                            float sl2, void* out, float* lse, int32_t* sel_out,
                            const DecodeWs& ws, hipStream_t st) {
  int nwg, per_wg;
  score_grid(Lmax / block, nwg, per_wg);
  const int cpw = (top_blocks + 7) / 8 * 8;
  const dim3 g1((unsigned)(B * Hkv), (unsigned)nwg);
  const dim3 g2((unsigned)(B * Hkv), (unsigned)n_splits);
  hipLaunchKernelGGL(decode_block_scores<D>, g1, dim3(kScoreThreads), 0, st, (const uint16_t*)q,
                     kbar, lens, Lmax, Hq, Hkv, block, per_wg, cpw, ws.cand, ws.counters);
  if (n_splits == 1)
    hipLaunchKernelGGL((decode_split_attn<D, kWholeWaves>), g2, dim3(64 * kWholeWaves), 0, st,
                       (const uint16_t*)q, (const uint16_t*)kcache, (const uint16_t*)vcache, lens,
                       Lmax, Hq, Hkv, block, top_blocks, window, n_splits, nwg * cpw, sl2,
                       ws.cand, ws.partials, ws.counters, sel_out, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((decode_split_attn<D, kSplitWaves>), g2, dim3(64 * kSplitWaves), 0, st,
                       (const uint16_t*)q, (const uint16_t*)kcache, (const uint16_t*)vcache, lens,
                       Lmax, Hq, Hkv, block, top_blocks, window, n_splits, nwg * cpw, sl2,
                       ws.cand, ws.partials, ws.counters, sel_out, (uint16_t*)out, lse);
}

// ------------------------------------------------------------------------ no-alloc scratch
// The workspace of sa_sparse_decode_noalloc: a file-scope device array (one copy per GPU,
// held until the process ends) instead of caller memory.  Its device address is looked
// up once per device with that device current, and that address, never the array's host
// name, is what host code hands to kernels.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_sparse_decode(const void* q, const void* kcache, const void* vcache,
                                const float* kbar, const int32_t* lens, int B, int Lmax, int Hq,
                                int Hkv, int D, int block, int top_blocks, int window,
                                int n_splits, float scale, void* out, float* lse,
                                int32_t* sel_out, const DecodeWs& ws, hipStream_t st) {
  const float sl2 = scale * kLog2e;
  if (D == 128)
    launch_decode_d<128>(q, kcache, vcache, kbar, lens, B, Lmax, Hq, Hkv, block, top_blocks,
                         window, n_splits, sl2, out, lse, sel_out, ws, st);
  else
    launch_decode_d<64>(q, kcache, vcache, kbar, lens, B, Lmax, Hq, Hkv, block, top_blocks,
                        window, n_splits, sl2, out, lse, sel_out, ws, st);
  return hipGetLastError();
}

}  // namespace sa
