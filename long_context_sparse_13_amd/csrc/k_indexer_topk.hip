// Fused indexer -> top-k: the exact per-row top-k of the indexer scores without writing
// the score matrix.
//
// [IC] IndexCache page, body paragraphs 2-3: the indexer scores every earlier token
// and only a small subset is kept; writing and re-reading all scores (4 bytes per
// (t, s) pair) is what bounds the two-step path, so here the scores stay on chip.
//
// The result is the same as sa_indexer_scores followed by sa_topk_select, bit for bit:
// every kernel below scores through IdxWave (indexer_tile.h), so a (t, s) score is the
// same float32 value wherever it is computed.
//
//  1. sample  (indexer_mfma, sshift > 0): scores of the key slots s = j * 2^sshift.
//  2. sample_threshold: per row, thr = a lower bound of the jrank-th largest sample score
//     (the floor of its 22-bit key prefix).  About k / 2^sshift sampled scores are
//     expected above the row's k-th largest score; jrank adds four standard deviations,
//     so thr is almost always below the k-th largest score.
//  3. indexer_cand: full MFMA scoring of 32 rows x 64 keys per wavefront step, staged in
//     LDS; then, row by row, one ballot over the 64 keys finds the scores >= thr, which
//     go as (score bits, position) to the row's list for the chunk's group: the 256-key
//     chunks c with the same c mod 64 are scored by one wavefront, one after the other,
//     and share a list of at most 256 entries, in position order within each chunk
//     (counts[row, chunk] = the list's length once that chunk is appended).  Nothing else
//     is written.
//  4. cand_topk: one wavefront per row; the chunks' runs of entries, concatenated in
//     position order, are spread over the lanes' registers (up to 4096 entries) and the
//     exact top-k is taken from them: a radix select whose digits cover only the key range
//     actually present (so a few hot bins do not serialise the histogram), then output
//     ranks from two wavefront scans.  Every score >= thr is in the lists, so when they
//     hold at least k entries they hold the k largest.  Rows with more than 4096 entries
//     are selected with streaming passes over the lists instead; rows with fewer than k
//     (thr was above the k-th score) or a list that ran out of room are listed and
//  5. fix_score / fix_rows_k recompute them in full into a slot of their own and select
//     there with passes over global memory: the answer is exact in every case.
#include "indexer_tile.h"
#include "sa_launch.h"
#include "sa_device.h"
#include "topk_common.h"

#include <climits>
#include <type_traits>
#include <utility>

namespace sa {

namespace {

__device__ __forceinline__ float key_to_float(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key ^ 0x80000000u) : ~key;
  return __uint_as_float(u);
}

// Within one wavefront: the bin d (of nb bins in h, top bin first) holding the kk-th
// largest element, kk minus the count above it, and whether that is the bin's whole
// count.  Lane L owns bins [top - per + 1, top], top = nb - 1 - L * per.
__device__ __forceinline__ void wave_find_bin(const uint32_t* h, int nb, int kk, int lane,
                                              int& digit, int& rem, bool& whole) {
  const int per = (nb + 63) / 64;
  const int top = nb - 1 - lane * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (top - i >= 0) local += (int)h[top - i];
  int total;
  const int above0 = wave_excl_sum(local, total);
  const bool mine = above0 < kk && kk <= above0 + local;
  int d = 0, r = 0, wh = 0;
  if (mine) {
    int above = above0;
    for (int i = 0; i < per; ++i) {
      const int c = top - i >= 0 ? (int)h[top - i] : 0;
      if (above + c >= kk) {
        d = top - i;
        r = kk - above;
        wh = r == c;
        break;
      }
      above += c;
    }
  }
  const int src = (int)__builtin_ctzll(ballot(mine));
  digit = __builtin_amdgcn_readlane(d, src);
  rem = __builtin_amdgcn_readlane(r, src);
  whole = __builtin_amdgcn_readlane(wh, src) != 0;
}

__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
}

constexpr int kRadixBins = 1024;

// One wavefront: the kk-th largest key v among the keys its lanes enumerate with
// for_each(f) (keys outside [lo, lo + span] are skipped) and take = how many keys equal
// to v are kept (keys > v are all kept).  Radix digits of up to 10 bits over the
// remaining range (bins hold (key - lo) >> shift); stops early when the digit holding
// the kk-th key is kept whole.  whole: every key equal to v is kept too when take > 0
// (the kept set is then the keys > v - 1; when take == 0 it is the keys > v).
template <typename ForEach>
__device__ __forceinline__ void wave_radix_kth(uint32_t lo, uint32_t span, int kk,
                                               ForEach&& for_each, uint32_t* hist, int lane,
                                               uint32_t& v, int& take, bool& whole) {
  for (;;) {
    const int bits = span == 0u ? 0 : 32 - __builtin_clz(span);
    const int shift = bits > 10 ? bits - 10 : 0;
    const int nb = (int)(span >> shift) + 1;
    for (int i = lane; i < nb; i += 64) hist[i] = 0u;
    wave_lds_sync();
    for_each([&](uint32_t key) {
      const uint32_t d = key - lo;
      if (key >= lo && d <= span) atomicAdd(&hist[d >> shift], 1u);
    });
    wave_lds_sync();
    int dbin, rem;
    bool wh;
    wave_find_bin(hist, nb, kk, lane, dbin, rem, wh);
    const uint32_t bin = (uint32_t)dbin;
    wave_lds_sync();  // hist is rewritten by the next round
    const uint32_t blo = lo + (bin << shift);
    if (shift == 0) {
      v = blo;
      take = rem;
      whole = wh;
      return;
    }
    if (wh) {  // every key of the bin is kept: keep keys >= blo
      v = blo - 1u;
      take = 0;
      whole = true;
      return;
    }
    lo = blo;
    span = (1u << shift) - 1u;
    kk = rem;
  }
}

}  // namespace

// ---------------------------------------------------------------- 2. thresholds
// One wavefront per row; the row's samples go to registers (lane L holds samples
// 4 L + 256 i .. + 3), and thr = the jrank-th largest of them, exactly (the radix
// select of the selection kernel).  thr = +inf for rows that keep all their positions
// (t + 1 <= k), -inf when the row has no more than jrank samples (every score is a
// candidate).  Block 0 also clears the recompute counter of this call.
constexpr int kSampleVec = 16;  // float4 loads per lane: up to 4096 samples per row

__global__ __launch_bounds__(256) void sample_threshold(const float* __restrict__ samp,
                                                        int64_t lds, int B, int row_begin,
                                                        int row_end, int k, int sshift,
                                                        int jrank, float* __restrict__ thr,
                                                        uint32_t* __restrict__ n_recomputed) {
  __shared__ uint32_t hist_s[4][kRadixBins];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_recomputed = 0u;
  const int R = row_end - row_begin;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= (int64_t)B * R) return;
  const int t = row_begin + (int)(item % R);
  if (t + 1 <= k || ((t >> sshift) + 1) <= jrank) {
    if (lane == 0) thr[item] = t + 1 <= k ? INFINITY : -INFINITY;
    return;
  }
  const int ns = (t >> sshift) + 1;
  // the row's samples through a buffer resource over its first ns floats rounded up to a
  // 16-byte load (within the row: lds is a multiple of 4): loads past it read zero with
  // no per-lane condition; positions e >= ns take key 0, below every finite score's key
  // (so below mn, and the radix skips them)
  const __amdgpu_buffer_rsrc_t rowr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(samp + item * lds), 0, ((ns + 3) & ~3) * 4, 0x00020000);
  // groups of 256 samples wholly past ns are skipped here and in the radix passes (their
  // keys are never read)
  int nq = ns;
  asm volatile("" : "+s"(nq));  // a scalar compare per group
  uint32_t key[4 * kSampleVec];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < kSampleVec; ++i) {
    if (256 * i < nq) {
      const int e = 256 * i + 4 * lane;
      const f32x4 x =
          __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rowr, e * 4, 0, 0));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t kv = e + u < ns ? order_key(x[u]) : 0u;
        key[4 * i + u] = kv;
        mn = min(mn, kv != 0u ? kv : 0xffffffffu);
        mx = max(mx, kv);
      }
    }
  }
  wave_minmax(mn, mx);
  uint32_t v;
  int take;
  bool whole;
  wave_radix_kth(mn, mx - mn, jrank,
                 [&](auto&& f) {
                   int nq2 = ns;
                   asm volatile("" : "+s"(nq2));  // a scalar compare per group, no kept masks
#pragma unroll
                   for (int i = 0; i < kSampleVec; ++i)
                     if (256 * i < nq2) {
#pragma unroll
                       for (int u = 0; u < 4; ++u) f(key[4 * i + u]);
                     }
                 },
                 hist_s[wv], lane, v, take, whole);
  // v is the jrank-th largest sample, or one below the smallest key kept whole
  if (lane == 0) thr[item] = key_to_float(take > 0 ? v : v + 1u);
}

// ---------------------------------------------------------------- 3. candidates
// A row keeps one candidate list per chunk group (the chunks c with the same c mod
// kIdxGroups, which one wavefront scores) of at most kGroupCap entries, kListLd apart.  A
// length of kListFull (recorded once a list was offered more than kGroupCap entries) marks
// a list that ran out of room; its stores went to the kListLd - kGroupCap spare entries
// behind it (writes start at most kListFull and a block adds at most 64).
constexpr int kGroupCap = 256;
constexpr uint32_t kListFull = kGroupCap + 1;
constexpr int kListLd = kGroupCap + 1 + 64 + 3;  // 324 entries

// v gets, in lane r, the 16-bit count r of the packed scalar pairs c2 (one v_writelane
// per row; the lane is an immediate)
template <int R>
__device__ __forceinline__ void count_to_lane(int& v, const uint32_t* c2) {
  asm("v_writelane_b32 %0, %1, %2"
      : "+v"(v)
      : "s"((int)((c2[R >> 1] >> (16 * (R & 1))) & 0xffffu)), "i"(R));
}
template <int... R>
__device__ __forceinline__ void counts_to_lanes(int& v, const uint32_t* c2,
                                                std::integer_sequence<int, R...>) {
  (count_to_lane<R>(v, c2), ...);
}

template <int H, int DI, bool F8>
__global__ __launch_bounds__(256) void indexer_cand(const uint8_t* __restrict__ qi,
                                                     const uint8_t* __restrict__ ki,
                                                     const float* __restrict__ wgt, int T,
                                                     int row_begin, int row_end, int k,
                                                     const float* __restrict__ thr,
                                                     uint16_t* __restrict__ counts,
                                                     u32x2* __restrict__ cand, int nch, int ng) {
  using IW = IdxWave<H, DI, F8>;
  constexpr int SB = 64;        // keys per staged block (4 tiles)
  constexpr int SROW = SB + 4;  // padded LDS row (floats)
  __shared__ __attribute__((aligned(16))) float stage[kIdxWaves][IW::ROWS * SROW];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int R = row_end - row_begin;
  const int strips = (R + kIdxStrip - 1) / kIdxStrip;
  const int strip = strips - 1 - (int)(blockIdx.x / kIdxGroups);  // longest strips first
  const int group = (int)(blockIdx.x % kIdxGroups);
  const int b = blockIdx.y;
  const int t0 = row_begin + strip * kIdxStrip + wv * IW::ROWS;
  if (t0 >= row_end) return;
  const int t_last = min(t0 + IW::ROWS, row_end) - 1;
  // every row of this wavefront keeps all its positions, or no chunk meets its rows (the
  // condition is wave-uniform; readfirstlane says so to the compiler, whose backend
  // otherwise fails on this kernel)
  if (__builtin_amdgcn_readfirstlane((int)(t_last < k || group > t_last / kIdxChunk))) return;
  const int wave_chunks = t_last / kIdxChunk + 1;

  IW iw;
  iw.load(qi + (int64_t)b * T * H * DI * IW::EB, t0, row_end, wgt, n, grp);
  const uint8_t* kib = ki + (int64_t)b * T * DI * IW::EB;
  float* st = stage[wv];

  // row rr of the wavefront is kept by lane rr: its threshold (+inf: no candidates)
  const int my_t = t0 + (lane & 31);
  const bool my_ok = lane < IW::ROWS && my_t < row_end && my_t >= k;
  const float thr_v = my_ok ? thr[(int64_t)b * R + (my_t - row_begin)] : INFINITY;
  float thr_s[IW::ROWS];  // the same, wave-uniform: compared from scalar registers
#pragma unroll
  for (int rr = 0; rr < IW::ROWS; ++rr)
    thr_s[rr] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(thr_v), rr));
  const int64_t row0 = (int64_t)b * R + (t0 - row_begin);

  // This wavefront's rows keep one list per row for its group (chunks group, group +
  // kIdxGroups, ...), appended chunk after chunk.  Running lengths (uniform; at most 64
  // per 64-key block of the group, so below 2^16): rows 2i and 2i + 1 in the low and high
  // halves of cnt2[i], so the 32 lengths take 16 scalar registers.
  uint32_t cnt2[IW::ROWS / 2];
#pragma unroll
  for (int i = 0; i < IW::ROWS / 2; ++i) cnt2[i] = 0u;
  for (int c = group; c < wave_chunks; c += kIdxGroups) {
    const int s_lo = c * kIdxChunk;
    const int s_hi = min(s_lo + kIdxChunk, t_last + 1);
    typename IW::Keys bk;
    IW::load_keys(kib, min(s_lo + n, T - 1), grp, bk);
    for (int j0 = s_lo; j0 < s_hi; j0 += SB) {
#pragma unroll
      for (int nt = 0; nt < SB / 16; ++nt) {
        typename IW::Keys bn;
        IW::load_keys(kib, min(j0 + nt * 16 + 16 + n, T - 1), grp, bn);
        float sc[IW::NSC];
        iw.scores(bk, sc);
#pragma unroll
        for (int i = 0; i < IW::NSC; ++i) st[IW::token(i, grp) * SROW + nt * 16 + n] = sc[i];
        bk = bn;
      }
      wave_lds_sync();
      // ---- row by row: one lane per key of the block
      const int s = j0 + lane;
      const int sd = s - t0;  // key s follows row rr when sd > rr (an immediate compare)
      float vals[IW::ROWS];
#pragma unroll
      for (int rr = 0; rr < IW::ROWS; ++rr) vals[rr] = st[rr * SROW + lane];
      // the group lists of the wavefront's 32 rows as one buffer resource: a lane's store
      // goes to byte offset 8 (rr * rstride + entry), the row's part (rr * rstride plus
      // its current length) in the store's scalar offset and the lane's place among the
      // row's hits in the vector offset.  Lanes without a candidate get the vector offset
      // 2^31, past the range (under 2^31 bytes) whether or not the hardware adds the
      // scalar offset (under 2^31) before its range check, and the hardware drops those
      // stores, so the compaction needs no exec-mask changes or branches.  Entries past
      // kGroupCap (a list that ran out of room) go to the list's spare entries, the write
      // position held at kListFull.  The base and the row pitch are opaque per block so
      // the compiler forms them (and the 32 row offsets) here instead of holding them in
      // scalar registers across blocks, which leaves room there for the 32 thresholds.
      int64_t cbo = (row0 * ng + group) * kListLd;
      asm volatile("" : "+s"(cbo));
      const uint32_t rstride8 = (uint32_t)ng * kListLd * 8u;  // bytes between rows' lists
      const __amdgpu_buffer_rsrc_t lists = __builtin_amdgcn_make_buffer_rsrc(
          cand + cbo, 0, (int)(rstride8 * IW::ROWS), 0x00020000);
      uint32_t rs8 = rstride8;
      asm volatile("" : "+s"(rs8));
      auto compact = [&](auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        uint32_t rowoff = 0u;
#pragma unroll
        for (int rr = 0; rr < IW::ROWS; ++rr) {
          const bool hit = vals[rr] >= thr_s[rr] && (!DIAG || sd <= rr);
          const uint64_t m = ballot(hit);
          const uint32_t cnt = min((cnt2[rr >> 1] >> (16 * (rr & 1))) & 0xffffu, kListFull);
          const uint32_t at = (uint32_t)lanes_below(m) * 8u;
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(vals[rr]), (uint32_t)s}, lists,
                                               hit ? at : 0x80000000u, (int)(rowoff + cnt * 8u), 0);
          rowoff += rs8;
          cnt2[rr >> 1] += (uint32_t)__popcll(m) << (16 * (rr & 1));
        }
      };
      if (j0 + SB - 1 > t0) compact(std::true_type{});  // some key follows some row
      else compact(std::false_type{});
      wave_lds_sync();
    }
    // lane rr: row rr's list length after this chunk (kListFull once past kGroupCap)
    int cnt_v = 0;
    counts_to_lanes(cnt_v, cnt2, std::make_integer_sequence<int, IW::ROWS>{});
    if (my_ok) counts[(row0 + lane) * nch + c] = (uint16_t)min((uint32_t)cnt_v, kListFull);
  }
}

// ---------------------------------------------------------------- 4. selection
// One wavefront per row (4 rows per workgroup, longest rows first).  The row's
// non-empty chunk lists, concatenated in position order, are held in registers with
// entry e = 64 j + lane in slot j (up to 64 slots: 4096 entries), so that loads and the
// output stores of a slot are contiguous.  The list holding entry e is found from a
// table in LDS that marks where each list starts, with a running maximum over the lanes.
constexpr int kCandPerLane = 64;
constexpr int kMarkCap = 64 * kCandPerLane;  // entries the mark table covers

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void cand_topk(
    int B, int T, int row_begin, int row_end, int k, const float* __restrict__ thr,
    const uint16_t* __restrict__ counts, const u32x2* __restrict__ cand, int nch, int ng,
    int32_t* __restrict__ idx, uint32_t* __restrict__ n_recomputed, int* __restrict__ fix_rows) {
  constexpr int J = kCandPerLane;
  // per wavefront: the list-start marks (during the gather) or the radix histogram
  __shared__ uint32_t work_s[4][kMarkCap / 2 > kRadixBins ? kMarkCap / 2 : kRadixBins];
  __shared__ uint32_t nz_s[4][1028];  // (chunk << 16) | list offset, non-empty lists only
  __shared__ uint32_t sbin_s[4][64];  // lists starting in each 64-entry slot
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = row_end - row_begin;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= (int64_t)B * R) return;
  const int b = (int)(item / R);
  const int r = R - 1 - (int)(item % R);  // longest rows first
  const int t = row_begin + r;
  const int n = t + 1;
  int32_t* __restrict__ out = idx + ((int64_t)b * T + t) * k;
  if (n <= k) {
    for (int i = lane; i < k; i += 64) out[i] = i < n ? i : -1;
    return;
  }
  const int64_t rowi = (int64_t)b * R + r;
  const uint16_t* __restrict__ cr = counts + rowi * nch;
  const u32x2* __restrict__ cl = cand + rowi * ng * kListLd;
  uint32_t* hist = work_s[wv];
  uint16_t* mark = reinterpret_cast<uint16_t*>(work_s[wv]);
  uint32_t* nz = nz_s[wv];
  uint32_t* sbin = sbin_s[wv];
  const int nc = t / kIdxChunk + 1;  // chunks of this row (<= 1024)

  // ---- list lengths.  counts[row, c] is the length of chunk c's group list once chunk c
  // was appended; lane L holds chunks 256 g + 4 L + i (g < 4, i < 4) in registers, and the
  // previous chunk of the same group, c - kIdxGroups, is held by lane L - 16 (by lane
  // L + 48 in the previous g): chunk c's entries are that list's [prev, count).
  static_assert(kIdxGroups == 64, "the lane mapping of the group lists assumes 64 groups");
  uint32_t len4[4][2], prv4[4][2];  // two u16 values per word
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = 256 * g + 4 * lane;
    u32x2 x = {0u, 0u};
    if (c < nc) x = *reinterpret_cast<const u32x2*>(cr + c);  // (nch is a multiple of 4)
    len4[g][0] = x[0];
    len4[g][1] = x[1];
  }
  {
    uint32_t up[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) up[g][w2] = (uint32_t)shfl_i((int)len4[g][w2], (lane + 48) & 63);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) prv4[g][w2] = lane >= 16 ? up[g][w2] : g > 0 ? up[g - 1][w2] : 0u;
  }
  auto half16 = [](uint32_t wd, int i) -> int { return (int)((wd >> (16 * (i & 1))) & 0xffffu); };
  auto len_of = [&](int g, int i) -> int {
    const int c = 256 * g + 4 * lane + i;
    return c < nc ? half16(len4[g][i >> 1], i) - half16(prv4[g][i >> 1], i) : 0;
  };
  // a list that ran out of room: the row is recomputed in full
  bool full = false;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      full |= 256 * g + 4 * lane + i < nc && half16(len4[g][i >> 1], i) == (int)kListFull;
  if (ballot(full) != 0ull) {
    if (lane == 0) fix_rows[atomicAdd(n_recomputed, 1u)] = (int)rowi;
    return;
  }
  int n_hits = 0, n_nz = 0, run[4], zrun[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    run[g] = n_hits;
    zrun[g] = n_nz;
    if (256 * g < nc) {
      int l = 0, z = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l += len_of(g, i);
        z += len_of(g, i) > 0;
      }
      int tl, tz;
      run[g] += wave_excl_sum(l, tl);
      zrun[g] += wave_excl_sum(z, tz);
      n_hits += tl;
      n_nz += tz;
    }
  }

  uint32_t v;
  int take_eq;
  bool whole;
  if (n_hits >= k && n_hits <= 64 * J) {
    // ---- the non-empty lists (chunk, offset), a mark where each one starts, and how
    // many start in each 64-entry slot
    const int nw = (n_hits + 1) / 2;
    for (int i = lane; i < nw; i += 64) work_s[wv][i] = 0xffffffffu;  // no mark
    sbin[lane] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      int o = run[g], zo = zrun[g];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = len_of(g, i);
        if (x > 0) {
          // entry e (o <= e < o + x) of the concatenation is cl[nz + e]
          nz[zo] = (uint32_t)(((4 * lane + i) & (kIdxGroups - 1)) * kListLd +
                              half16(prv4[g][i >> 1], i) - o);
          mark[o] = (uint16_t)zo;
          atomicAdd(&sbin[o >> 6], 1u);
          ++zo;
        }
        o += x;
      }
    }
    wave_lds_sync();
    // lane j: the list holding the entry just before slot j (lists that start in earlier
    // slots, minus one); slot 0 starts with list 0
    int n_lists;
    const int before_v = wave_excl_sum((int)sbin[lane], n_lists) - 1;
    // ---- gather: slot j holds entry 64 j + lane.  The list of an entry is the last one
    // starting at or before it: the running maximum of the marks within the slot, or
    // the list carried into the slot.  Slots are independent, eight per straight-line
    // group; lanes past the last entry load the last entry again and are ignored.
    uint32_t key[J];
    int pos[J];
#pragma unroll
    for (int j0 = 0; j0 < J; j0 += 8) {
      if (64 * j0 < n_hits) {
#pragma unroll
        for (int j = j0; j < j0 + 8; ++j) {
          const int e = min(64 * j + lane, n_hits - 1);
          const int mr = (int)mark[e];
          const int m = max(__builtin_amdgcn_readlane(before_v, j),
                            wave_incl_scan(mr != 0xffff ? mr : INT_MIN, INT_MIN,
                                           [](int x, int y) { return max(x, y); }));
          const u32x2 ent = cl[(int)nz[m] + e];
          key[j] = ent[0];
          pos[j] = (int)ent[1];
        }
      }
    }
    const int jn = (n_hits + 63) / 64;  // slots in use (the last one partly)
    // ordered keys; lanes past the last entry take key 0, below every finite score's key
    // (so they are never kept and the radix skips them)
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (j < jn) {
        key[j] = 64 * j + lane < n_hits ? order_key(__uint_as_float(key[j])) : 0u;
        mx = max(mx, key[j]);
      }
    }
    mx = wave_max_u32(mx);
    // every candidate scored at least the row's threshold
    const uint32_t lo = order_key(thr[rowi]);
    wave_lds_sync();  // the marks are dead: the histogram takes their place
    wave_radix_kth(lo, mx - lo, k,
                   [&](auto&& f) {
                     int jq = jn;
                     asm volatile("" : "+s"(jq));  // a scalar compare per slot, no kept masks
#pragma unroll
                     for (int j = 0; j < J; ++j)
                       if (j < jq) f(key[j]);
                   },
                   hist, lane, v, take_eq, whole);
    // ---- output: per slot, the kept entries ranked by a ballot and written through a
    // buffer store that drops the other lanes
    const uint64_t ob = reinterpret_cast<uint64_t>(out);  // uniform: keep it in SGPRs
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<int32_t*>(
            ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ob >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ob)),
        0, k * 4, 0x00020000);
    int kr = 0;  // kept entries in the slots before
    int jn_e = jn;
    asm volatile("" : "+s"(jn_e));  // a fresh scalar compare per slot, not a kept mask
    if (whole) {  // the kept set is the keys above one value
      const uint32_t vk = take_eq == 0 ? v : v - 1u;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (j < jn_e) {
          const bool keep = key[j] > vk;
          const uint64_t mk = ballot(keep);
          __builtin_amdgcn_raw_buffer_store_b32(
              (uint32_t)pos[j], orsrc, keep ? (uint32_t)(kr + lanes_below(mk)) * 4u : 0xffffffffu, 0, 0);
          kr += __popcll(mk);
        }
      }
    } else {  // keys > v, and the first take_eq keys == v in position order
      int er = 0;  // keys == v in the slots before
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (j < jn_e) {
          const bool eq = key[j] == v;
          const int eb = er + lanes_below(ballot(eq));
          const bool keep = key[j] > v || (eq && eb < take_eq);
          const uint64_t mk = ballot(keep);
          __builtin_amdgcn_raw_buffer_store_b32(
              (uint32_t)pos[j], orsrc, keep ? (uint32_t)(kr + lanes_below(mk)) * 4u : 0xffffffffu, 0, 0);
          kr += __popcll(mk);
          er += __popcll(ballot(eq));
        }
      }
    }
    return;
  }

  if (n_hits > k) {
    // ---- more entries than the registers hold: streaming passes over the lists, lane L
    // taking the chunks L, L + 64, ... (each list read in batches of 16 entries)
    auto each_entry = [&](int c, auto&& f) {
      const int st = c >= kIdxGroups ? (int)cr[c - kIdxGroups] : 0;
      const int len = (int)cr[c] - st;
      const u32x2* src = cl + (c & (kIdxGroups - 1)) * kListLd + st;
      for (int e0 = 0; e0 < len; e0 += 16) {
        u32x2 ev[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (e0 + u < len) ev[u] = src[e0 + u];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (e0 + u < len) f(order_key(__uint_as_float(ev[u][0])), (int)ev[u][1]);
      }
    };
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int c = lane; c < nc; c += 64)
      each_entry(c, [&](uint32_t key, int) {
        mn = min(mn, key);
        mx = max(mx, key);
      });
    wave_minmax(mn, mx);
    wave_radix_kth(mn, mx - mn, k,
                   [&](auto&& f) {
                     for (int c = lane; c < nc; c += 64)
                       each_entry(c, [&](uint32_t key, int) { f(key); });
                   },
                   hist, lane, v, take_eq, whole);
    // output in chunk order: 64 consecutive chunks per round, one per lane
    int gsum = 0, esum = 0;
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const int c = c0 + lane;
      int ng = 0, ne = 0;
      if (c < nc)
        each_entry(c, [&](uint32_t key, int) {
          ng += key > v;
          ne += key == v;
        });
      int tg, te;
      int gb = gsum + wave_excl_sum(ng, tg);
      int eb = esum + wave_excl_sum(ne, te);
      gsum += tg;
      esum += te;
      if (c < nc)
        each_entry(c, [&](uint32_t key, int p) {
          const bool g = key > v, e = key == v;
          const int at = g ? gb + min(eb, take_eq) : gb + eb;
          if (g || (e && eb < take_eq)) out[at] = p;
          gb += g;
          eb += e;
        });
    }
    return;
  }

  // ---- fewer entries than k (the threshold was above the k-th score): the row is listed,
  // and fix_score / fix_select recompute and select it over the whole grid
  if (lane == 0) fix_rows[atomicAdd(n_recomputed, 1u)] = (int)rowi;
}

// ---------------------------------------------------------------- 5. listed rows
// The rows cand_topk listed are recomputed in full (t + 1 scores, the same MFMA
// arithmetic as every other indexer kernel) into recompute slots of one row each, then
// selected there with the two-step path's two-pass radix selection (topk_row).
// fix_score scores the first nslots listed rows, one wavefront per 256-key chunk of a row,
// spread over the whole grid; fix_rows_k then has workgroup w select listed row w from
// slot w and, for listed rows beyond the slots (w + nslots, w + 2 nslots, ...), score each
// in the workgroup (its wavefronts taking the chunks in turn) and select it in slot w.
// With no listed row both return at once.
template <int H, int DI, bool F8>
__device__ __forceinline__ void fix_score_chunk(const uint8_t* __restrict__ qi,
                                                const uint8_t* __restrict__ ki,
                                                const float* __restrict__ wgt, int T, int b,
                                                int t, int c, float* __restrict__ frow,
                                                int lane) {
  using IW = IdxWave<H, DI, F8>;
  IW iw;
  iw.load_single(qi + (int64_t)b * T * H * DI * IW::EB, t, wgt, lane & 15, lane >> 4);
  const uint8_t* kib = ki + (int64_t)b * T * DI * IW::EB;
  constexpr int U = kIdxChunk / 16;  // the chunk's key tiles, all in flight
  typename IW::Keys bk[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    IW::load_keys(kib, min(c * kIdxChunk + u * 16 + (lane & 15), T - 1), lane >> 4, bk[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float sc = iw.score_single(bk[u]);
    const int key = c * kIdxChunk + u * 16 + (lane & 15);
    if (lane < 16 && key <= t) frow[key] = sc;
  }
}

template <int H, int DI, bool F8>
__global__ __launch_bounds__(256) void fix_score(const uint8_t* __restrict__ qi,
                                                 const uint8_t* __restrict__ ki,
                                                 const float* __restrict__ wgt, int T,
                                                 int row_begin, int row_end,
                                                 float* __restrict__ area, int64_t area_ld,
                                                 int nslots, const uint32_t* __restrict__ n_fix,
                                                 const int* __restrict__ fix_rows) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = row_end - row_begin;
  const int maxch = (row_end - 1) / kIdxChunk + 1;
  const int rows = min(__builtin_amdgcn_readfirstlane((int)*n_fix), nslots);
  const int64_t items = (int64_t)rows * maxch;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wv; it < items; it += (int64_t)gridDim.x * 4) {
    const int i = (int)(it / maxch), c = (int)(it % maxch);
    const int rowi = fix_rows[i];
    const int b = rowi / R, t = row_begin + rowi % R;
    if (c * kIdxChunk > t) continue;
    fix_score_chunk<H, DI, F8>(qi, ki, wgt, T, b, t, c, area + (int64_t)i * area_ld, lane);
  }
}

template <int H, int DI, bool F8>
__global__ __launch_bounds__(kTkThreads) void fix_rows_k(const uint8_t* __restrict__ qi,
                                                         const uint8_t* __restrict__ ki,
                                                         const float* __restrict__ wgt, int T,
                                                         int row_begin, int row_end, int k,
                                                         float* __restrict__ area,
                                                         int64_t area_ld,
                                                         int32_t* __restrict__ idx,
                                                         const uint32_t* __restrict__ n_fix,
                                                         const int* __restrict__ fix_rows) {
  __shared__ TopkShared sh;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = row_end - row_begin;
  const int cnt = __builtin_amdgcn_readfirstlane((int)*n_fix);
  float* __restrict__ frow = area + (int64_t)blockIdx.x * area_ld;
  for (int i = blockIdx.x; i < cnt; i += gridDim.x) {
    const int rowi = fix_rows[i];
    const int b = rowi / R, t = row_begin + rowi % R;
    if (i >= (int)gridDim.x) {  // beyond the slots fix_score filled: score it here
      for (int c = wv; c * kIdxChunk <= t; c += kTkWaves)
        fix_score_chunk<H, DI, F8>(qi, ki, wgt, T, b, t, c, frow, lane);
      __syncthreads();  // the row's scores are in the slot
    }
    topk_row(frow, t + 1, k, idx + ((int64_t)b * T + t) * k, sh);
    __syncthreads();  // the slot is free for the next row
  }
}

// ---------------------------------------------------------------- host side
namespace {

struct IdxTopkPlan {
  int sshift, jrank, nch, ng, nslots;
  int64_t ns_ld, fix_ld;
  size_t off_stat, off_samp, off_thr, off_cnt, off_fix, off_cand, off_area, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IdxTopkPlan plan_indexer_topk(int B, int row_begin, int row_end, int k) {
  IdxTopkPlan p{};
  // sample stride 2^sshift: about kf0 .. 2 kf0 sampled scores above the k-th largest.  The
  // candidate lists then hold about (1 + 4 / sqrt(kf0)) k entries: kf0 = 64 for k <= 2048,
  // 256 above, so that they fit the 4096 entries held in registers up to k of about 3000
  const int kf0 = k <= 2048 ? 64 : 256;
  int sshift = 0;
  while ((k >> (sshift + 1)) >= kf0) ++sshift;
  // at most 64 * 4 * kSampleVec samples per row (the threshold kernel holds them in
  // registers): longer rows take a sparser sample and a wider margin
  while (((row_end - 1) >> sshift) + 1 > 64 * 4 * kSampleVec) ++sshift;
  const int kf = max(1, k >> sshift);
  int sq = 0;
  while (sq * sq < kf) ++sq;
  p.sshift = sshift;
  p.jrank = kf + 4 * sq + 4;
  const int nchunks = (row_end - 1) / kIdxChunk + 1;
  p.nch = (nchunks + 3) / 4 * 4;  // multiple of 4: 8-byte count loads
  p.ng = nchunks < kIdxGroups ? nchunks : kIdxGroups;  // candidate lists per row
  p.ns_ld = ((int64_t)((row_end - 1) >> sshift) + 1 + 3) / 4 * 4;
  const int64_t rows = (int64_t)B * (row_end - row_begin);
  // the recompute slots: one full row of scores each, as many as fit 256 MB (1 to 256,
  // and no more than there are rows)
  p.fix_ld = ((int64_t)row_end + 63) / 64 * 64;
  const int64_t fit = ((int64_t)256 << 20) / (p.fix_ld * (int64_t)sizeof(float));
  p.nslots = (int)(fit < 1 ? 1 : fit > 256 ? 256 : fit);
  if (p.nslots > rows) p.nslots = (int)rows;
  size_t o = 0;
  p.off_stat = o;  // uint32: rows recomputed in full by the last call
  o = align256(o + sizeof(uint32_t));
  p.off_samp = o;
  o = align256(o + (size_t)rows * p.ns_ld * sizeof(float));
  p.off_thr = o;
  o = align256(o + (size_t)rows * sizeof(float));
  p.off_cnt = o;
  o = align256(o + (size_t)rows * p.nch * sizeof(uint16_t));
  p.off_fix = o;  // int32: rows listed for recomputation
  o = align256(o + (size_t)rows * sizeof(int));
  p.off_cand = o;  // per row: ng lists of kListLd (score bits, position) pairs
  o = align256(o + (size_t)rows * p.ng * kListLd * sizeof(u32x2));
  p.off_area = o;  // float: the recompute slots
  o = align256(o + (size_t)p.nslots * p.fix_ld * sizeof(float));
  p.total = o;
  return p;
}

}  // namespace

size_t indexer_topk_workspace_bytes(int B, int row_begin, int row_end, int k) {
  return plan_indexer_topk(B, row_begin, row_end, k).total;
}

hipError_t launch_indexer_topk(const void* qi, const void* ki, const float* w, int B, int T,
                               int H_I, int D_I, bool f8, int row_begin, int row_end, int k,
                               int32_t* idx, void* workspace, hipStream_t st) {
  const IdxTopkPlan p = plan_indexer_topk(B, row_begin, row_end, k);
  char* ws = static_cast<char*>(workspace);
  float* samp = reinterpret_cast<float*>(ws + p.off_samp);
  float* thr = reinterpret_cast<float*>(ws + p.off_thr);
  uint16_t* cnt = reinterpret_cast<uint16_t*>(ws + p.off_cnt);
  u32x2* cand = reinterpret_cast<u32x2*>(ws + p.off_cand);
  uint32_t* stat = reinterpret_cast<uint32_t*>(ws + p.off_stat);
  int* fix = reinterpret_cast<int*>(ws + p.off_fix);
  float* area = reinterpret_cast<float*>(ws + p.off_area);
  const int R = row_end - row_begin;

  // the sample: slot chunks of 64 spread the short sampled rows over more workgroups
  hipError_t e = launch_indexer_mfma(qi, ki, w, B, T, H_I, D_I, f8, row_begin, row_end,
                                     p.sshift, p.sshift > 0 ? 64 : kIdxChunk, samp, p.ns_ld, st);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)B * R;
  hipLaunchKernelGGL(sample_threshold, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, samp,
                     p.ns_ld, B, row_begin, row_end, k, p.sshift, p.jrank, thr, stat);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int strips = (R + kIdxStrip - 1) / kIdxStrip;
  const dim3 g3((unsigned)(strips * kIdxGroups), (unsigned)B);
  const dim3 g4((unsigned)((rows + 3) / 4));
  return dispatch_indexer(H_I, D_I, f8, [&](auto h, auto d, auto f) {
    constexpr int HH = decltype(h)::value, DD = decltype(d)::value;
    constexpr bool FF = decltype(f)::value;
    hipLaunchKernelGGL((indexer_cand<HH, DD, FF>), g3, dim3(256), 0, st, (const uint8_t*)qi,
                       (const uint8_t*)ki, w, T, row_begin, row_end, k, thr, cnt, cand, p.nch,
                       p.ng);
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL(cand_topk, g4, dim3(256), 0, st, B, T, row_begin, row_end, k, thr, cnt,
                       cand, p.nch, p.ng, idx, stat, fix);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    hipLaunchKernelGGL((fix_score<HH, DD, FF>), dim3(512), dim3(256), 0, st, (const uint8_t*)qi,
                       (const uint8_t*)ki, w, T, row_begin, row_end, area, p.fix_ld, p.nslots,
                       stat, fix);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    hipLaunchKernelGGL((fix_rows_k<HH, DD, FF>), dim3((unsigned)p.nslots), dim3(kTkThreads), 0, st,
                       (const uint8_t*)qi, (const uint8_t*)ki, w, T, row_begin, row_end, k, area,
                       p.fix_ld, idx, stat, fix);
    return hipGetLastError();
  });
}

}  // namespace sa
