// One wavefront attends one query (all query heads of one KV group, up to 16) to a
// stream of gathered keys, 32 keys per step, with an online softmax.
//
// Both products run on the gfx950 16x16x32 bf16 MFMA with the 16 query heads as the
// N dimension, so each gathered K/V row is fetched once for the whole group:
//   S^T[key, h] = K[key, :] . Q[h, :]       A = K rows (straight from memory, 16 B per
//                                           lane), B = Q (registers)
//   O^T[d, h]  += V^T[d, key] P^T[key, h]   A = V^T (LDS, transposed read), B = P^T
//                                           (the S^T accumulators, rounded to bf16)
// Lane (n = lane % 16, grp = lane / 16) holds, in the 16x16 MFMA C layout, rows
// grp*4 .. grp*4+3 of column n.  Column n is the query head, so the softmax statistics
// and the O^T accumulators of a head all live in the four lanes n, n+16, n+32, n+48 and
// the rescale by exp(m_old - m_new) is lane-local.
//
// The reduction (K) slot (grp, j) of the P.V product is mapped to the key
// kmap(grp, j) = grp*4 + j (j < 4) or 16 + grp*4 + j - 4 (j >= 4): exactly the keys
// whose scores the lane already holds from the two S^T tiles, so P needs no shuffle.
// The V^T operand of a d tile is two transposing LDS reads of the row-major staged V
// rows (keys grp*4 .. grp*4+3, then 16 + grp*4 ..); a row pitch of 2D + 32 bytes puts the
// 8 rows read by each half wavefront on distinct banks.
#pragma once

#include "sa_device.h"

namespace sa {

// OFS32: every row this wavefront reads lies less than 4 GB past kbase / vbase, so row
// addresses are a wave-uniform base plus a 32-bit byte offset (the loads' scalar-base
// form, slightly cheaper for the memory pipeline than 64-bit per-lane addresses).
template <int D, bool OFS32 = false>
struct GroupAttn {
  static constexpr int KS = D / 32;        // 32-wide k-steps of Q.K
  static constexpr int DT = D / 16;        // 16-wide d tiles of the output
  static constexpr int CH = D * 2 / 16;    // 16-byte chunks per bf16 row
  static constexpr int LROW = D * 2 + 32;  // LDS bytes per staged V row (padded)
  static constexpr int LDS_BYTES = 32 * LROW;

  bf16x8 qB[KS];
  f32x4 acc[DT];
  float m_run;  // running max of the log2-domain logits (same in the 4 lanes of a head)
  float l_run;  // lane-partial running sum of exp2(logit - m_run)

  // qrow: this lane's head row (D bf16) or nullptr for a padding head.
  __device__ __forceinline__ void init(const uint16_t* qrow, int grp) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qrow) w = ld16_nt(qrow + ks * 32 + grp * 8);
      qB[ks] = as_bf16x8(w);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // As init, with qrow an in-bounds row for every lane and `valid` false for a padding
  // head: the loads are issued unconditionally (no branch for the compiler's wait
  // placement to account for) and the padding heads' rows set to zero.
  __device__ __forceinline__ void init_masked(const uint16_t* qrow, bool valid, int grp) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = ld16_nt(qrow + ks * 32 + grp * 8);
      qB[ks] = as_bf16x8(valid ? w : u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // Registers of one gathered 32-key tile: K rows as MFMA A operands, V rows waiting to
  // be staged in LDS, and the slot mask (bit i set = slot i attended).
  struct Tile {
    u32x4 kA[2][KS];
    u32x4 vw[CH / 2];
    uint32_t vm;
  };

  // Issue the loads of one tile.  Every lane passes `key` = the key of slot (lane & 31)
  // (any in-bounds row index when that slot is invalid) and the slot mask `vm`.
  // kbase/vbase point at row 0 of this KV head; `stride` is the element distance between
  // consecutive rows.
  __device__ __forceinline__ void load(Tile& tl, const uint16_t* __restrict__ kbase,
                                       const uint16_t* __restrict__ vbase, int64_t stride,
                                       int key, uint32_t vm, int lane) const {
    const int n = lane & 15, grp = lane >> 4;
    tl.vm = vm;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int slot = c2 * 16 + n;
      const int kr = shfl_i(key, slot);
      const bool ok = (vm >> slot) & 1u;
      const uint16_t* kp = kbase + (int64_t)kr * stride + grp * 8;
      const uint32_t kofs = (uint32_t)kr * ((uint32_t)stride * 2u) + grp * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok) {
          if constexpr (OFS32) w = ld16(reinterpret_cast<const char*>(kbase) + (kofs + ks * 64));
          else w = ld16(kp + ks * 32);
        }
        tl.kA[c2][ks] = w;
      }
    }
    constexpr int RPI = 64 / CH;  // rows per wave instruction
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
      const int r = lane / CH + RPI * i;
      const int c = lane % CH;
      const int vr = shfl_i(key, r);
      u32x4 w = {0u, 0u, 0u, 0u};
      if ((vm >> r) & 1u) {
        if constexpr (OFS32)
          w = ld16(reinterpret_cast<const char*>(vbase) +
                   ((uint32_t)vr * ((uint32_t)stride * 2u) + c * 16));
        else w = ld16(vbase + (int64_t)vr * stride + c * 8);
      }
      tl.vw[i] = w;
    }
  }

  // First half of a tile's update: the scores S^T (returned) and the V rows staged in LDS.
  // After it the tile's registers are free for the next tile's loads.
  __device__ __forceinline__ void scores_and_stage(const Tile& tl, unsigned char* vl,
                                                   f32x4 (&s)[2], int lane) {
    // ---- S^T = K . Q^T for the two 16-key halves
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      s[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tl.kA[c2][ks]), qB[ks], s[c2], 0, 0, 0);
    }

    // stage V while the score MFMAs drain
    constexpr int RPI = 64 / CH;
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
      const int r = lane / CH + RPI * i;
      const int c = lane % CH;
      st16(vl + r * LROW + c * 16, tl.vw[i]);
    }
  }

  // Second half: online-softmax update with the scores s of a tile with slot mask vm
  // (not 0) and O^T += V^T P^T from the staged rows.  `vl` is this wave's LDS staging area
  // of LDS_BYTES.
  __device__ __forceinline__ void update(const f32x4 (&s)[2], uint32_t vm, unsigned char* vl,
                                         float scale_log2, int lane) {
    const int n = lane & 15, grp = lane >> 4;

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
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
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
    if (ballot(alpha != 1.f) != 0ull) {  // no head's maximum moved: nothing to rescale
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }

    const u32x4 pw = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    const bf16x8 pB = as_bf16x8(pw);

    wave_lds_sync();  // V rows written by other lanes are visible

    // ---- O^T += V^T . P^T; lane (n, grp) names row grp*4 + n/4 (then 16 + grp*4 + n/4),
    // columns dt*16 + 4*(n%4) .. +3, and receives V[kmap(grp, j)][dt*16 + n], j = 0..7
    const unsigned char* tr = vl + (grp * 4 + (n >> 2)) * LROW + (n & 3) * 8;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2 lo = lds_read_tr16(tr + dt * 32);
      const u32x2 hi = lds_read_tr16(tr + 16 * LROW + dt * 32);
      const u32x4 aw = {lo[0], lo[1], hi[0], hi[1]};
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw), pB, acc[dt], 0, 0, 0);
    }

    wave_lds_sync();  // the staging area may be overwritten by the next tile
  }

  // Streams `ntiles` tiles with one tile's registers (fewer registers, so more wavefronts
  // per SIMD, which beats two tiles of registers in each wavefront): once a tile's K rows
  // have fed the score MFMAs and its V rows are staged in LDS, the next non-empty tile's
  // rows are requested into the same registers, so they are in flight during this tile's
  // softmax and P.V (5.10 -> 5.02 ms on the 64K workload, same bits); empty tiles are
  // skipped.  fetch(i) returns this lane's raw key of tile i (it may issue a load, which
  // is started one tile ahead); finish(i, raw, key, vm) turns it into the slot key and
  // the tile's slot mask.
  template <typename Fetch, typename Finish>
  __device__ __forceinline__ void run(int ntiles, Fetch&& fetch, Finish&& finish,
                                      const uint16_t* __restrict__ kbase,
                                      const uint16_t* __restrict__ vbase, int64_t stride,
                                      unsigned char* vl, float scale_log2, int lane) {
    if (ntiles <= 0) return;
    Tile A;
    int key;
    uint32_t vm;
    int i = 0;
    int r = fetch(0);
    // load the next non-empty tile into A; false when none is left
    auto advance = [&]() -> bool {
      while (i < ntiles) {
        finish(i, r, key, vm);
        ++i;
        if (i < ntiles) r = fetch(i);  // the next raw key is in flight meanwhile
        if (vm != 0u) {
          load(A, kbase, vbase, stride, key, vm, lane);
          return true;
        }
      }
      return false;
    };
    bool have = advance();
    while (have) {
      const uint32_t cur_vm = A.vm;
      f32x4 s[2];
      scores_and_stage(A, vl, s, lane);
      // A's registers are consumed: the next tile's rows are requested now and arrive
      // while this tile's softmax and P.V run
      have = advance();
      update(s, cur_vm, vl, scale_log2, lane);
    }
  }

  // Sum of the lane-partial l over the 4 lanes of head n.
  __device__ __forceinline__ float total_l() const {
    float l = l_run;
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    return l;
  }
};

}  // namespace sa
