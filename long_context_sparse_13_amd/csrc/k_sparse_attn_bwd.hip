// Gathered causal sparse attention backward: dQ, dK, dV for the forward over
// S_t = listed indices U window (the same key order and masks as the forward).
//
// [NSA] Native Sparse Attention page, "Puntos Clave": the backward pass of sparse attention
// (6x at 64K there) beside the forward; "Análisis Profundo": one K/V fetch per GQA group.
//
// sparse_attn_bwd_mfma<D>: bf16, up to 16 query heads per KV head.  One wavefront per
// (batch, token, KV head), 32 gathered keys per step, the 16 query heads as the MFMA N
// dimension (as in the forward):
//   S^T  = K . Q^T        A = K rows (16 B per lane, also staged in LDS), B = Q
//   dP^T = V . dO^T       A = V rows, B = dO
//   P = exp2(S * scale * log2 e - lse2),  dS = P (dP - delta),  delta = dO . O
//   dQ^T += K^T . dS^T    A = K^T read transposed from LDS, B = dS^T (bf16)
//   dV    = P^T . dO      16x16x16: A = P^T through LDS, B = dO (registers, once per
//   dK    = dS^T . Q      wavefront); each atomic instruction covers 16 consecutive floats
//                         of 4 rows
// dK and dV rows are added with float atomics into float32 buffers that the launch clears
// first (a key is selected by many queries); dQ is written once per (token, head).  The
// atomics bound the kernel: at 64K (139 M selected (query, key) pairs, 256 float adds
// each) they take ~95% of its time.
#include "attn_tile.h"
#include "sa_launch.h"

namespace sa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void clear_f32(float* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) *reinterpret_cast<f32x4*>(p + 4 * i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
__global__ __launch_bounds__(64) void sparse_attn_bwd_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ o, const float* __restrict__ lse,
    const uint16_t* __restrict__ dout, int B, int T, int Hq, int Hkv, int topk, int window,
    float scale, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int LROW = D * 2 + 16;  // padded LDS row of a staged K row
  __shared__ __attribute__((aligned(16))) unsigned char kl[32 * LROW];
  __shared__ __attribute__((aligned(16))) uint16_t pl[32][16];  // P as [key][head] (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t sl[32][16];  // dS as [key][head]

  const int lane = threadIdx.x;
  const int n = lane & 15, grp = lane >> 4;
  const int64_t item = xcd_item(blockIdx.x, (int64_t)B * T * Hkv);
  if (item < 0) return;
  const int g = (int)(item % Hkv);
  const int t = (int)((item / Hkv) % T);
  const int b = (int)(item / ((int64_t)Hkv * T));
  const int G = Hq / Hkv;
  const int h = g * G + n;
  const bool hv = n < G;
  const float scale_log2 = scale * 1.4426950408889634f;

  // ---- per (token, head): Q and dO as B operands; delta = dO . O; the log2-domain lse
  const int64_t hrow = ((int64_t)b * T + t) * Hq + h;
  bf16x8 qB[KS], dB[KS];
  float delta = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 wq = {0u, 0u, 0u, 0u}, wd = wq, wo = wq;
    if (hv) {
      wq = ld16(q + hrow * D + ks * 32 + grp * 8);
      wd = ld16(dout + hrow * D + ks * 32 + grp * 8);
      wo = ld16(o + hrow * D + ks * 32 + grp * 8);
    }
    qB[ks] = as_bf16x8(wq);
    dB[ks] = as_bf16x8(wd);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      delta += bf16_lo(wd[c]) * bf16_lo(wo[c]) + bf16_hi(wd[c]) * bf16_hi(wo[c]);
  }
  delta += shfl_xor_f(delta, 16);
  delta += shfl_xor_f(delta, 32);
  const float lse2 = hv ? lse[((int64_t)b * Hq + h) * T + t] * 1.4426950408889634f : 0.f;

  // ---- A operands of the 16x16x16 products: dO^T and Q^T, d = dt*16 + n, heads grp*4 + j
  s16x4 aDO[DT], aQ[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = grp * 4 + j;
      const bool ok = hh < G;
      const int64_t r = (((int64_t)b * T + t) * Hq + g * G + hh) * D + dt * 16 + n;
      aDO[dt][j] = ok ? (short)dout[r] : (short)0;
      aQ[dt][j] = ok ? (short)q[r] : (short)0;
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
  const int n_idx = (topk + 31) / 32;
  const int n_win = (window + 31) / 32;
  const int slot = lane & 31;
  const int last_listed = t - window;
  const int wlo = t - window + 1;

  for (int tile = 0; tile < n_idx + n_win; ++tile) {
    // the tile's keys, as in the forward: listed positions outside [0, t - window] and
    // window positions outside [0, t] are masked out, so each key counts once
    int raw;
    bool ok;
    if (tile < n_idx) {
      const int e = tile * 32 + slot;
      raw = e < topk ? irow[e] : -1;
      ok = raw >= 0 && raw <= last_listed;
    } else {
      raw = wlo + (tile - n_idx) * 32 + slot;
      ok = raw >= 0 && raw <= t;
    }
    const uint32_t vm = (uint32_t)ballot(ok);
    if (vm == 0u) continue;
    const int key = ok ? raw : 0;

    // K and V rows of the tile's two 16-key halves as A operands
    u32x4 kA[2][KS], vA[2][KS];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int sl_ = c2 * 16 + n;
      const int kr = shfl_i(key, sl_);
      const bool okr = (vm >> sl_) & 1u;
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
    f32x4 s[2], dp[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      s[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[c2] = s[c2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kA[c2][ks]), qB[ks], s[c2], 0, 0, 0);
        dp[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vA[c2][ks]), dB[ks], dp[c2], 0, 0, 0);
      }
      // stage the K rows (key c2*16 + n, features ks*32 + grp*8) for the K^T reads
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st16(kl + (c2 * 16 + n) * LROW + (ks * 32 + grp * 8) * 2, kA[c2][ks]);
    }

    // P and dS: lane (n, grp) holds keys c2*16 + grp*4 + i of head n
    float pv[8], dsv[8];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sk = c2 * 16 + grp * 4 + i;
        const bool on = hv && ((vm >> sk) & 1u);
        const float p = on ? exp2f(s[c2][i] * scale_log2 - lse2) : 0.f;
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
    // registers (heads grp*4 + j, d = dt*16 + n); C: keys c2*16 + grp*4 + i, d = dt*16 + n,
    // so each atomic instruction covers 16 consecutive floats of 4 rows
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const s16x4 aP = *reinterpret_cast<const s16x4*>(&pl[c2 * 16 + n][grp * 4]);
      const s16x4 aS = *reinterpret_cast<const s16x4*>(&sl[c2 * 16 + n][grp * 4]);
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
    wave_lds_sync();  // the staging areas are rewritten by the next tile
  }

  if (hv) {
    float* qr = dq + hrow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(qr + dt * 16 + grp * 4) = acc[dt] * scale;
  }
}

hipError_t launch_sparse_attn_bwd(const void* q, const void* k, const void* v, const int32_t* idx,
                                  int B, int T, int Hq, int Hkv, int D, int topk, int window,
                                  float scale, const void* out, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv,
                                  hipStream_t st) {
  const int64_t n4 = (int64_t)B * T * Hkv * D / 4;
  const dim3 gc((unsigned)((n4 + 255) / 256));
  hipLaunchKernelGGL(clear_f32, gc, dim3(256), 0, st, dk, n4);
  hipLaunchKernelGGL(clear_f32, gc, dim3(256), 0, st, dv, n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = (int64_t)B * T * Hkv;
  const dim3 grid((unsigned)((items + 7) / 8 * 8));
  if (D == 128)
    hipLaunchKernelGGL(sparse_attn_bwd_mfma<128>, grid, dim3(64), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, idx, (const uint16_t*)out, lse,
                       (const uint16_t*)dout, B, T, Hq, Hkv, topk, window, scale, dq, dk, dv);
  else
    hipLaunchKernelGGL(sparse_attn_bwd_mfma<64>, grid, dim3(64), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, idx, (const uint16_t*)out, lse,
                       (const uint16_t*)dout, B, T, Hq, Hkv, topk, window, scale, dq, dk, dv);
  return hipGetLastError();
}

}  // namespace sa
