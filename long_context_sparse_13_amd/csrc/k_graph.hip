// Fixed-graph distance-logit attention.
//
// [SLM] SpatialLM-Mini page, "Cómo eligen los tokens a quién escuchar": the positions a
// token may attend to are fixed in advance — itself, its near predecessors and the
// positions at distances 1, 2, 4, 8, ... — never future ones; the weight of an allowed
// neighbour grows as the distance between learned 3-D query and key coordinates
// shrinks, shifted by a learned parameter.  The page also notes that the original
// implementation built intermediate tensors while gathering neighbours; here nothing is
// materialised outside the chip.
//
// graph_attn_block<D> (bf16, D in {64, 128}, local <= 64): one workgroup per (batch,
// block of 64 tokens, head).  The block's local neighbourhoods form a band: the rows
// [t0 - local, t0 + 64) hold every neighbour at offset <= local of every token of the
// block, so V^T of the band is staged once in LDS and the band part of P.V runs on the
// 16x16x32 bf16 MFMA (probabilities rounded to bf16, the normaliser summed from the
// same rounded values).  Four workgroups per CU (the LDS allows four; at D = 64 the
// register cap of four wavefronts per SIMD costs a 12-byte spill and gains 11 %).  The far neighbours (offsets 2^j > local) are one row per
// token and offset; their contributions are added on the vector units from coalesced
// row loads.  Logits and softmax are float32.  Items are handed to the XCDs in
// contiguous (block, head) ranges, so the rows a block shares with the blocks just
// before it are served from that XCD's L2.
//
// graph_attn<BF> (any dtype, D % 8 == 0, the general case): one wavefront per (batch,
// token, group of 64 eight-element chunks of the token's H*D values).  A lane owns one
// 8-element chunk of one head, computes that head's logits itself and runs an online
// softmax over the neighbour list.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

template <bool BF>
__device__ __forceinline__ float g_ld(const void* p, int64_t i) {
  if constexpr (BF) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <bool BF>
__global__ __launch_bounds__(64) void graph_attn(const void* __restrict__ cq,
                                                  const void* __restrict__ ck,
                                                  const void* __restrict__ v,
                                                  const float* __restrict__ bias, float tau_log2,
                                                  int B, int T, int H, int D, int local,
                                                  int n_pow2, void* __restrict__ out,
                                                  float* __restrict__ lse) {
  const int lane = threadIdx.x;
  const int HD8 = H * D / 8;               // 8-element chunks per token
  const int groups = (HD8 + 63) / 64;
  const int64_t item = xcd_item(blockIdx.x, (int64_t)B * T * groups);
  if (item < 0) return;
  const int cg = (int)(item % groups);
  const int t = (int)((item / groups) % T);
  const int b = (int)(item / ((int64_t)groups * T));
  const int c = cg * 64 + lane;
  if (c >= HD8) return;
  const int h = (c * 8) / D;
  const int d0 = c * 8 - h * D;

  const int64_t tok0 = (int64_t)b * T;
  const int64_t cqo = ((tok0 + t) * H + h) * 3;
  const float qx = g_ld<BF>(cq, cqo), qy = g_ld<BF>(cq, cqo + 1), qz = g_ld<BF>(cq, cqo + 2);
  const float bl2 = bias[h] * kLog2e;

  float m = -INFINITY, l = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  auto visit = [&](int s) {
    const int64_t cko = ((tok0 + s) * H + h) * 3;
    const float dx = qx - g_ld<BF>(ck, cko), dy = qy - g_ld<BF>(ck, cko + 1),
                dz = qz - g_ld<BF>(ck, cko + 2);
    const float lg = bl2 - tau_log2 * (dx * dx + dy * dy + dz * dz);  // log2 domain
    float vv[8];
    const int64_t vo = ((tok0 + s) * H + h) * (int64_t)D + d0;
    if constexpr (BF) {
      const u32x4 w = ld16(reinterpret_cast<const uint16_t*>(v) + vo);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vv[2 * i] = bf16_lo(w[i]);
        vv[2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      const float* vp = reinterpret_cast<const float*>(v) + vo;
      const f32x4 a = *reinterpret_cast<const f32x4*>(vp);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(vp + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vv[i] = a[i];
        vv[4 + i] = bb[i];
      }
    }
    const float mn = fmaxf(m, lg);
    const float al = exp2_hw(m - mn);
    const float p = exp2_hw(lg - mn);
    l = l * al + p;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] * al + p * vv[i];
    m = mn;
  };

  const int nloc = min(local, t);
  for (int o = 0; o <= nloc; ++o) visit(t - o);
  for (int j = 0; j < n_pow2; ++j) {
    const int o = 1 << j;
    if (o > t) break;
    if (o > local) visit(t - o);
  }

  const float inv = 1.f / l;  // l >= 1: the token itself is always a neighbour
  const int64_t oo = ((tok0 + t) * H + h) * (int64_t)D + d0;
  if constexpr (BF) {
    const u32x4 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    st16(reinterpret_cast<uint16_t*>(out) + oo, w);
  } else {
    float* op = reinterpret_cast<float*>(out) + oo;
    *reinterpret_cast<f32x4*>(op) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(op + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (lse && d0 == 0) lse[((int64_t)b * H + h) * T + t] = (m + __log2f(l)) * kLn2;
}


constexpr int kGTB = 64;   // tokens per block
constexpr int kGBR = 128;  // band rows held (block + local, local <= 64)
constexpr int kGPR = kGBR + 8;  // LDS row pitch of P and V^T (bf16), 16-byte multiple
constexpr int kGFar = 8;   // far offsets (2^j > local) handled: n_pow2 - #{2^j <= local} <= 8
constexpr int kGLoc = 17;  // band logits per thread: (local + 1) / 4 rounded up, local <= 64

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void graph_attn_block(
    const uint16_t* __restrict__ cq, const uint16_t* __restrict__ ck,
    const uint16_t* __restrict__ v, const float* __restrict__ bias, float tau_log2, int B, int T,
    int H, int local, int n_pow2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int DC = D / 8;              // 8-value chunks per row
  constexpr int CPT = DC / 4;            // output chunks per thread (4 threads per token)
  constexpr int VPT = kGBR * DC / 256;   // band V chunks loaded per thread
  constexpr int PBYTES = kGTB * (D + 4) * 4 > kGTB * kGPR * 2 ? kGTB * (D + 4) * 4 : kGTB * kGPR * 2;
  __shared__ __attribute__((aligned(16))) uint16_t vt[D][kGPR];  // V^T of the band
  // band probabilities (bf16, [token][kGPR]), then the band P.V (float, [token][D + 4])
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[PBYTES];
  __shared__ float cqs[kGTB][3], cks[kGBR][3];
  uint16_t(*pb)[kGPR] = reinterpret_cast<uint16_t(*)[kGPR]>(pbuf);
  float* ob = reinterpret_cast<float*>(pbuf);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nblk = (T + kGTB - 1) / kGTB;
  const int64_t item = xcd_item(blockIdx.x, (int64_t)B * nblk * H);
  if (item < 0) return;
  const int h = (int)(item % H);
  const int blk = (int)((item / H) % nblk);
  const int b = (int)(item / ((int64_t)H * nblk));
  const int t0 = blk * kGTB;
  const int nt = min(kGTB, T - t0);  // tokens of this block
  const int sb = t0 - local;         // position of band row 0
  const int nbr = nt + local;        // band rows in use
  const int64_t tok0 = (int64_t)b * T;
  const float bl2 = bias[h] * kLog2e;
  int nf = 0;  // far offsets 2^j > local: j = jf0 .. n_pow2 - 1
  for (int j = 0; j < n_pow2; ++j) nf += (1 << j) > local;
  const int jf0 = n_pow2 - nf;
  // this thread's token (4 threads per token) and its output chunks q + 4 i
  const int tt = tid >> 2, q = tid & 3;
  const int t = t0 + tt;
  const bool tok_ok = tt < nt;

  // ---- every global load first: band V and coordinates, far coordinates and far V rows
  u32x4 vb[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int e = tid + 256 * i, r = e / DC, s = sb + r;
    vb[i] = u32x4{0u, 0u, 0u, 0u};
    if (r < nbr && s >= 0) vb[i] = ld16(v + ((tok0 + s) * H + h) * D + (e - r * DC) * 8);
  }
  float ckv[2] = {0.f, 0.f};  // band coordinates: element tid and tid + 256 of [row][3]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i, r = e / 3, s = sb + r;
    if (e < kGBR * 3 && r < nbr && s >= 0) ckv[i] = bf16_to_f32(ck[((tok0 + s) * H + h) * 3 + (e - r * 3)]);
  }
  float cqv = 0.f;  // query coordinates: element tid of [token][3]
  if (tid < kGTB * 3 && tid / 3 < nt)
    cqv = bf16_to_f32(cq[((tok0 + t0 + tid / 3) * H + h) * 3 + tid % 3]);
  float fk[2][3];  // far coordinates: far offsets q and q + 4 of this thread's token
  int fs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int f = q + 4 * u;
    fs[u] = (tok_ok && f < nf) ? t - (1 << (jf0 + f)) : -1;
    fk[u][0] = fk[u][1] = fk[u][2] = 0.f;
    if (fs[u] >= 0) {
      const uint16_t* kp = ck + ((tok0 + fs[u]) * H + h) * 3;
      fk[u][0] = bf16_to_f32(kp[0]);
      fk[u][1] = bf16_to_f32(kp[1]);
      fk[u][2] = bf16_to_f32(kp[2]);
    }
  }
  // far V rows: this thread owns output chunks q + 4 c (c < CPT) of its token, and needs
  // every far offset's row for them
  u32x4 frow[kGFar][CPT];
#pragma unroll
  for (int f = 0; f < kGFar; ++f)
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      frow[f][c] = u32x4{0u, 0u, 0u, 0u};
      if (tok_ok && f < nf) {
        const int s = t - (1 << (jf0 + f));
        if (s >= 0) frow[f][c] = ld16(v + ((tok0 + s) * H + h) * D + (q + 4 * c) * 8);
      }
    }

  // ---- stage: V^T of the band, coordinates; P cleared.  A lane writes its 8 values
  // (features d0 .. d0+7 of one band row) in an order rotated by its chunk index, so that
  // at each step the lanes of different chunks write rows d0 + q with distinct q mod 8:
  // with a row pitch of 17 x 16 bytes those fall in distinct LDS banks (rows 8 apart
  // would share one).
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int e = tid + 256 * i, r = e / DC, c = e - r * DC, d0 = c * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int qv = (k + c) & 7;
      const uint32_t w01 = (qv & 2) ? vb[i][1] : vb[i][0];
      const uint32_t w23 = (qv & 2) ? vb[i][3] : vb[i][2];
      const uint32_t wv = (qv & 4) ? w23 : w01;
      vt[d0 + qv][r] = (uint16_t)((qv & 1) ? (wv >> 16) : (wv & 0xffffu));
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i;
    if (e < kGBR * 3) cks[e / 3][e % 3] = ckv[i];
  }
  if (tid < kGTB * 3) cqs[tid / 3][tid % 3] = cqv;
  for (int i = tid; i < kGTB * kGPR / 8; i += 256)
    reinterpret_cast<u32x4*>(&pb[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // ---- logits (log2 domain) and softmax: thread q of a token takes the band offsets
  // o = q, q + 4, ... and the far offsets q and q + 4
  const float qx = cqs[tt][0], qy = cqs[tt][1], qz = cqs[tt][2];
  auto logit = [&](float kx, float ky, float kz) {
    const float dx = qx - kx, dy = qy - ky, dz = qz - kz;
    return bl2 - tau_log2 * (dx * dx + dy * dy + dz * dz);
  };
  float lb[kGLoc], lf[2];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kGLoc; ++i) {
    const int o = q + 4 * i;
    lb[i] = -INFINITY;
    if (tok_ok && o <= local && t - o >= 0) {
      const int r = tt + local - o;
      lb[i] = logit(cks[r][0], cks[r][1], cks[r][2]);
    }
    mx = fmaxf(mx, lb[i]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    lf[u] = fs[u] >= 0 ? logit(fk[u][0], fk[u][1], fk[u][2]) : -INFINITY;
    mx = fmaxf(mx, lf[u]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  float sum = 0.f;   // normaliser of the weights as used (band weights rounded to bf16)
  float sume = 0.f;  // unrounded normaliser, for the log-sum-exp
#pragma unroll
  for (int i = 0; i < kGLoc; ++i) {
    if (lb[i] != -INFINITY) {
      const float p = exp2_hw(lb[i] - mx);
      const uint32_t pbits = f32_to_bf16_bits(p);
      sum += bf16_to_f32((uint16_t)pbits);
      sume += p;
      pb[tt][tt + local - (q + 4 * i)] = (uint16_t)pbits;
    }
  }
  float pfar[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    pfar[u] = lf[u] != -INFINITY ? exp2_hw(lf[u] - mx) : 0.f;
    sum += pfar[u];
    sume += pfar[u];
  }
  sum += __shfl_xor(sum, 1, 64);
  sum += __shfl_xor(sum, 2, 64);
  sume += __shfl_xor(sume, 1, 64);
  sume += __shfl_xor(sume, 2, 64);
  // every far weight of the token, from the 4 threads that computed them
  float pall[kGFar];
#pragma unroll
  for (int f = 0; f < kGFar; ++f) pall[f] = __shfl(pfar[f >> 2], (lane & ~3) | (f & 3), 64);
  __syncthreads();

  // ---- band P.V on MFMA: wavefront w takes tokens 16w .. 16w+15, all D columns
  {
    const int n16 = lane & 15, grp = lane >> 4;
    f32x4 acc[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kGBR / 32; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(&pb[16 * w + n16][kk * 32 + grp * 8]);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(&vt[c * 16 + n16][kk * 32 + grp * 8]);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bv), acc[c],
                                                         0, 0, 0);
      }
    }
    __syncthreads();  // P is read by every wavefront before the area takes the output
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[(16 * w + grp * 4 + i) * (D + 4) + c * 16 + n16] = acc[c][i];
  }
  __syncthreads();

  // ---- far neighbours, normalisation, output
  if (tok_ok) {
    const float inv = 1.f / sum;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int d0 = (q + 4 * c) * 8;
      float o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = ob[tt * (D + 4) + d0 + u];
#pragma unroll
      for (int f = 0; f < kGFar; ++f) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[2 * k] += pall[f] * bf16_lo(frow[f][c][k]);
          o[2 * k + 1] += pall[f] * bf16_hi(frow[f][c][k]);
        }
      }
      const u32x4 wv = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                        pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
      st16(out + ((tok0 + t) * H + h) * D + d0, wv);
    }
    if (lse && q == 0) lse[((int64_t)b * H + h) * T + t] = (mx + __log2f(sume)) * kLn2;
  }
}

hipError_t launch_graph_attn_fwd(const void* cq, const void* ck, const void* v, const float* bias,
                                 float tau, int B, int T, int H, int D, int local, int n_pow2,
                                 bool bf16, void* out, float* lse, hipStream_t st) {
  const float tl2 = tau * kLog2e;
  int n_far = 0;
  for (int j = 0; j < n_pow2; ++j) n_far += (1 << j) > local;
  if (bf16 && (D == 64 || D == 128) && local <= kGBR - kGTB && n_far <= kGFar) {
    const int nblk = (T + kGTB - 1) / kGTB;
    const dim3 grid((unsigned)xcd_grid((int64_t)B * nblk * H));
    if (D == 64)
      hipLaunchKernelGGL(graph_attn_block<64>, grid, dim3(256), 0, st, (const uint16_t*)cq,
                         (const uint16_t*)ck, (const uint16_t*)v, bias, tl2, B, T, H, local,
                         n_pow2, (uint16_t*)out, lse);
    else
      hipLaunchKernelGGL(graph_attn_block<128>, grid, dim3(256), 0, st, (const uint16_t*)cq,
                         (const uint16_t*)ck, (const uint16_t*)v, bias, tl2, B, T, H, local,
                         n_pow2, (uint16_t*)out, lse);
    return hipGetLastError();
  }
  const int groups = (H * D / 8 + 63) / 64;
  const dim3 grid((unsigned)xcd_grid((int64_t)B * T * groups));
  if (bf16)
    hipLaunchKernelGGL(graph_attn<true>, grid, dim3(64), 0, st, cq, ck, v, bias, tl2, B, T, H, D,
                       local, n_pow2, out, lse);
  else
    hipLaunchKernelGGL(graph_attn<false>, grid, dim3(64), 0, st, cq, ck, v, bias, tl2, B, T, H, D,
                       local, n_pow2, out, lse);
  return hipGetLastError();
}

}  // namespace sa
