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
// block, so the band's V rows are staged once in LDS (row-major, 16-byte writes) and the
// band part of P.V runs on the 16x16x32 bf16 MFMA, its V^T operand read with gfx950's
// transposing LDS read (probabilities rounded to bf16, the normaliser summed from the
// same rounded values).  The far neighbours (offsets 2^j > local) are one row per token
// and offset; their weights are rounded to bf16 too and their contributions added two
// offsets at a time with the bf16 dot-product instruction (v_dot2c_f32_bf16: exact bf16
// products, float32 sums).  Logits and softmax are float32.  The kernel is bound by
// instruction issue more than by memory, so its rows are read through buffer resources
// (one per tensor, at this batch's and head's row 0) with 32-bit offsets — rows that do
// not exist get an offset past the resource and read as zero, with no branch — and the
// band loops run only as far as `local` needs.  At D = 64 four workgroups per CU (the
// LDS allows four); at D = 128 the LDS holds two, so the register cap asks for two
// wavefronts per SIMD only.  Items are (head, block) pairs in head-major order, handed
// to the XCDs in contiguous ranges: an XCD works through the blocks of one head (or a
// few) in order, so the rows its far neighbours re-read, up to 2^13 tokens back, are that
// head's recent rows and stay in the XCD's L2.
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


// Exchanges inside each quad of lanes (the 4 threads of a token) with DPP moves, no LDS
// round trip: the value of lane l ^ 1, of lane l ^ 2, and of the quad's lane k.
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_bcast(float v, int k) {  // k in 0..3, a constant
  const int x = __float_as_int(v);
  switch (k) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x00, 0xF, 0xF, true));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x55, 0xF, 0xF, true));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xAA, 0xF, 0xF, true));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xFF, 0xF, 0xF, true));
  }
}

constexpr int kGTB = 64;   // tokens per block
constexpr int kGBR = 128;  // band rows held (block + local, local <= 64)
constexpr int kGPR = kGBR + 8;  // LDS row pitch of P (bf16), 16-byte multiple
constexpr int kGFar = 8;   // far offsets (2^j > local) handled: n_pow2 - #{2^j <= local} <= 8
constexpr int kGLoc = 17;  // band logits per thread: (local + 1) / 4 rounded up, local <= 64
// A buffer offset past every resource of the block kernel: loads there read zero.  Rows
// of one batch span less than 2 GB (checked on the host), so this offset plus any in-row
// offset stays out of range.
constexpr uint32_t kGOut = 0x80000000u;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2))) void graph_attn_block(
    const uint16_t* __restrict__ cq, const uint16_t* __restrict__ ck,
    const uint16_t* __restrict__ v, const float* __restrict__ bias, float tau_log2, int B, int T,
    int H, int local, int n_pow2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int DC = D / 8;              // 8-value chunks per row
  constexpr int CPT = DC / 4;            // output chunks per thread (4 threads per token)
  constexpr int VPT = kGBR * DC / 256;   // band V chunks loaded per thread
  constexpr int PBYTES = kGTB * (D + 4) * 4 > kGTB * kGPR * 2 ? kGTB * (D + 4) * 4 : kGTB * kGPR * 2;
  // band V rows, row-major with a pitch of 2D + 32 bytes: the 4 rows x 8 bytes named by
  // each 16 lanes of a transposing read fall on distinct banks.  The 32 bytes past a row's
  // values hold coordinates as float (x, y, z, 0): band row r's at 2D, the query token
  // t0 + r's at 2D + 16 (r < 64).
  constexpr int VROW = 2 * D + 32;
  __shared__ __attribute__((aligned(16))) unsigned char vrow[kGBR * VROW];
  // band probabilities (bf16, [token][kGPR]), then the band P.V (float, [token][D + 4])
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[PBYTES];
  uint16_t(*pb)[kGPR] = reinterpret_cast<uint16_t(*)[kGPR]>(pbuf);
  float* ob = reinterpret_cast<float*>(pbuf);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nblk = (T + kGTB - 1) / kGTB;
  // items (block, head) of batch blockIdx.y, in contiguous ranges per XCD (fewer than
  // 2^31 of them: checked on the host, so the index arithmetic is 32-bit)
  const int item = (int)xcd_item(blockIdx.x, (int64_t)nblk * H);
  if (item < 0) return;
  const int h = (int)((uint32_t)item / (uint32_t)nblk);
  const int blk = (int)((uint32_t)item % (uint32_t)nblk);
  const int b = blockIdx.y;
  const int t0 = blk * kGTB;
  const int nt = min(kGTB, T - t0);  // tokens of this block
  const int sb = t0 - local;         // position of band row 0
  const int nbr = nt + local;        // band rows in use
  const float bl2 = bias[h] * kLog2e;
  int nf = 0;  // far offsets 2^j > local: j = jf0 .. n_pow2 - 1
  for (int j = 0; j < n_pow2; ++j) nf += (1 << j) > local;
  const int jf0 = n_pow2 - nf;
  const int nlb = local / 4 + 1;     // band steps: offsets q + 4 i, i < nlb
  // this thread's token (4 threads per token) and its output chunks q + 4 i
  const int tt = tid >> 2, q = tid & 3;
  const int t = t0 + tt;
  const bool tok_ok = tt < nt;

  // this (batch, head) of V, O and the coordinates as buffer resources: row s of V / O at
  // byte s * vp, of a coordinate array at s * cp
  const int vp = H * D * 2, cp = H * 6;
  const int64_t hrow = (int64_t)b * T * H + h;
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(v + hrow * D), 0, T * vp - h * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      out + hrow * D, 0, T * vp - h * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ck + hrow * 3), 0, T * cp - h * 6, 0x00020000);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(cq + hrow * 3), 0, T * cp - h * 6, 0x00020000);
  auto ld_c = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t off, int i) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * i, 0, 0);
  };

  // ---- every global load first, with no branch between them (a load whose row does not
  // exist gets an offset past its resource and reads zero), and none of their values
  // used before the last is issued: band V and coordinates, query coordinates, far
  // coordinates and far V rows
  u32x4 vb[VPT];
  {
    constexpr int RS = 256 / DC;   // band rows between this thread's loads
    const int r0 = tid / DC, s0 = sb + r0;
    const uint32_t o0 = (uint32_t)s0 * (uint32_t)vp + (uint32_t)(tid % DC) * 16u;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const bool ok = r0 + i * RS < nbr && s0 + i * RS >= 0;
      vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ok ? o0 + (uint32_t)(i * RS * vp) : kGOut, 0, 0);
    }
  }
  // coordinates (bf16 bits): threads 0..127 load band row tid, threads 128..191 query
  // token t0 + tid - 128, each from its own tensor; the other load of a thread is out of
  // range and reads zero, so the two combine with an OR
  uint32_t crd[3];
  {
    const int s = sb + tid, tq = tid - kGBR;
    const uint32_t o = tid < nbr && s >= 0 ? (uint32_t)s * (uint32_t)cp : kGOut;  // nbr <= kGBR
    const uint32_t oq = tq >= 0 && tq < nt ? (uint32_t)(t0 + tq) * (uint32_t)cp : kGOut;
#pragma unroll
    for (int i = 0; i < 3; ++i) crd[i] = ld_c(rk, o, i) | ld_c(rq, oq, i);
  }
  // far rows of this thread's token: offset 2^(jf0 + f) for f < nf; row t - 2^j exists
  // when t >= 2^j
  const uint32_t tvo = (uint32_t)t * (uint32_t)vp + (uint32_t)q * 16u;
  const uint32_t tco = (uint32_t)t * (uint32_t)cp;
  uint32_t fkr[2][3];  // far coordinates: far offsets q and q + 4 (bf16 bits)
  bool fok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int f = q + 4 * u;
    const int sh = min(jf0 + f, 30);
    fok[u] = tok_ok && f < nf && t >= (1 << sh);
    const uint32_t o = fok[u] ? tco - ((uint32_t)cp << sh) : kGOut;
#pragma unroll
    for (int i = 0; i < 3; ++i) fkr[u][i] = ld_c(rk, o, i);
  }
  // far V rows: this thread owns output chunks q + 4 c (c < CPT) of its token, and needs
  // every far offset's row for them
  u32x4 frow[kGFar][CPT];
#pragma unroll
  for (int f = 0; f < kGFar; ++f) {
    const int sh = min(jf0 + f, 30);
    const bool ok = tok_ok && f < nf && t >= (1 << sh);
    const uint32_t o = ok ? tvo - ((uint32_t)vp << sh) : kGOut;
#pragma unroll
    for (int c = 0; c < CPT; ++c) frow[f][c] = __builtin_amdgcn_raw_buffer_load_b128(rv, o + c * 64, 0, 0);
  }

  // ---- stage: the band's V rows (row-major), coordinates; P cleared
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int e = tid + 256 * i;
    st16(vrow + (e / DC) * VROW + (e % DC) * 16, vb[i]);
  }
  // every thread writes its coordinates (threads 192..255: zeros into the unused second
  // half of rows 64..127's spare bytes), so no load waits behind a branch
  {
    const int slot = tid < kGBR ? tid * VROW + 2 * D : (tid - kGBR) * VROW + 2 * D + 16;
    *reinterpret_cast<f32x4*>(vrow + slot) =
        f32x4{bf16_to_f32((uint16_t)crd[0]), bf16_to_f32((uint16_t)crd[1]),
              bf16_to_f32((uint16_t)crd[2]), 0.f};
  }
  for (int i = tid; i < kGTB * kGPR / 8; i += 256)
    reinterpret_cast<u32x4*>(&pb[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // ---- logits (log2 domain) and softmax: thread q of a token takes the band offsets
  // o = q, q + 4, ... (<= local) and the far offsets q and q + 4
  const f32x4 qc = *reinterpret_cast<const f32x4*>(vrow + tt * VROW + 2 * D + 16);
  auto logit = [&](float kx, float ky, float kz) {
    const float dx = qc[0] - kx, dy = qc[1] - ky, dz = qc[2] - kz;
    return bl2 - tau_log2 * (dx * dx + dy * dy + dz * dz);
  };
  float lb[kGLoc], lf[2];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kGLoc; ++i) {
    if (i >= nlb) break;  // uniform
    const int o = q + 4 * i;
    const bool ok = tok_ok && o <= local && t - o >= 0;
    const f32x4 kc = *reinterpret_cast<const f32x4*>(vrow + (ok ? tt + local - o : 0) * VROW + 2 * D);
    lb[i] = ok ? logit(kc[0], kc[1], kc[2]) : -INFINITY;
    mx = fmaxf(mx, lb[i]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    lf[u] = fok[u] ? logit(bf16_to_f32((uint16_t)fkr[u][0]), bf16_to_f32((uint16_t)fkr[u][1]),
                           bf16_to_f32((uint16_t)fkr[u][2]))
                   : -INFINITY;
    mx = fmaxf(mx, lf[u]);
  }
  mx = fmaxf(mx, quad_xor1(mx));
  mx = fmaxf(mx, quad_xor2(mx));
  float sum = 0.f;   // normaliser of the weights as used (rounded to bf16)
  float sume = 0.f;  // unrounded normaliser, for the log-sum-exp
#pragma unroll
  for (int i = 0; i < kGLoc; ++i) {
    if (i >= nlb) break;  // uniform
    if (lb[i] != -INFINITY) {
      const float p = exp2_hw(lb[i] - mx);
      const uint32_t pbits = f32_to_bf16_bits(p);
      sum += bf16_to_f32((uint16_t)pbits);
      sume += p;
      pb[tt][tt + local - (q + 4 * i)] = (uint16_t)pbits;
    }
  }
  float pfar[2];  // far weights rounded to bf16 (the dot-product inputs)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float p = lf[u] != -INFINITY ? exp2_hw(lf[u] - mx) : 0.f;
    pfar[u] = bf16_to_f32((uint16_t)f32_to_bf16_bits(p));
    sum += pfar[u];
    sume += p;
  }
  sum += quad_xor1(sum);
  sum += quad_xor2(sum);
  sume += quad_xor1(sume);
  sume += quad_xor2(sume);
  // every far weight of the token, from the 4 threads that computed them
  float pall[kGFar];
#pragma unroll
  for (int f = 0; f < kGFar; ++f) pall[f] = quad_bcast(pfar[f >> 2], f & 3);
  __syncthreads();

  // ---- band P.V on MFMA: wavefront w takes tokens 16w .. 16w+15, all D columns; band
  // rows from nbr on have P = 0, so 32-row steps past them are skipped
  {
    const int n16 = lane & 15, grp = lane >> 4;
    f32x4 acc[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // B operand of band rows kk*32 + grp*8 .. +7, columns c*16 + n16: two transposing
    // reads, lane (4j + q) of each 16 naming row j (then j + 4), columns 4q .. 4q+3
    const unsigned char* tr = vrow + (grp * 8 + (n16 >> 2)) * VROW + (n16 & 3) * 8;
#pragma unroll
    for (int kk = 0; kk < kGBR / 32; ++kk) {
      if (kk * 32 >= nbr) break;  // uniform
      const u32x4 a = *reinterpret_cast<const u32x4*>(&pb[16 * w + n16][kk * 32 + grp * 8]);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x2 lo = lds_read_tr16(tr + (kk * 32) * VROW + c * 32);
        const u32x2 hi = lds_read_tr16(tr + (kk * 32 + 4) * VROW + c * 32);
        const u32x4 bv = {lo[0], lo[1], hi[0], hi[1]};
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
    // far weights of offsets (2i, 2i + 1) packed as bf16 pairs
    bf16x2 pp[kGFar / 2];
#pragma unroll
    for (int i = 0; i < kGFar / 2; ++i)
      pp[i] = __builtin_bit_cast(bf16x2, pack_bf16x2(pall[2 * i], pall[2 * i + 1]));
    const uint32_t orow = (uint32_t)t * (uint32_t)vp;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int d0 = (q + 4 * c) * 8;
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&ob[tt * (D + 4) + d0]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&ob[tt * (D + 4) + d0 + 4]);
      float o[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < kGFar / 2; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // (V_f[d], V_f+1[d]) and (V_f[d+1], V_f+1[d+1]) for d = d0 + 2k, f = 2i
          const uint32_t a = frow[2 * i][c][k], b2 = frow[2 * i + 1][c][k];
          const uint32_t lo = __builtin_amdgcn_perm(b2, a, 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(b2, a, 0x07060302u);
          o[2 * k] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lo), pp[i],
                                                     o[2 * k], false);
          o[2 * k + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), pp[i],
                                                         o[2 * k + 1], false);
        }
      }
      const u32x4 wv = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                        pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
      __builtin_amdgcn_raw_buffer_store_b128(wv, ro, orow + d0 * 2, 0, 0);
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
  // the block kernel addresses one batch's rows with 32-bit buffer offsets
  const bool rows32 = (int64_t)T * H * D * 2 < ((int64_t)1 << 31);
  if (bf16 && (D == 64 || D == 128) && local <= kGBR - kGTB && n_far <= kGFar && rows32 &&
      B <= 65535) {
    const int nblk = (T + kGTB - 1) / kGTB;
    const dim3 grid((unsigned)xcd_grid((int64_t)nblk * H), (unsigned)B);
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
