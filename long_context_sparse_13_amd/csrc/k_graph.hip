// Fixed-graph distance-logit attention.
//
// [SLM] SpatialLM-Mini page, "Cómo eligen los tokens a quién escuchar": the positions a
// token may attend to are fixed in advance — itself, its near predecessors and the
// positions at distances 1, 2, 4, 8, ... — never future ones; the weight of an allowed
// neighbour grows as the distance between learned 3-D query and key coordinates
// shrinks, shifted by a learned parameter.  The page also notes that the original
// implementation built intermediate tensors while gathering neighbours; here nothing is
// materialised: each lane streams its neighbours' rows straight into registers.
//
// One wavefront per (batch, token, group of 64 eight-element chunks of the token's
// H*D values).  A lane owns one 8-element chunk of one head, computes that head's
// logits itself (3-D squared distance in float32) and runs an online softmax over the
// neighbour list, so no cross-lane traffic is needed.  Neighbour rows of consecutive
// tokens overlap almost entirely; tokens are handed to the XCDs in contiguous ranges so
// those rows are reused from each XCD's L2.
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
    const float al = exp2f(m - mn);
    const float p = exp2f(lg - mn);
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

hipError_t launch_graph_attn_fwd(const void* cq, const void* ck, const void* v, const float* bias,
                                 float tau, int B, int T, int H, int D, int local, int n_pow2,
                                 bool bf16, void* out, float* lse, hipStream_t st) {
  const int groups = (H * D / 8 + 63) / 64;
  const dim3 grid((unsigned)xcd_grid((int64_t)B * T * groups));
  const float tl2 = tau * kLog2e;
  if (bf16)
    hipLaunchKernelGGL(graph_attn<true>, grid, dim3(64), 0, st, cq, ck, v, bias, tl2, B, T, H, D,
                       local, n_pow2, out, lse);
  else
    hipLaunchKernelGGL(graph_attn<false>, grid, dim3(64), 0, st, cq, ck, v, bias, tl2, B, T, H, D,
                       local, n_pow2, out, lse);
  return hipGetLastError();
}

}  // namespace sa
