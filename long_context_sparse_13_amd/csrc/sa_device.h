// Device-side helpers shared by the libsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

namespace sa {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bfloat16 <-> float
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> packed bfloat16 pair (lo in bits 0-15), round to nearest even; one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// ---------------------------------------------------------------- vector memory
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Cache-policy operand of buffer loads and stores: sc1, the policy agent-scope atomic
// accesses compile to on gfx950 (data written so is seen by workgroups on other XCDs).
constexpr int kSc1 = 16;

// Streaming (non-temporal) accesses for data touched once, so that it does not push
// reused data (gathered K/V rows) out of the caches.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ int ld_nt(const int* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing LDS read (ds_read_b64_tr_b16, gfx950).  Every lane names 8 bytes (four
// 16-bit values); within each block of 16 lanes, lane i receives, for j = 0..3, value
// i % 4 of the 8 bytes named by lane 4j + i / 4 of the same block (layout checked on the
// device).  So if lane 4j + q names row j, columns 4q..4q+3 of a 16-bit matrix, lane i
// receives column i of rows 0..3.  p must point into LDS, 8-byte aligned.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)const_cast<void*>(p)));
}

// 2^x on the hardware's exponential unit (one v_exp_f32, about 1 ulp).  The library's
// exp2f adds a rescaling step so that results below 2^-126 come out as denormals; the
// softmax weights never need those (they are below 2^-126 of the row maximum).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- cross-lane
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_i(int v, int src) { return __shfl(v, src, kWave); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}

// Sum over each aligned group of 8 lanes with DPP moves (no LDS round trip): xor 1,
// xor 2 within quads, then the mirror inside each half row pairs the two quads.
__device__ __forceinline__ float sum8_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
  return v;
}

// Maximum / sum of v over the lanes l, l ^ 16, l ^ 32 and l ^ 48 (the same position in the
// four 16-lane rows), in every one of them: gfx950's row-swap permutes exchange rows inside
// the vector unit, with no LDS round trip.  Every lane of the wavefront must be active.
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Inclusive scan over the 64 lanes with DPP moves (no LDS round trips): shifts by 1, 2,
// 4, 8 inside each row of 16 lanes, then row 0's total into rows 1 and 3 (row_bcast:15)
// and lane 31's running total into rows 2 and 3 (row_bcast:31).  op(a, b) must be
// associative with identity id (the value shifted in at row edges and masked rows).
template <typename Op>
__device__ __forceinline__ int wave_incl_scan(int x, int id, Op op) {
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the 64 lanes; total = the sum over all lanes.
__device__ __forceinline__ int wave_excl_sum(int v, int& total) {
  const int x = wave_incl_scan(v, 0, [](int a, int b) { return a + b; });
  total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Minimum and maximum over the 64 lanes (unsigned).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const int x = wave_incl_scan((int)v, -1, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  const int x = wave_incl_scan((int)v, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Orders LDS accesses of the lanes of one wavefront (LDS executes a wavefront's
// instructions in order; this keeps the compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
}

// ---------------------------------------------------------------- ordered keys
// Map a finite float to a uint32 whose unsigned order is the float order, with -0.0
// and +0.0 mapped to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- XCD-aware block order
// Work items are handed out so that each of the 8 XCDs (which round-robin consecutive
// workgroup ids) processes one contiguous range of items; neighbouring items then share
// that XCD's L2.  Returns -1 for padding ids when n is not a multiple of 8.
__device__ __forceinline__ int64_t xcd_item(int64_t bid, int64_t n) {
  const int64_t per = (n + 7) / 8;
  const int64_t item = (bid % 8) * per + bid / 8;
  return item < n ? item : -1;
}
__host__ __device__ inline int64_t xcd_grid(int64_t n) { return ((n + 7) / 8) * 8; }

// The same over `phases` consecutive ranges of ceil(n / phases) items, the last range
// first: blocks [r * G, (r + 1) * G) (G = xcd_grid of the range size) take range
// phases - 1 - r, dealt to the XCDs as xcd_item does.  Workgroups start roughly in block
// order, so the device works through one range of items at a time.
__device__ __forceinline__ int64_t xcd_item_phased(int64_t bid, int64_t n, int phases) {
  const int64_t m = (n + phases - 1) / phases;
  const int64_t g = xcd_grid(m);
  const int64_t base = (phases - 1 - bid / g) * m;
  const int64_t mp = n - base < m ? n - base : m;  // items of this range
  const int64_t bb = bid % g;
  if (mp <= 0 || bb >= xcd_grid(mp)) return -1;
  const int64_t it = xcd_item(bb, mp);
  return it < 0 ? -1 : base + it;
}
__host__ __device__ inline int64_t xcd_grid_phased(int64_t n, int phases) {
  return phases * xcd_grid((n + phases - 1) / phases);
}

}  // namespace sa
