// Read-bandwidth probe of the memory hierarchy (measurement only; not part of the C ABI of
// libsa).  bench.py times it to check the cache and HBM read peaks against which the
// gather kernels are held: a buffer small enough for every XCD's L2 (each XCD re-reads
// its own slice), one that fits the Infinity Cache but not the L2s, and one far larger
// than both (HBM).
//
// Workgroups are dealt to the 8 XCDs round-robin by their index, so workgroup w runs on
// XCD w % 8 and reads slice w % 8 of the buffer (slices = 8 when the buffer is meant to
// stay L2-resident, 1 otherwise).  Each lane reads 16 bytes per load, a wavefront 1 KB of
// contiguous memory per instruction, 4 loads in flight per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void read_probe(const u32x4* __restrict__ buf,
                                                       int64_t n16_per_slice, int slices,
                                                       int passes, uint32_t* __restrict__ sink) {
  const int xcd_slot = (int)(blockIdx.x % 8);
  const int slice = xcd_slot % slices;
  const int64_t wgs_on_slice = (int64_t)gridDim.x / 8 * (8 / slices);  // workgroups sharing it
  const int64_t rank = slices == 8 ? (int64_t)(blockIdx.x / 8) : (int64_t)blockIdx.x;
  const u32x4* base = buf + (int64_t)slice * n16_per_slice;
  const int64_t stride = wgs_on_slice * kThreads;
  uint32_t acc = 0;
  for (int p = 0; p < passes; ++p) {
    int64_t i = rank * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16_per_slice; i += kUnroll * stride) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = base[i + u * stride];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16_per_slice; i += stride) {
      const u32x4 v = base[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;  // keeps the loads alive
}

}  // namespace

extern "C" {

// Reads `bytes` of buf (16-byte aligned, a multiple of 16 * slices) `passes` times with
// `workgroups` workgroups (a multiple of 8); slices = 8 gives each XCD its own 1/8 of the
// buffer, slices = 1 streams the whole buffer from every XCD.  sink holds workgroups * 256
// uint32.  Returns the hipError_t of the launch.
int sa_probe_read(const void* buf, int64_t bytes, int slices, int passes, int workgroups,
                  void* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || (slices != 1 && slices != 8) || passes < 1 ||
      workgroups < 8 || workgroups % 8 || bytes % (16 * slices))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16 / slices;
  hipLaunchKernelGGL(read_probe, dim3(workgroups), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(buf),
                     n16, slices, passes, reinterpret_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"
