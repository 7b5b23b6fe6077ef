// kvc_measure.hip -- measurement helper behind the C ABI: a streaming read
// of a device buffer with the same non-temporal 16-byte loads the attend
// kernels use for the K/V rows, so that a benchmark can quote an achievable
// read ceiling of the part next to the vendor peak.  No part of the step
// calls it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/kvc.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;  // 16-byte loads per thread per iteration

typedef unsigned int rd_u32x4 __attribute__((ext_vector_type(4)));

// Workgroup g reads the contiguous slab [g * slab, (g + 1) * slab) in steps
// of kThreads * kInFlight * 16 bytes; every lane folds what it read into one
// word so that no load is dead.  slab is a multiple of the step (host checks).
__global__ __launch_bounds__(kThreads) void read_slabs_kernel(const uint8_t* __restrict__ buf,
                                                             uint64_t slab,
                                                             uint32_t* __restrict__ sink) {
  constexpr uint64_t kStep = static_cast<uint64_t>(kThreads) * kInFlight * 16;
  const uint8_t* p = buf + blockIdx.x * slab + threadIdx.x * 16;
  uint32_t acc = 0;
  for (uint64_t off = 0; off < slab; off += kStep) {
    rd_u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; u++)
      v[u] = __builtin_nontemporal_load(
          reinterpret_cast<const rd_u32x4*>(p + off + static_cast<uint64_t>(u) * kThreads * 16));
#pragma unroll
    for (int u = 0; u < kInFlight; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

size_t kvc_read_ceiling_sink_bytes(int workgroups) {
  return workgroups > 0 ? static_cast<size_t>(workgroups) * kThreads * sizeof(uint32_t) : 0;
}

int kvc_read_ceiling(const void* buffer, size_t bytes, int workgroups, void* sink,
                     size_t sink_bytes, void* stream) {
  if (!buffer || !sink) return KVC_ERR_NULL;
  const uint64_t step = static_cast<uint64_t>(kThreads) * kInFlight * 16;
  if (workgroups < 1 || bytes == 0 || bytes % (static_cast<uint64_t>(workgroups) * step) != 0)
    return KVC_ERR_SHAPE;
  if (sink_bytes < kvc_read_ceiling_sink_bytes(workgroups)) return KVC_ERR_WORKSPACE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_slabs_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buffer),
                     static_cast<uint64_t>(bytes / workgroups), static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

}  // extern "C"
