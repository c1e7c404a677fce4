// Measurement aid: sustained HBM read bandwidth (include/hspec_probe.h).
#include <hip/hip_runtime.h>

#include "../../include/hspec_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" int hspec_probe_stream_read(void* stream, const void* buf, size_t bytes, uint32_t* sink) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15)) return -1;
  hipLaunchKernelGGL(k_stream_read<4>, dim3(16384), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
