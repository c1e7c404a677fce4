// Measurement aid: sustained HBM read bandwidth (include/hspec_probe.h).
#include <hip/hip_runtime.h>

#include "../../include/hspec_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Each workgroup streams its own contiguous slice of `per16` 16-byte pieces
// (the last one the remainder), U nontemporal loads in flight per thread; a
// wave's load covers 1 KB of consecutive bytes.  Loads past the buffer are
// clamped to its last piece (only ever in the tail slice).
template <int U>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, size_t n16, size_t per16,
                                                     uint32_t* sink) {
  uint32_t acc = 0;
  const size_t base = size_t(blockIdx.x) * per16;
  const size_t end = base + per16 < n16 ? base + per16 : n16;
  for (size_t i = base + threadIdx.x; i < end; i += size_t(256) * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + size_t(u) * 256;
      v[u] = __builtin_nontemporal_load(p + (k < n16 ? k : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" int hspec_probe_stream_read(void* stream, const void* buf, size_t bytes, uint32_t* sink) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15)) return -1;
  constexpr int kGrid = 512, kU = 8;
  const size_t n16 = bytes / 16, step = size_t(256) * kU;
  const size_t per16 = ((n16 + kGrid - 1) / kGrid + step - 1) / step * step;
  hipLaunchKernelGGL(k_stream_read<kU>, dim3(kGrid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, per16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
