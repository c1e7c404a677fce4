// Measurement aids (include/hspec_probe.h): sustained HBM read bandwidth, and
// the LDS cost of one wave-wide access pattern.
#include <hip/hip_runtime.h>

#include "../../include/hspec_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// LDS bytes of the access-pattern probe (a power of two)
constexpr uint32_t kProbeLdsBytes = 16384;

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

namespace {

struct LdsPattern {
  uint32_t off[64];  // byte offset of each lane's access, host-checked
};

// Every wave of every workgroup repeats one LDS access of the given kind at
// its lane's offset `iters` times (the offset passes through an empty asm
// before each access, so the compiler can neither merge nor hoist one, but
// may keep eight in flight); nothing else touches memory until the one store
// at the end, which the data gate keeps from happening.  KIND 0: 16-byte read,
// 1: 16-byte write, 2: 8-byte read.
template <int KIND>
__global__ __launch_bounds__(256) void k_lds_pattern(LdsPattern p, int iters, uint32_t* sink) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  uint32_t off = p.off[lane] & (kProbeLdsBytes - (KIND == 2 ? 8 : 16));
  // defined contents: each thread clears its own 16 bytes of every 4 KiB
  for (uint32_t o = threadIdx.x * 16; o < kProbeLdsBytes; o += 256 * 16)
    *reinterpret_cast<u32x4*>(lds + o) = u32x4{0, 0, 0, 0};
  __syncthreads();
  uint32_t acc = 0;
  u32x4 val = {threadIdx.x, 1, 2, 3};
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      asm volatile("" : "+v"(off));   // the offset is opaque: no access is combined with another
      if constexpr (KIND == 0) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(lds + off);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
      } else if constexpr (KIND == 1) {
        *reinterpret_cast<u32x4*>(lds + off) = val;
        val.x += 1;
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(lds + off);
        acc ^= x.x ^ x.y;
      }
    }
  }
  __syncthreads();
  acc ^= *reinterpret_cast<const uint32_t*>(lds + (threadIdx.x * 4));
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" int hspec_probe_lds_pattern(void* stream, int kind, const uint32_t* offsets, int iters, int grid,
                                       uint32_t* sink) {
  if (!offsets || !sink || kind < 0 || kind > 2 || iters < 8 || iters % 8 || iters > (1 << 20) || grid < 1 ||
      grid > 65536)
    return -1;
  LdsPattern p;
  const uint32_t align = kind == 2 ? 8 : 16;
  for (int l = 0; l < 64; ++l) {
    if (offsets[l] % align || offsets[l] > kProbeLdsBytes - align) return -1;
    p.off[l] = offsets[l];
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(k_lds_pattern<0>, dim3(grid), dim3(256), kProbeLdsBytes, st, p, iters, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(k_lds_pattern<1>, dim3(grid), dim3(256), kProbeLdsBytes, st, p, iters, sink);
  else
    hipLaunchKernelGGL(k_lds_pattern<2>, dim3(grid), dim3(256), kProbeLdsBytes, st, p, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
