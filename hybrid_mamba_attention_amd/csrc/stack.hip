// The residual stream of the drafter stack between its layers: one kernel
// per layer boundary adds the layer's half outputs into the fp32 stream and
// normalises it for the next layer (H-Spec, Abstract: a backbone of Mamba-2
// and attention modules; the stack's wiring is stated with the C ABI).
//
//   h = src ? decode(src) : h + add0 + add1        (fp32 [T, d], in place)
//   x = h / sqrt(mean(h^2) + eps) * w               (activation type, when w is set)
//
// One wave per token row; with d = 256*NV the row is held in registers as
// float4 (one read of h, one write of each output), otherwise two passes.
#include "common.h"
#include "kernels.h"

namespace hspec {

namespace {

template <typename T> __device__ __forceinline__ float4 load4(const T* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                     bf16_to_f32(v.y >> 16));
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

}  // namespace

// Row held in registers as NV float4 per lane.  The inputs are fixed at
// compile time (SRC: decode src; otherwise h plus NADD of add0 / add1; NORM:
// write x), so every load of the row is issued before the first use: with
// the pointer tests inside the loop the loads went out one round trip at a
// time (15 us for 16 rows).
template <typename T, int NV, bool SRC, int NADD, bool NORM>
__global__ __launch_bounds__(256) void k_add_norm_v4(AddNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const size_t base = size_t(row) * a.d;
  float4 hv[NV];
  if constexpr (SRC) {
#pragma unroll
    for (int v = 0; v < NV; ++v) hv[v] = load4(static_cast<const T*>(a.src) + base + 4 * (lane + 64 * v));
  } else {
    float4 x0[NADD >= 1 ? NV : 1], x1[NADD >= 2 ? NV : 1];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const size_t c = base + 4 * (lane + 64 * v);
      hv[v] = *reinterpret_cast<const float4*>(a.h + c);
      if constexpr (NADD >= 1) x0[v] = load4(static_cast<const T*>(a.add0) + c);
      if constexpr (NADD >= 2) x1[v] = load4(static_cast<const T*>(a.add1) + c);
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (NADD >= 1) hv[v] = add4(hv[v], x0[v]);
      if constexpr (NADD >= 2) hv[v] = add4(hv[v], x1[v]);
    }
  }
  float4 w[NORM ? NV : 1];
  if constexpr (NORM) {
#pragma unroll
    for (int v = 0; v < NV; ++v) w[v] = *reinterpret_cast<const float4*>(a.norm_w + 4 * (lane + 64 * v));
  }
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    *reinterpret_cast<float4*>(a.h + base + 4 * (lane + 64 * v)) = hv[v];
    const float4 h = hv[v];
    ss = fmaf(h.x, h.x, fmaf(h.y, h.y, fmaf(h.z, h.z, fmaf(h.w, h.w, ss))));
  }
  if constexpr (NORM) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss = wave_xor_sum(ss, m);
    const float r = rsqrtf(ss / float(a.d) + a.eps);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = 4 * (lane + 64 * v);
      store_out4(static_cast<T*>(a.x) + base + c,
                 make_float4(hv[v].x * r * w[v].x, hv[v].y * r * w[v].y, hv[v].z * r * w[v].z, hv[v].w * r * w[v].w));
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_add_norm(AddNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const size_t base = size_t(row) * a.d;
  float ss = 0.f;
  for (int i = lane; i < a.d; i += 64) {
    float h;
    if (a.src) {
      h = to_f32(static_cast<const T*>(a.src)[base + i]);
    } else {
      h = a.h[base + i];
      if (a.add0) h += to_f32(static_cast<const T*>(a.add0)[base + i]);
      if (a.add1) h += to_f32(static_cast<const T*>(a.add1)[base + i]);
    }
    a.h[base + i] = h;
    ss = fmaf(h, h, ss);
  }
  if (!a.norm_w) return;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss = wave_xor_sum(ss, m);
  const float r = rsqrtf(ss / float(a.d) + a.eps);
  for (int i = lane; i < a.d; i += 64)
    store_out(static_cast<T*>(a.x) + base + i, a.h[base + i] * r * a.norm_w[i]);
}

// The input combinations the stack uses: decode (pre-norm of the first
// layer) with x; h plus one or two halves, with x (between layers) or without
// (after the last layer).  Any other combination takes the general kernel.
template <typename T, int NV>
static bool launch_v4(hipStream_t st, const AddNormArgs& a, dim3 grid) {
  const bool norm = a.norm_w != nullptr;
  const int nadd = (a.add0 ? 1 : 0) + (a.add1 ? 1 : 0);
  AddNormArgs b = a;
  if (!a.add0 && a.add1) {  // a single half comes first
    b.add0 = a.add1;
    b.add1 = nullptr;
  }
  if (a.src && norm) {
    hipLaunchKernelGGL((k_add_norm_v4<T, NV, true, 0, true>), grid, dim3(256), 0, st, b);
  } else if (a.src) {
    return false;
  } else if (nadd == 2) {
    if (norm) hipLaunchKernelGGL((k_add_norm_v4<T, NV, false, 2, true>), grid, dim3(256), 0, st, b);
    else hipLaunchKernelGGL((k_add_norm_v4<T, NV, false, 2, false>), grid, dim3(256), 0, st, b);
  } else if (nadd == 1) {
    if (norm) hipLaunchKernelGGL((k_add_norm_v4<T, NV, false, 1, true>), grid, dim3(256), 0, st, b);
    else hipLaunchKernelGGL((k_add_norm_v4<T, NV, false, 1, false>), grid, dim3(256), 0, st, b);
  } else {
    return false;
  }
  return true;
}

template <typename T>
static void launch_t(hipStream_t st, const AddNormArgs& a) {
  const dim3 grid((a.T + 3) / 4);
  const int nv = a.d / 256;
  if (a.d % 256 == 0 && nv >= 1 && nv <= 32) {
    bool done = false;
    switch (nv) {
      case 1: done = launch_v4<T, 1>(st, a, grid); break;
      case 2: done = launch_v4<T, 2>(st, a, grid); break;
      case 4: done = launch_v4<T, 4>(st, a, grid); break;
      case 8: done = launch_v4<T, 8>(st, a, grid); break;
      case 16: done = launch_v4<T, 16>(st, a, grid); break;
      case 20: done = launch_v4<T, 20>(st, a, grid); break;
      case 32: done = launch_v4<T, 32>(st, a, grid); break;
      default: break;
    }
    if (done) return;
  }
  hipLaunchKernelGGL((k_add_norm<T>), grid, dim3(256), 0, st, a);
}

hipError_t launch_add_norm(hipStream_t st, int dtype, const AddNormArgs& a) {
  if (dtype == 1)
    launch_t<bf16_t>(st, a);
  else
    launch_t<float>(st, a);
  return hipGetLastError();
}

}  // namespace hspec
