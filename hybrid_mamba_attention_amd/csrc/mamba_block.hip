// The Mamba-2 block around the scan (Mamba-2 as Dao & Gu describe it; H-Spec,
// Abstract, builds its drafter from Mamba-2 modules):
//
//   zxbcdt = hidden . W_in^T                  k_gemm_tn      (+ k_splitk_sum)
//   x, B, C = SiLU(causal conv4(xBC)),        k_ssd_scan     (ssd.hip: the scan reads the
//   delta = softplus(dt_raw + dt_bias),                       raw rows and applies the
//   y = SSD scan from h0 (+ D x)                              convolution in its loads)
//   normed = RMSNorm(y * SiLU(z)) * w_norm     k_gate_norm
//   out = normed . W_out^T                     k_gemm_tn      (+ k_splitk_sum)
//
// The projections run on k_gemm_tn (gemm.hip).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace hspec {

// ---------------------------------------------------------------------------
// gated RMS normalisation
// ---------------------------------------------------------------------------

// One wave per token row: g = y * SiLU(z), normed = g / sqrt(mean(g^2) + eps) * w.
template <typename OutT>
__global__ __launch_bounds__(256) void k_gate_norm(GateNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const float* y = a.y + size_t(row) * a.d_inner;
  const float* z = a.zx + size_t(row) * a.d_proj;
  float ss = 0.f;
  for (int i = lane; i < a.d_inner; i += 64) {
    const float gv = y[i] * silu_f(z[i]);
    ss = fmaf(gv, gv, ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss = wave_xor_sum(ss, m);
  const float r = rsqrtf(ss / float(a.d_inner) + a.eps);
  OutT* o = static_cast<OutT*>(a.out) + size_t(row) * a.d_inner;
  for (int i = lane; i < a.d_inner; i += 64) store_out(o + i, y[i] * silu_f(z[i]) * r * a.norm_w[i]);
}

// The same with d_inner = 256*NV and 16-byte rows: lane l holds the four
// channels 4*(l + 64*v) .. +3 for v < NV, so y and z are read once, as float4.
template <typename OutT, int NV>
__global__ __launch_bounds__(256) void k_gate_norm_v4(GateNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const float4* y = reinterpret_cast<const float4*>(a.y + size_t(row) * a.d_inner);
  const float4* z = reinterpret_cast<const float4*>(a.zx + size_t(row) * a.d_proj);
  float4 gv[NV];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const float4 yv = y[lane + 64 * v], zv = z[lane + 64 * v];
    gv[v] = make_float4(yv.x * silu_f(zv.x), yv.y * silu_f(zv.y), yv.z * silu_f(zv.z), yv.w * silu_f(zv.w));
    ss = fmaf(gv[v].x, gv[v].x, fmaf(gv[v].y, gv[v].y, fmaf(gv[v].z, gv[v].z, fmaf(gv[v].w, gv[v].w, ss))));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss = wave_xor_sum(ss, m);
  const float r = rsqrtf(ss / float(a.d_inner) + a.eps);
  const float4* w = reinterpret_cast<const float4*>(a.norm_w);
  OutT* o = static_cast<OutT*>(a.out) + size_t(row) * a.d_inner;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int c = 4 * (lane + 64 * v);
    const float4 wv = w[lane + 64 * v];
    store_out4(o + c, make_float4(gv[v].x * r * wv.x, gv[v].y * r * wv.y, gv[v].z * r * wv.z,
                                  gv[v].w * r * wv.w));
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <int NV>
static void launch_gate_norm_v4(hipStream_t st, int dtype, const GateNormArgs& a, dim3 grid) {
  if (dtype == 1)
    hipLaunchKernelGGL((k_gate_norm_v4<bf16_t, NV>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gate_norm_v4<float, NV>), grid, dim3(256), 0, st, a);
}

hipError_t launch_gate_norm(hipStream_t st, int dtype, const GateNormArgs& a) {
  const dim3 grid((a.T + 3) / 4);
  const int nv = a.d_inner / 256;
  const bool v4 = a.d_inner % 256 == 0 && a.d_proj % 4 == 0 && (nv == 1 || nv == 2 || nv == 4 || nv == 8);
  if (v4) {
    switch (nv) {
      case 1: launch_gate_norm_v4<1>(st, dtype, a, grid); break;
      case 2: launch_gate_norm_v4<2>(st, dtype, a, grid); break;
      case 4: launch_gate_norm_v4<4>(st, dtype, a, grid); break;
      default: launch_gate_norm_v4<8>(st, dtype, a, grid); break;
    }
  } else if (dtype == 1) {
    hipLaunchKernelGGL((k_gate_norm<bf16_t>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_gate_norm<float>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hspec
