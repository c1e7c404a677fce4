// The Mamba-2 block around the scan (Mamba-2 as Dao & Gu describe it; H-Spec,
// Abstract, builds its drafter from Mamba-2 modules):
//
//   zxbcdt = hidden . W_in^T                  k_gemm_tn      (+ k_splitk_sum)
//   x, B, C = SiLU(causal conv4(xBC)),        k_conv_act
//   delta = softplus(dt_raw + dt_bias)
//   y = SSD scan from h0 (+ D x)               k_ssd_scan     (ssd.hip, fp32 inputs)
//   normed = RMSNorm(y * SiLU(z)) * w_norm     k_gate_norm
//   out = normed . W_out^T                     k_gemm_tn      (+ k_splitk_sum)
//
// The projections run on k_gemm_tn (gemm.hip).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace hspec {

namespace {

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + __expf(-v)); }

// log(1 + e^v); above 20 the correction is below fp32 resolution.
__device__ __forceinline__ float softplus_f(float v) { return v > 20.f ? v : log1pf(__expf(v)); }

}  // namespace

// ---------------------------------------------------------------------------
// convolution, activations and step sizes
// ---------------------------------------------------------------------------

// One thread per (request, channel): channels [0, conv_dim) are x | B | C
// (width-4 causal convolution from the block start, then SiLU); channels
// [conv_dim, conv_dim + H) are the step sizes.  Loads of one position are
// coalesced across the channels of a workgroup.
__global__ __launch_bounds__(256) void k_conv_act(ConvActArgs c) {
  const int ch = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  const int conv_dim = c.d_inner + 2 * c.ngN;
  const float* zx = c.zx + size_t(b) * c.K * c.d_proj + c.d_inner + ch;
  if (ch < conv_dim) {
    const float4 w = reinterpret_cast<const float4*>(c.conv_w)[ch];
    const float bias = c.conv_b ? c.conv_b[ch] : 0.f;
    float* dst;
    int stride;
    if (ch < c.d_inner) {
      dst = c.x + size_t(b) * c.K * c.d_inner + ch;
      stride = c.d_inner;
    } else if (ch < c.d_inner + c.ngN) {
      dst = c.B + size_t(b) * c.K * c.ngN + (ch - c.d_inner);
      stride = c.ngN;
    } else {
      dst = c.Cm + size_t(b) * c.K * c.ngN + (ch - c.d_inner - c.ngN);
      stride = c.ngN;
    }
    float x1 = 0.f, x2 = 0.f, x3 = 0.f;    // raw values 1, 2, 3 positions back
    for (int t = 0; t < c.K; ++t) {
      const float r = zx[size_t(t) * c.d_proj];
      const float v = fmaf(w.w, r, fmaf(w.z, x1, fmaf(w.y, x2, fmaf(w.x, x3, bias))));
      dst[size_t(t) * stride] = silu_f(v);
      x3 = x2;
      x2 = x1;
      x1 = r;
    }
  } else if (ch < conv_dim + c.H) {
    const int h = ch - conv_dim;
    const float bias = c.dt_bias[h];
    for (int t = 0; t < c.K; ++t)
      c.delta[(size_t(b) * c.K + t) * c.H + h] = softplus_f(zx[size_t(t) * c.d_proj] + bias);
  }
}

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

hipError_t launch_conv_act(hipStream_t st, const ConvActArgs& c) {
  const int ch = c.d_inner + 2 * c.ngN + c.H;
  hipLaunchKernelGGL(k_conv_act, dim3((ch + 255) / 256, c.C), dim3(256), 0, st, c);
  return hipGetLastError();
}

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
