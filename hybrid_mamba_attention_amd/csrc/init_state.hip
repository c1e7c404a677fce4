// a1: initial Mamba-2 state h0 = u . W_init (H-Spec, Abstract: the Mamba
// module starts from a projection of the target's last-token hidden state).
//
// A skinny GEMM: M = C requests (1..128), N = S = H*P*N state entries
// (4096..131072), K = d_model.  Every call streams all of W_init (256 MiB to
// 1.25 GiB in bf16) once, so the kernel is HBM-bound at every C and its job
// is to keep W flowing at full rate while the matrix cores do the C flops per
// weight byte.
//
// Workgroup = 64 output columns x (up to) 128 rows, 4 waves splitting the
// d_model contraction four ways and summing through LDS at the end.  Each
// lane reads 8 W rows x 4 adjacent columns per 32-deep step (16 lanes cover a
// 128-byte row segment), transposes them in registers into matrix-core B
// operands (output column n0 + 4*(lane%16) + c of MFMA c), and the u rows
// come in as A operands.  The next step's W loads are in flight while the
// current step's MFMAs run.
#include "common.h"
#include "kernels.h"

namespace hspec {

template <typename T> struct W4;
template <> struct W4<bf16_t> { uint2 v; };
template <> struct W4<float> { float4 v; };

__device__ __forceinline__ void wload(W4<bf16_t>& w, const bf16_t* p) { w.v = *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void wload(W4<float>& w, const float* p) { w.v = *reinterpret_cast<const float4*>(p); }

// B operand of output column c: element e = W[row e][column c]
__device__ __forceinline__ void wtrans(Vec8<bf16_t>& o, const W4<bf16_t> (&w)[8], int c) {
  auto el = [&](int e) -> uint32_t { return half_of(c < 2 ? w[e].v.x : w[e].v.y, c & 1); };
  o.v.x = el(0) | (el(1) << 16);
  o.v.y = el(2) | (el(3) << 16);
  o.v.z = el(4) | (el(5) << 16);
  o.v.w = el(6) | (el(7) << 16);
}
__device__ __forceinline__ void wtrans(Vec8<float>& o, const W4<float> (&w)[8], int c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = c == 0 ? w[e].v.x : c == 1 ? w[e].v.y : c == 2 ? w[e].v.z : w[e].v.w;
}

template <typename T, int MT>
__global__ __launch_bounds__(256) void k_init_state(InitArgs a) {
  const int n0 = blockIdx.x * 64;
  const int m0 = blockIdx.y * MT * 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int C = a.C, d = a.d, S = a.S;
  const T* __restrict__ u = static_cast<const T*>(a.u);
  const T* __restrict__ W = static_cast<const T*>(a.w);

  f32x4 acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = d >> 5;
  const T* wcol = W + n0 + li * 4;
  W4<T> cur[8], nxt[8];
  if (wave < nk) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wload(cur[e], wcol + size_t(wave * 32 + lg * 8 + e) * S);
  }
  for (int ks = wave; ks < nk; ks += 4) {
    const int kn = ks + 4;
    if (kn < nk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wload(nxt[e], wcol + size_t(kn * 32 + lg * 8 + e) * S);
    }
    Vec8<T> bop[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) wtrans(bop[c], cur, c);
    const int kb = ks * 32 + lg * 8;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int row = m0 + m * 16 + li;
      Vec8<T> aop;
      if (row < C)
        load8(aop, u + size_t(row) * d + kb);
      else
        zero8(aop);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[m][c] = mma8(aop, bop[c], acc[m][c]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) cur[e] = nxt[e];
  }

  // sum the four waves' partial tiles: 3 -> 1, 2 -> 0, then 1 -> 0
  __shared__ float4 red[2][MT * 4 * 64];
  if (wave >= 2) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = acc[m][c];
        red[wave - 2][(m * 4 + c) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = red[wave][(m * 4 + c) * 64 + lane];
        acc[m][c] += f32x4{v.x, v.y, v.z, v.w};
      }
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = acc[m][c];
        red[0][(m * 4 + c) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v = red[0][(m * 4 + c) * 64 + lane];
      acc[m][c] += f32x4{v.x, v.y, v.z, v.w};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + m * 16 + 4 * lg + r;
      if (row < C)
        *reinterpret_cast<float4*>(a.h0 + size_t(row) * S + n0 + li * 4) =
            make_float4(acc[m][0][r], acc[m][1][r], acc[m][2][r], acc[m][3][r]);
    }
  }
}

template <typename T>
static hipError_t launch_init_t(hipStream_t st, const InitArgs& a) {
  const dim3 block(256);
  if (a.C <= 16) {
    hipLaunchKernelGGL((k_init_state<T, 1>), dim3(a.S / 64, 1), block, 0, st, a);
  } else if (a.C <= 32) {
    hipLaunchKernelGGL((k_init_state<T, 2>), dim3(a.S / 64, 1), block, 0, st, a);
  } else if (a.C <= 64) {
    hipLaunchKernelGGL((k_init_state<T, 4>), dim3(a.S / 64, 1), block, 0, st, a);
  } else {
    hipLaunchKernelGGL((k_init_state<T, 8>), dim3(a.S / 64, (a.C + 127) / 128), block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_init_state(hipStream_t st, int dtype, const InitArgs& a) {
  return dtype == 1 ? launch_init_t<bf16_t>(st, a) : launch_init_t<float>(st, a);
}

}  // namespace hspec
