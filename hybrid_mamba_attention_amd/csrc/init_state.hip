// a1: initial Mamba-2 state h0 = u . W_init (H-Spec, Abstract: the Mamba
// module starts from a projection of the target's last-token hidden state).
//
// A skinny GEMM: M = C requests (1..128), N = S = H*P*N state entries
// (4096..131072), K = d_model.  Every call streams all of W_init (256 MiB to
// 1.25 GiB in bf16) once, so the kernel is HBM-bound at every C: its job is
// to keep enough W bytes in flight while the matrix cores do C flops per
// weight element.
//
// Workgroup = 16*NCL output columns x (up to) 16*MT rows; its 4 waves split
// the d_model contraction four ways (k-steps of 32 rows dealt round-robin)
// and sum their tiles through LDS at the end.  Per k-step a lane reads 8 W
// rows x NCL adjacent columns (16 lanes cover one 16*NCL-column row segment)
// off a scalar column base, transposes them in registers into NCL matrix-core
// B operands (output column n0 + NCL*(lane%16) + c of MFMA c), and takes its
// u rows as A operands.  PF k-steps of W are kept in flight per wave.
#include "common.h"
#include "kernels.h"

namespace hspec {

template <typename T, int NCL> struct WRow;  // NCL adjacent W elements of one row
template <> struct WRow<bf16_t, 4> { uint2 v; };
template <> struct WRow<bf16_t, 8> { uint4 v; };
template <> struct WRow<float, 4> { float4 v; };

__device__ __forceinline__ void wload(WRow<bf16_t, 4>& w, const char* p) { w.v = *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void wload(WRow<bf16_t, 8>& w, const char* p) { w.v = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void wload(WRow<float, 4>& w, const char* p) { w.v = *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ uint32_t wdw(const WRow<bf16_t, 4>& w, int i) { return i ? w.v.y : w.v.x; }
__device__ __forceinline__ uint32_t wdw(const WRow<bf16_t, 8>& w, int i) { return dword_of(w.v, i); }

// B operand of column c of the lane's group: element e = W[row e][column c]
template <int NCL>
__device__ __forceinline__ void wtrans(Vec8<bf16_t>& o, const WRow<bf16_t, NCL> (&w)[8], int c) {
  const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
  const int d = c >> 1;
  o.v.x = __builtin_amdgcn_perm(wdw(w[1], d), wdw(w[0], d), sel);
  o.v.y = __builtin_amdgcn_perm(wdw(w[3], d), wdw(w[2], d), sel);
  o.v.z = __builtin_amdgcn_perm(wdw(w[5], d), wdw(w[4], d), sel);
  o.v.w = __builtin_amdgcn_perm(wdw(w[7], d), wdw(w[6], d), sel);
}
template <int NCL>
__device__ __forceinline__ void wtrans(Vec8<float>& o, const WRow<float, NCL> (&w)[8], int c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = c == 0 ? w[e].v.x : c == 1 ? w[e].v.y : c == 2 ? w[e].v.z : w[e].v.w;
}

template <typename T, int MT, int NCL, int PF>
__global__ __launch_bounds__(256) void k_init_state(InitArgs a) {
  constexpr int NC = 16 * NCL;
  static_assert(PF % 2 == 0, "even depth keeps the A-operand double buffer parity static");
  const int n0 = blockIdx.x * NC;
  const int m0 = blockIdx.y * MT * 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int C = a.C, d = a.d, S = a.S;
  const T* __restrict__ u = static_cast<const T*>(a.u);
  const char* __restrict__ wcol = static_cast<const char*>(a.w) + size_t(n0) * sizeof(T);
  const size_t kstep_b = size_t(32) * S * sizeof(T);  // bytes between consecutive k-steps

  f32x4 acc[MT][NCL];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < NCL; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane's 8 rows of a k-step, as byte offsets from the k-step's first row
  uint32_t roff[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) roff[e] = uint32_t((lg * 8 + e) * S + li * NCL) * sizeof(T);

  const int nk = d >> 5;
  const int nmine = nk > wave ? (nk - wave + 3) >> 2 : 0;  // k-steps wave, wave+4, ...
  WRow<T, NCL> ring[PF][8];
  auto issue = [&](int i, WRow<T, NCL> (&dst)[8]) __attribute__((always_inline)) {
    const char* base = wcol + size_t(wave + 4 * i) * kstep_b;
#pragma unroll
    for (int e = 0; e < 8; ++e) wload(dst[e], base + roff[e]);
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < nmine) issue(p, ring[p]);

  // A operands (u rows) run one k-step ahead of their MFMAs: they come from
  // L2, and at one wave per SIMD nothing else would hide that latency.
  auto load_a = [&](int i, Vec8<T> (&dst)[MT]) __attribute__((always_inline)) {
    const int kb = (wave + 4 * i) * 32 + lg * 8;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int row = m0 + m * 16 + li;
      if (row < C)
        load8(dst[m], u + size_t(row) * d + kb);
      else
        zero8(dst[m]);
    }
  };
  Vec8<T> aop[2][MT];
  if (nmine > 0) load_a(0, aop[0]);
  for (int i0 = 0; i0 < nmine; i0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int i = i0 + p;
      if (i < nmine) {
        Vec8<T> bop[NCL];
#pragma unroll
        for (int c = 0; c < NCL; ++c) wtrans<NCL>(bop[c], ring[p], c);
        if (i + PF < nmine) issue(i + PF, ring[p]);
        if (i + 1 < nmine) load_a(i + 1, aop[(p + 1) & 1]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int c = 0; c < NCL; ++c) acc[m][c] = mma8(aop[p & 1][m], bop[c], acc[m][c]);
      }
    }
  }

  // sum the four waves' partial tiles: 3 -> 1, 2 -> 0, then 1 -> 0
  __shared__ float4 red[2][MT * NCL * 64];
  if (wave >= 2) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const f32x4 v = acc[m][c];
        red[wave - 2][(m * NCL + c) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const float4 v = red[wave][(m * NCL + c) * 64 + lane];
        acc[m][c] += f32x4{v.x, v.y, v.z, v.w};
      }
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const f32x4 v = acc[m][c];
        red[0][(m * NCL + c) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      const float4 v = red[0][(m * NCL + c) * 64 + lane];
      acc[m][c] += f32x4{v.x, v.y, v.z, v.w};
    }
    // lane holds rows 4*lg + r of m-tile m, columns n0 + NCL*li + c
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + m * 16 + 4 * lg + r;
      if (row < C) {
        float* dst = a.h0 + size_t(row) * S + n0 + li * NCL;
#pragma unroll
        for (int c = 0; c < NCL; c += 4)
          *reinterpret_cast<float4*>(dst + c) =
              make_float4(acc[m][c][r], acc[m][c + 1][r], acc[m][c + 2][r], acc[m][c + 3][r]);
      }
    }
  }
}

template <typename T, int MT, int NCL, int PF>
static hipError_t launch_cfg(hipStream_t st, const InitArgs& a) {
  const int mblocks = (a.C + MT * 16 - 1) / (MT * 16);
  hipLaunchKernelGGL((k_init_state<T, MT, NCL, PF>), dim3(a.S / (16 * NCL), mblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_init_state(hipStream_t st, int dtype, const InitArgs& a) {
  if (dtype == 1) {
    if (a.C <= 16) return launch_cfg<bf16_t, 1, 4, 8>(st, a);
    if (a.C <= 32) return launch_cfg<bf16_t, 2, 4, 8>(st, a);
    if (a.C <= 64) return launch_cfg<bf16_t, 4, 4, 6>(st, a);
    return launch_cfg<bf16_t, 8, 4, 4>(st, a);
  }
  if (a.C <= 16) return launch_cfg<float, 1, 4, 4>(st, a);
  if (a.C <= 32) return launch_cfg<float, 2, 4, 4>(st, a);
  if (a.C <= 64) return launch_cfg<float, 4, 4, 2>(st, a);
  return launch_cfg<float, 8, 4, 2>(st, a);
}

}  // namespace hspec
