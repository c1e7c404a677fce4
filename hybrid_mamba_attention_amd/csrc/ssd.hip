// a2: Mamba-2 (SSD) chunked parallel scan over the K-token draft block.
//
// H-Spec (Abstract): despite being a recurrence, the Mamba module drafts the
// whole block in parallel through its parallel scan.  The arithmetic is the
// Mamba-2 SSD layer (Dao & Gu 2024, chunked form): for each chunk of Q
// positions,
//   lam_t   = sum_{r = chunk start .. t} delta_r * A         (wave scan)
//   M[t,s]  = exp(lam_t - lam_s) * (Cm_t . B_s) * delta_s    for s <= t, else 0
//   y_t     = sum_s M[t,s] x_s + exp(lam_t) * H_in Cm_t (+ Dskip x_t)
//   H_out   = exp(lam_end) H_in + sum_s exp(lam_end - lam_s) delta_s x_s (outer) B_s
// with H_in of the first chunk = h0, the projected last-token state.
//
// One workgroup of ceil(P/64) waves per (request, head).  Thread p owns state
// row H[p][0..N) in registers for the whole block, so the state never leaves
// registers between chunks; the chunk's B and Cm rows, the decay-weighted
// C.B^T matrix M and the cumulative log-decays sit in LDS and are read as
// broadcasts (every lane reads the same address).  The cumulative sum runs
// across one wave's lanes with shuffles.  Memory traffic per (request, head):
// h0 in (P*N fp32), x/B/Cm in, y out (and h_final when asked for).
#include "common.h"
#include "kernels.h"

namespace hspec {

template <typename T, int NB, int QB>
__global__ __launch_bounds__(128) void k_ssd_scan(SsdArgs a) {
  const int H = a.H, P = a.P, N = a.N, K = a.K, Q = a.chunk;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int grp = h / (H / a.ng);
  const int tid = threadIdx.x;
  const int p = tid;  // owned state row
  const bool own = p < P;

  constexpr int NBS = NB + 1;  // padded B/Cm rows: the C.B^T products read rows across lanes
  __shared__ float sB[QB * NBS], sC[QB * NBS], sM[QB * QB], slam[QB], sw[QB], sdt[QB];

  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ Bm = static_cast<const T*>(a.B);
  const T* __restrict__ Cm = static_cast<const T*>(a.Cm);
  const float Ah = a.A[h];
  const float Dh = a.Dskip ? a.Dskip[h] : 0.f;

  float Hs[NB];
  {
    const float* h0 = a.h0 ? a.h0 + ((size_t(b) * H + h) * P + p) * N : nullptr;
#pragma unroll
    for (int n = 0; n < NB; ++n) Hs[n] = (own && h0 && n < N) ? h0[n] : 0.f;
  }

  for (int c0 = 0; c0 < K; c0 += Q) {
    const int q = min(Q, K - c0);
    // the chunk's B and Cm rows (fp32), shared by all heads of the group
    for (int i = tid; i < q * N; i += blockDim.x) {
      const int t = i / N, n = i % N;
      const size_t src = ((size_t(b) * K + c0 + t) * a.ng + grp) * N + n;
      sB[t * NBS + n] = to_f32(Bm[src]);
      sC[t * NBS + n] = to_f32(Cm[src]);
    }
    if (tid < 64) {
      // in-chunk cumulative log-decay: inclusive scan across the wave's lanes
      const float dt = tid < q ? a.delta[(size_t(b) * K + c0 + tid) * H + h] : 0.f;
      float v = dt * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_up(v, off, 64);
        if (tid >= off) v += u;
      }
      const float lend = __shfl(v, q - 1, 64);
      if (tid < q) {
        slam[tid] = v;
        sdt[tid] = dt;
        sw[tid] = __expf(lend - v) * dt;
      }
    }
    // this thread's x values of the chunk
    float xs[QB];
#pragma unroll
    for (int s = 0; s < QB; ++s)
      xs[s] = (own && s < q) ? to_f32(x[((size_t(b) * K + c0 + s) * H + h) * P + p]) : 0.f;
    __syncthreads();
    // decay-weighted C.B^T, masked before the exponential
    for (int i = tid; i < q * q; i += blockDim.x) {
      const int t = i / q, s = i % q;
      float v = 0.f;
      if (s <= t) {
        float dot = 0.f;
        for (int n = 0; n < N; ++n) dot = fmaf(sC[t * NBS + n], sB[s * NBS + n], dot);
        v = __expf(slam[t] - slam[s]) * dot * sdt[s];
      }
      sM[t * QB + s] = v;
    }
    __syncthreads();
    if (own) {
      // outputs of the chunk: y[t][p]
      for (int t = 0; t < q; ++t) {
        float yd = 0.f, xt = 0.f;  // (register arrays are only indexed by unrolled constants)
#pragma unroll
        for (int s = 0; s < QB; ++s) {
          if (s <= t) yd = fmaf(sM[t * QB + s], xs[s], yd);
          if (s == t) xt = xs[s];
        }
        float yo = 0.f;
#pragma unroll
        for (int n = 0; n < NB; ++n)
          if (n < N) yo = fmaf(Hs[n], sC[t * NBS + n], yo);
        a.y[((size_t(b) * K + c0 + t) * H + h) * P + p] = yd + __expf(slam[t]) * yo + Dh * xt;
      }
      // state passing to the next chunk
      const float dend = __expf(slam[q - 1]);
#pragma unroll
      for (int n = 0; n < NB; ++n) Hs[n] *= dend;
#pragma unroll
      for (int s = 0; s < QB; ++s) {
        if (s < q) {
          const float coef = sw[s] * xs[s];
#pragma unroll
          for (int n = 0; n < NB; ++n)
            if (n < N) Hs[n] = fmaf(coef, sB[s * NBS + n], Hs[n]);
        }
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }
  if (a.h_final && own) {
    float* hf = a.h_final + ((size_t(b) * H + h) * P + p) * N;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      if (n < N) hf[n] = Hs[n];
  }
}

// Static LDS of the instantiation a shape selects (chunks of up to 16).
size_t ssd_lds_bytes(int P, int N, int Q) {
  (void)P;
  (void)Q;
  const int nb = N <= 16 ? 16 : N <= 32 ? 32 : N <= 64 ? 64 : 128;
  constexpr int qb = 16;
  return (size_t(2) * qb * (nb + 1) + size_t(qb) * qb + 3 * qb) * sizeof(float);
}

template <typename T, int NB, int QB>
static hipError_t launch_nq(hipStream_t st, const SsdArgs& a) {
  const int threads = a.P <= 64 ? 64 : 128;
  hipLaunchKernelGGL((k_ssd_scan<T, NB, QB>), dim3(a.C * a.H), dim3(threads), 0, st, a);
  return hipGetLastError();
}

template <typename T, int NB>
static hipError_t launch_n(hipStream_t st, const SsdArgs& a) {
  return launch_nq<T, NB, 16>(st, a);  // chunks above 16 are refused by validation
}

template <typename T>
static hipError_t launch_t(hipStream_t st, const SsdArgs& a) {
  if (a.N <= 16) return launch_n<T, 16>(st, a);
  if (a.N <= 32) return launch_n<T, 32>(st, a);
  if (a.N <= 64) return launch_n<T, 64>(st, a);
  return launch_n<T, 128>(st, a);
}

hipError_t launch_ssd_scan(hipStream_t st, int dtype, const SsdArgs& a) {
  return dtype == 1 ? launch_t<bf16_t>(st, a) : launch_t<float>(st, a);
}

}  // namespace hspec
