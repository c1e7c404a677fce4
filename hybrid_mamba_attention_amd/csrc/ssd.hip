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
// One workgroup per (request, head); the state, the chunk's x/B/Cm and the
// decay matrix live in LDS; the cumulative sum runs on one wave's lanes with
// shuffles.  The scan is small next to the KV read: it moves h0 in (P*N fp32)
// and y out.
#include "common.h"
#include "kernels.h"

namespace hspec {

struct SsdLds {
  int P, N, Q;
  int hs() const { return N + 1; }  // padded state row (bank spread)
  size_t floats() const {
    return size_t(P) * hs() + size_t(Q) * P + 2 * size_t(Q) * N + size_t(Q) * Q + 2 * size_t(Q) + 64;
  }
};

template <typename T>
__global__ __launch_bounds__(256) void k_ssd_scan(SsdArgs a) {
  const int H = a.H, P = a.P, N = a.N, K = a.K, Q = a.chunk;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int grp = h / (H / a.ng);
  const int tid = threadIdx.x;
  const int HS = N + 1;

  extern __shared__ __align__(16) float sm[];
  float* sH = sm;                      // [P][N+1]
  float* sx = sH + P * HS;             // [Q][P]
  float* sB = sx + Q * P;              // [Q][N]
  float* sC = sB + Q * N;              // [Q][N]
  float* sM = sC + Q * N;              // [Q][Q]
  float* slam = sM + Q * Q;            // [Q]
  float* sw = slam + Q;                // [Q]  exp(lam_end - lam_s) * delta_s
  float* sdt = sw + Q;                 // [64] delta of the chunk

  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ Bm = static_cast<const T*>(a.B);
  const T* __restrict__ Cm = static_cast<const T*>(a.Cm);
  const float Ah = a.A[h];
  const float Dh = a.Dskip ? a.Dskip[h] : 0.f;

  for (int i = tid; i < P * N; i += 256) {
    const int p = i / N, n = i % N;
    sH[p * HS + n] = a.h0 ? a.h0[(size_t(b) * H + h) * P * N + i] : 0.f;
  }

  for (int c0 = 0; c0 < K; c0 += Q) {
    const int q = min(Q, K - c0);
    for (int i = tid; i < q * P; i += 256) {
      const int t = i / P, p = i % P;
      sx[i] = to_f32(x[((size_t(b) * K + c0 + t) * H + h) * P + p]);
    }
    for (int i = tid; i < q * N; i += 256) {
      const int t = i / N, n = i % N;
      const size_t src = ((size_t(b) * K + c0 + t) * a.ng + grp) * N + n;
      sB[i] = to_f32(Bm[src]);
      sC[i] = to_f32(Cm[src]);
    }
    if (tid < 64) {
      // in-chunk cumulative log-decay by a wave-wide inclusive scan
      const float dt = tid < q ? a.delta[(size_t(b) * K + c0 + tid) * H + h] : 0.f;
      float v = dt * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_up(v, off, 64);
        if (tid >= off) v += u;
      }
      if (tid < q) {
        slam[tid] = v;
        sdt[tid] = dt;
      }
      const float lend = __shfl(v, q - 1, 64);
      if (tid < q) sw[tid] = __expf(lend - v) * dt;
    }
    __syncthreads();
    // decay-weighted C.B^T (the segsum matrix), masked before the exponential
    for (int i = tid; i < q * q; i += 256) {
      const int t = i / q, s = i % q;
      float v = 0.f;
      if (s <= t) {
        float dot = 0.f;
        for (int n = 0; n < N; ++n) dot = fmaf(sC[t * N + n], sB[s * N + n], dot);
        v = __expf(slam[t] - slam[s]) * dot * sdt[s];
      }
      sM[t * Q + s] = v;
    }
    __syncthreads();
    // outputs of the chunk
    for (int i = tid; i < q * P; i += 256) {
      const int t = i / P, p = i % P;
      float yd = 0.f;
      for (int s = 0; s <= t; ++s) yd = fmaf(sM[t * Q + s], sx[s * P + p], yd);
      float yo = 0.f;
      for (int n = 0; n < N; ++n) yo = fmaf(sH[p * HS + n], sC[t * N + n], yo);
      const float yv = yd + __expf(slam[t]) * yo + Dh * sx[t * P + p];
      a.y[((size_t(b) * K + c0 + t) * H + h) * P + p] = yv;
    }
    __syncthreads();
    // state passing to the next chunk
    const float dend = __expf(slam[q - 1]);
    for (int i = tid; i < P * N; i += 256) {
      const int p = i / N, n = i % N;
      float acc = dend * sH[p * HS + n];
      for (int s = 0; s < q; ++s) acc = fmaf(sw[s] * sx[s * P + p], sB[s * N + n], acc);
      sH[p * HS + n] = acc;
    }
    __syncthreads();
  }
  if (a.h_final) {
    for (int i = tid; i < P * N; i += 256) {
      const int p = i / N, n = i % N;
      a.h_final[(size_t(b) * H + h) * P * N + i] = sH[p * HS + n];
    }
  }
}

size_t ssd_lds_bytes(int P, int N, int Q) { return SsdLds{P, N, Q}.floats() * sizeof(float); }

hipError_t launch_ssd_scan(hipStream_t st, int dtype, const SsdArgs& a) {
  const size_t lds = ssd_lds_bytes(a.P, a.N, a.chunk);
  const void* kern = dtype == 1 ? reinterpret_cast<const void*>(k_ssd_scan<bf16_t>)
                                : reinterpret_cast<const void*>(k_ssd_scan<float>);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  if (dtype == 1)
    hipLaunchKernelGGL(k_ssd_scan<bf16_t>, dim3(a.C * a.H), dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL(k_ssd_scan<float>, dim3(a.C * a.H), dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace hspec
