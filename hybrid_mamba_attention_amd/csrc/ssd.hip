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
// One workgroup per (request, head).  The state lives in registers for the
// whole block: N/8 waves per 64 state rows, each holding 8 columns of every
// row, and every thread keeps one accumulator per chunk position for its
// outputs (no serial reduction chains).  The chunk's B and
// Cm rows, the decay-weighted C.B^T matrix M and the cumulative log-decays sit
// in LDS and are read as float4 broadcasts.  The cumulative sum runs across
// one wave's lanes with shuffles.  Memory traffic per (request, head):
// h0 in (P*N fp32), x/B/Cm in, y out (and h_final when asked for).
#include "common.h"
#include "kernels.h"

namespace hspec {

// Workgroup: NWQ = NB/8 waves per 64 state rows (at most 16 waves, since
// P*N <= 8192).  Wave w (nq = w % NWQ, row block rb = w / NWQ) owns columns
// [8*nq, 8*nq + 8) of rows rb*64 + lane, so every LDS operand a wave reads is
// the same address in all its lanes (a broadcast) and per-thread registers
// stay small for every state size.  The waves' partial outputs meet in LDS.
template <int NWQ> struct SsdLayout {
  static constexpr int NB = 8 * NWQ, QB = 16;
  // dynamic LDS, in floats
  static constexpr int oB = 0;                       // sB[QB][NB]   B rows by position
  static constexpr int oCT = oB + QB * NB;           // sCT[NB][QB]  Cm, position-minor
  static constexpr int oMT = oCT + NB * QB;          // sMT[QB][QB]  M[t][s] at [s][t]
  static constexpr int oLam = oMT + QB * QB;         // lam[QB], w[QB], dt[QB], pad
  static constexpr int oX = oLam + 4 * QB;           // sX[RB][QB][64]
  static size_t floats(int RB) { return size_t(oX) + size_t(RB) * QB * 64 + size_t(RB) * NWQ * QB * 64; }
};

template <typename T, int NWQ>
__global__ __launch_bounds__(1024) void k_ssd_scan(SsdArgs a) {
  using L = SsdLayout<NWQ>;
  constexpr int NB = L::NB, QB = L::QB, NQ = 8;
  const int H = a.H, P = a.P, N = a.N, K = a.K, Q = a.chunk;
  const int RB = (P + 63) >> 6;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int grp = h / (H / a.ng);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nq = wave % NWQ, rb = wave / NWQ;
  const int p = rb * 64 + lane;  // state row
  const bool own = p < P;
  const int n0 = nq * NQ;        // first owned column

  extern __shared__ __align__(16) float lds[];
  float* sB = lds + L::oB;
  float* sCT = lds + L::oCT;
  float* sMT = lds + L::oMT;
  float* slam = lds + L::oLam;
  float* sw = slam + QB;
  float* sdt = sw + QB;
  float* sX = lds + L::oX;                              // [RB][QB][64]
  float* sZ = sX + size_t(RB) * QB * 64;                // [RB][NWQ][QB][64]

  const T* __restrict__ Bm = static_cast<const T*>(a.B);
  const T* __restrict__ Cm = static_cast<const T*>(a.Cm);
  const float Ah = a.A[h];
  const float Dh = a.Dskip ? a.Dskip[h] : 0.f;
  // per-position rows as uniform bases + the lane's row p
  const size_t HP = size_t(H) * P;
  const T* __restrict__ xrow = static_cast<const T*>(a.x) + (size_t(b) * K * H + h) * P;
  float* __restrict__ yrow = a.y + (size_t(b) * K * H + h) * P;

  float Hs[NQ];
  {
    const float* h0 = (a.h0 && own) ? a.h0 + ((size_t(b) * H + h) * P + p) * N + n0 : nullptr;
    if (h0 && n0 + NQ <= N && (N & 3) == 0) {
      const float4 v0 = reinterpret_cast<const float4*>(h0)[0];
      const float4 v1 = reinterpret_cast<const float4*>(h0)[1];
      Hs[0] = v0.x; Hs[1] = v0.y; Hs[2] = v0.z; Hs[3] = v0.w;
      Hs[4] = v1.x; Hs[5] = v1.y; Hs[6] = v1.z; Hs[7] = v1.w;
    } else {
#pragma unroll
      for (int k = 0; k < NQ; ++k) Hs[k] = (h0 && n0 + k < N) ? h0[k] : 0.f;
    }
  }

  for (int c0 = 0; c0 < K; c0 += Q) {
    const int q = min(Q, K - c0);
    for (int i = tid; i < QB * NB; i += blockDim.x) {
      const int t = i / NB, n = i % NB;
      float bv = 0.f, cv = 0.f;
      if (t < q && n < N) {
        const size_t src = ((size_t(b) * K + c0 + t) * a.ng + grp) * N + n;
        bv = to_f32(Bm[src]);
        cv = to_f32(Cm[src]);
      }
      sB[t * NB + n] = bv;
      sCT[n * QB + t] = cv;
    }
    if (nq == 0) {  // one wave per row block brings the chunk's x of its rows
#pragma unroll
      for (int s = 0; s < QB; ++s)
        sX[(rb * QB + s) * 64 + lane] = (own && s < q) ? to_f32(xrow[size_t(c0 + s) * HP + p]) : 0.f;
    }
    if (wave == 0) {
      // in-chunk cumulative log-decay: inclusive scan across the wave's lanes
      const float dt = lane < q ? a.delta[(size_t(b) * K + c0 + lane) * H + h] : 0.f;
      float v = dt * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
      }
      const float lend = __shfl(v, q - 1, 64);
      if (lane < QB) {
        slam[lane] = v;
        sdt[lane] = dt;
        sw[lane] = lane < q ? __expf(lend - v) * dt : 0.f;
      }
    }
    __syncthreads();
    // decay-weighted C.B^T, masked before the exponential: M[t][s] -> sMT[s][t]
    for (int i = tid; i < QB * QB; i += blockDim.x) {
      const int t = i % QB, s = i / QB;
      float v = 0.f;
      if (s <= t && t < q) {
        float d0 = 0.f, d1 = 0.f;
        for (int n = 0; n + 1 < N; n += 2) {
          d0 = fmaf(sCT[n * QB + t], sB[s * NB + n], d0);
          d1 = fmaf(sCT[(n + 1) * QB + t], sB[s * NB + n + 1], d1);
        }
        if (N & 1) d0 = fmaf(sCT[(N - 1) * QB + t], sB[s * NB + N - 1], d0);
        v = __expf(slam[t] - slam[s]) * (d0 + d1) * sdt[s];
      }
      sMT[s * QB + t] = v;
    }
    __syncthreads();
    // this wave's share of y[t][p]: owned columns for the state term,
    // positions s = nq, nq + NWQ, ... for the in-chunk term
    float z[QB];
#pragma unroll
    for (int t = 0; t < QB; ++t) z[t] = 0.f;
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const float hk = Hs[k];
#pragma unroll
      for (int t = 0; t < QB; t += 4) {
        const float4 c = *reinterpret_cast<const float4*>(sCT + (n0 + k) * QB + t);
        z[t] = fmaf(hk, c.x, z[t]);
        z[t + 1] = fmaf(hk, c.y, z[t + 1]);
        z[t + 2] = fmaf(hk, c.z, z[t + 2]);
        z[t + 3] = fmaf(hk, c.w, z[t + 3]);
      }
    }
#pragma unroll
    for (int t = 0; t < QB; ++t) z[t] *= __expf(slam[t]);
    for (int s = nq; s < QB; s += NWQ) {
      const float xv = sX[(rb * QB + s) * 64 + lane];
#pragma unroll
      for (int t = 0; t < QB; t += 4) {
        const float4 m = *reinterpret_cast<const float4*>(sMT + s * QB + t);
        z[t] = fmaf(m.x, xv, z[t]);
        z[t + 1] = fmaf(m.y, xv, z[t + 1]);
        z[t + 2] = fmaf(m.z, xv, z[t + 2]);
        z[t + 3] = fmaf(m.w, xv, z[t + 3]);
      }
    }
    float* zs = sZ + (size_t(rb) * NWQ + nq) * QB * 64 + lane;
#pragma unroll
    for (int t = 0; t < QB; ++t) zs[t * 64] = z[t];
    // state passing to the next chunk (owned columns)
    const float dend = __expf(slam[q - 1]);
#pragma unroll
    for (int k = 0; k < NQ; ++k) Hs[k] *= dend;
    for (int s = 0; s < q; ++s) {
      const float coef = sw[s] * sX[(rb * QB + s) * 64 + lane];
      const float4 b0 = *reinterpret_cast<const float4*>(sB + s * NB + n0);
      const float4 b1 = *reinterpret_cast<const float4*>(sB + s * NB + n0 + 4);
      Hs[0] = fmaf(coef, b0.x, Hs[0]); Hs[1] = fmaf(coef, b0.y, Hs[1]);
      Hs[2] = fmaf(coef, b0.z, Hs[2]); Hs[3] = fmaf(coef, b0.w, Hs[3]);
      Hs[4] = fmaf(coef, b1.x, Hs[4]); Hs[5] = fmaf(coef, b1.y, Hs[5]);
      Hs[6] = fmaf(coef, b1.z, Hs[6]); Hs[7] = fmaf(coef, b1.w, Hs[7]);
    }
    __syncthreads();
    // sum the waves' shares: wave nq writes positions t = nq, nq + NWQ, ...
    if (own) {
      for (int t = nq; t < q; t += NWQ) {
        const float* zr = sZ + size_t(rb) * NWQ * QB * 64 + t * 64 + lane;
        float yv = 0.f;
#pragma unroll
        for (int w = 0; w < NWQ; ++w) yv += zr[w * QB * 64];
        yrow[size_t(c0 + t) * HP + p] = yv + Dh * sX[(rb * QB + t) * 64 + lane];
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }
  if (a.h_final && own) {
    float* hf = a.h_final + ((size_t(b) * H + h) * P + p) * N + n0;
    if (n0 + NQ <= N && (N & 3) == 0) {
      reinterpret_cast<float4*>(hf)[0] = make_float4(Hs[0], Hs[1], Hs[2], Hs[3]);
      reinterpret_cast<float4*>(hf)[1] = make_float4(Hs[4], Hs[5], Hs[6], Hs[7]);
    } else {
#pragma unroll
      for (int k = 0; k < NQ; ++k)
        if (n0 + k < N) hf[k] = Hs[k];
    }
  }
}

static int nwq_for(int N) { return N <= 16 ? 2 : N <= 32 ? 4 : N <= 64 ? 8 : 16; }

size_t ssd_lds_bytes(int P, int N, int Q) {
  (void)Q;
  const int RB = (P + 63) / 64;
  switch (nwq_for(N)) {
    case 2: return SsdLayout<2>::floats(RB) * sizeof(float);
    case 4: return SsdLayout<4>::floats(RB) * sizeof(float);
    case 8: return SsdLayout<8>::floats(RB) * sizeof(float);
    default: return SsdLayout<16>::floats(RB) * sizeof(float);
  }
}

template <typename T, int NWQ>
static hipError_t launch_w(hipStream_t st, const SsdArgs& a) {
  const int RB = (a.P + 63) / 64;
  const size_t lds = SsdLayout<NWQ>::floats(RB) * sizeof(float);
  auto kern = k_ssd_scan<T, NWQ>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.C * a.H), dim3(64 * NWQ * RB), lds, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(hipStream_t st, const SsdArgs& a) {
  switch (nwq_for(a.N)) {
    case 2: return launch_w<T, 2>(st, a);
    case 4: return launch_w<T, 4>(st, a);
    case 8: return launch_w<T, 8>(st, a);
    default: return launch_w<T, 16>(st, a);
  }
}

hipError_t launch_ssd_scan(hipStream_t st, int dtype, const SsdArgs& a) {
  return dtype == 1 ? launch_t<bf16_t>(st, a) : launch_t<float>(st, a);
}

}  // namespace hspec
