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
// The work per (request, head) is a few thousand multiply-adds against
// P*N*4 bytes of state in and out, so the kernel is laid out for latency:
// one wave per 64 state rows of a head, each lane holding its whole state
// row (N values) in registers for the whole block, so every state-row
// product is a lane-local multiply-add chain fed by LDS broadcasts and no
// partial sums cross lanes or waves.  A workgroup takes up to 4 heads of one
// request that share a B/Cm group: the chunk's B and Cm rows and the
// head-independent Cm.B^T products are staged and formed once per workgroup;
// each wave then scales them by its own head's decays.  The in-chunk
// cumulative sum runs across one wave's lanes with shuffles.
#include "common.h"
#include "kernels.h"
#include "merge.h"

namespace hspec {

constexpr int kSsdQ = 16;  // largest chunk (positions staged per pass)

// Static LDS, in floats.  sB / sC rows are padded to NMAX + 4 so the
// per-thread Cm.B^T dot products (rows t and s in different lanes) spread
// over the banks; every other read is a wave-wide broadcast.
template <int NMAX> struct SsdLds {
  static constexpr int LDB = NMAX + 4;
  static constexpr int oB = 0;                        // sB[Q][LDB]   B_s
  static constexpr int oC = oB + kSsdQ * LDB;         // sC[Q][LDB]   Cm_t
  static constexpr int oCB = oC + kSsdQ * LDB;        // sCB[Q][Q]    Cm_t . B_s at [t][s]
  static constexpr int oWave = oCB + kSsdQ * kSsdQ;   // per wave: lam[Q], w[Q], dt[Q], pad[Q], M[Q][Q]
  static constexpr int WAVE = 4 * kSsdQ + kSsdQ * kSsdQ;
  static constexpr int floats = oWave + 4 * WAVE;
};

// Heads per workgroup: as many as fit in 4 waves and divide the heads of one
// B/Cm group (so a workgroup never spans two groups).
__host__ __device__ inline int ssd_heads_per_block(int H, int ng, int P) {
  const int RB = (P + 63) / 64;
  const int hg = H / ng;
  for (int hpw = 4 / RB; hpw > 1; hpw >>= 1)
    if (hg % hpw == 0) return hpw;
  return 1;
}

// Workgroup = 4 waves; wave w handles head hfirst + w / RB, state rows
// (w % RB) * 64 + lane, for w < HPW * RB (the rest only help staging).  Every
// global load of a chunk is issued before the first wait, with clamped
// indices and selects instead of per-element branches (a load under a branch
// gets its own wait, which would serialize the loads' memory latencies).
// CONV: the inputs are the Mamba-2 block's raw projection rows; the lane
// loads the Q + 3 raw values of its channel that its chunk's convolution
// reads (zero before the block), each thread the four raw positions of its B
// and Cm entries, and the conv + SiLU and softplus run after all of them are
// issued.
// The scan of workgroup `bid` (a device function so that the drafter layer's
// combined scan + merge launch runs the same code).
template <typename T, int NMAX, bool V4, bool CONV>
__device__ __forceinline__ void ssd_scan_block(const SsdArgs& a, int bid) {
  using L = SsdLds<NMAX>;
  constexpr int Q = kSsdQ, LDB = L::LDB;
  constexpr int E = Q * NMAX / 256;  // B and Cm entries staged per thread
  __shared__ __align__(16) float lds[L::floats];
  const int H = a.H, P = a.P, N = a.N, K = a.K, QC = a.chunk;
  const int RB = (P + 63) >> 6;
  const int HPW = ssd_heads_per_block(H, a.ng, P);
  const int hblocks = H / HPW;
  const int b = bid / hblocks, hfirst = (bid % hblocks) * HPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool active = wave < HPW * RB;
  const int h = min(hfirst + wave / RB, H - 1), p = (wave % RB) * 64 + lane;
  const bool own = active && p < P;
  const int pc = min(p, P - 1);
  const int grp = hfirst / (H / a.ng);

  float* sB = lds + L::oB;
  float* sC = lds + L::oC;
  float* sCB = lds + L::oCB;
  float* wl = lds + L::oWave + wave * L::WAVE;
  float* slam = wl;
  float* sw = wl + Q;
  float* sdt = wl + 2 * Q;
  float* sM = wl + 4 * Q;  // M[t][s] at [t * Q + s]

  const T* __restrict__ Bm = static_cast<const T*>(a.B);
  const T* __restrict__ Cm = static_cast<const T*>(a.Cm);
  const float Ah = a.A[h];
  const float Dh = a.Dskip ? a.Dskip[h] : 0.f;
  const size_t HP = size_t(H) * P;
  const T* __restrict__ xrow = static_cast<const T*>(a.x) + (CONV ? 0 : (size_t(b) * K * H + h) * P + pc);
  float* __restrict__ yrow = a.y + (size_t(b) * K * H + h) * P + p;

  // the lane's state row H[p, 0..N), zero past N (and for idle lanes)
  float Hs[NMAX];
#pragma unroll
  for (int k = 0; k < NMAX; ++k) Hs[k] = 0.f;
  if (a.h0) {
    const float* hrow = a.h0 + ((size_t(b) * H + h) * P + pc) * N;
    if constexpr (V4) {  // N % 4 == 0: 16-byte loads
#pragma unroll
      for (int k = 0; k < NMAX; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(hrow + min(k, N - 4));
        Hs[k] = v.x; Hs[k + 1] = v.y; Hs[k + 2] = v.z; Hs[k + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < NMAX; ++k) Hs[k] = hrow[min(k, N - 1)];
    }
  }
  bool hmasked = false;  // the selects on Hs run after the first chunk's loads are issued

  for (int c0 = 0; c0 < K; c0 += QC) {
    const int q = min(QC, K - c0);
    // issue: the lane's x[c0 + s, p], this thread's B / Cm entries, the lane's delta
    float xs[Q];
    float bv[E], cv[E];
    float dv;
    if constexpr (CONV) {
      // raw rows of request b: column d_inner + ch is conv channel ch; the
      // step sizes follow the conv channels
      const int ngN = a.ng * N, dpj = a.d_proj;
      const float* zb = a.zx + size_t(b) * K * dpj + a.d_inner;
      auto raw_at = [&](int t, int ch) { return zb[size_t(min(max(t, 0), K - 1)) * dpj + ch]; };
      const int cx = h * P + pc;
      float rx[Q + 3];
#pragma unroll
      for (int s = 0; s < Q + 3; ++s) rx[s] = raw_at(c0 - 3 + s, cx);
      float rb[E][4], rc[E][4];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = tid + 256 * e, t = i / NMAX, n = min(i % NMAX, N - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rb[e][j] = raw_at(c0 + t - 3 + j, a.d_inner + grp * N + n);
          rc[e][j] = raw_at(c0 + t - 3 + j, a.d_inner + ngN + grp * N + n);
        }
      }
      const float rdt = raw_at(c0 + lane, a.d_inner + 2 * ngN + h);
      // positions before the block start are zero
      auto conv = [&](int ch, int t_last, const float* r) {
        const float4 w = reinterpret_cast<const float4*>(a.conv_w)[ch];
        float v = a.conv_b ? a.conv_b[ch] : 0.f;
        v = fmaf(w.x, t_last - 3 >= 0 ? r[0] : 0.f, v);
        v = fmaf(w.y, t_last - 2 >= 0 ? r[1] : 0.f, v);
        v = fmaf(w.z, t_last - 1 >= 0 ? r[2] : 0.f, v);
        v = fmaf(w.w, r[3], v);
        return silu_f(v);
      };
#pragma unroll
      for (int s = 0; s < Q; ++s) xs[s] = conv(cx, c0 + s, rx + s);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = tid + 256 * e, t = i / NMAX, n = min(i % NMAX, N - 1);
        bv[e] = conv(a.d_inner + grp * N + n, c0 + t, rb[e]);
        cv[e] = conv(a.d_inner + ngN + grp * N + n, c0 + t, rc[e]);
      }
      dv = softplus_f(rdt + a.dt_bias[h]);
    } else {
#pragma unroll
      for (int s = 0; s < Q; ++s) xs[s] = to_f32(xrow[size_t(min(c0 + s, K - 1)) * HP]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = tid + 256 * e, t = i / NMAX, n = i % NMAX;
        const size_t src = ((size_t(b) * K + min(c0 + t, K - 1)) * a.ng + grp) * N + min(n, N - 1);
        bv[e] = to_f32(Bm[src]);
        cv[e] = to_f32(Cm[src]);
      }
      dv = a.delta[(size_t(b) * K + min(c0 + lane, K - 1)) * H + h];
    }
    if (!hmasked) {
#pragma unroll
      for (int k = 0; k < NMAX; ++k) Hs[k] = (own && k < N) ? Hs[k] : 0.f;
      hmasked = true;
    }
#pragma unroll
    for (int s = 0; s < Q; ++s) xs[s] = (own && s < q) ? xs[s] : 0.f;
    // the chunk's B and Cm rows of this group, zero-padded to Q x NMAX
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid + 256 * e, t = i / NMAX, n = i % NMAX;
      const bool in = t < q && n < N;
      sB[t * LDB + n] = in ? bv[e] : 0.f;
      sC[t * LDB + n] = in ? cv[e] : 0.f;
    }
    // this head's in-chunk cumulative log-decay (inclusive scan over lanes)
    {
      const float dt = lane < q ? dv : 0.f;
      float v = dt * Ah;
#pragma unroll
      for (int off = 1; off < Q; off <<= 1) {
        const float u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
      }
      const float lend = __shfl(v, q - 1, 64);
      if (lane < Q) {
        slam[lane] = v;
        sdt[lane] = dt;
        sw[lane] = lane < q ? __expf(lend - v) * dt : 0.f;
      }
    }
    __syncthreads();
    // head-independent Cm_t . B_s of the group (one entry per thread)
    {
      const int t = tid / Q, s = tid % Q;
      const float* cr = sC + t * LDB;
      const float* br = sB + s * LDB;
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int n = 0; n < NMAX; n += 4) {
        const float4 c = *reinterpret_cast<const float4*>(cr + n);
        const float4 bb = *reinterpret_cast<const float4*>(br + n);
        d0 = fmaf(c.x, bb.x, d0);
        d1 = fmaf(c.y, bb.y, d1);
        d0 = fmaf(c.z, bb.z, d0);
        d1 = fmaf(c.w, bb.w, d1);
      }
      sCB[tid] = d0 + d1;
    }
    __syncthreads();
    // this head's decay-weighted M, masked before the exponential
#pragma unroll
    for (int j = 0; j < Q * Q / 64; ++j) {
      const int i = lane + 64 * j;
      const int t = i / Q, s = i % Q;
      float v = 0.f;
      if (s <= t && t < q) v = __expf(slam[t] - slam[s]) * sCB[i] * sdt[s];
      sM[i] = v;
    }
    __syncthreads();
    // y[t, p] = exp(lam_t) H_in[p, :] . Cm_t + sum_{s <= t} M[t, s] x[s, p] + D x[t, p]
    if (own) {
#pragma unroll
      for (int t = 0; t < Q; ++t) {
        if (t < q) {
          const float* cr = sC + t * LDB;
          float z0 = 0.f, z1 = 0.f;
#pragma unroll
          for (int n = 0; n < NMAX; n += 4) {
            const float4 c = *reinterpret_cast<const float4*>(cr + n);
            z0 = fmaf(Hs[n], c.x, z0);
            z1 = fmaf(Hs[n + 1], c.y, z1);
            z0 = fmaf(Hs[n + 2], c.z, z0);
            z1 = fmaf(Hs[n + 3], c.w, z1);
          }
          float z = (z0 + z1) * __expf(slam[t]);
          const float* mr = sM + t * Q;
#pragma unroll
          for (int s = 0; s <= t; s += 4) {
            const float4 m = *reinterpret_cast<const float4*>(mr + s);
            z = fmaf(m.x, xs[s], z);
            if (s + 1 <= t) z = fmaf(m.y, xs[s + 1], z);
            if (s + 2 <= t) z = fmaf(m.z, xs[s + 2], z);
            if (s + 3 <= t) z = fmaf(m.w, xs[s + 3], z);
          }
          yrow[size_t(c0 + t) * HP] = fmaf(Dh, xs[t], z);
        }
      }
    }
    // state passing: H_out[p, n] = exp(lam_end) H_in[p, n] + sum_s w_s x[s, p] B[s, n]
    // (after the last chunk only h_final needs it)
    if (c0 + QC >= K && !a.h_final) break;
    const float dend = __expf(slam[q - 1]);
#pragma unroll
    for (int n = 0; n < NMAX; ++n) Hs[n] *= dend;
#pragma unroll
    for (int s = 0; s < Q; ++s) {
      if (s < q) {
        const float coef = sw[s] * xs[s];
        const float* br = sB + s * LDB;
#pragma unroll
        for (int n = 0; n < NMAX; n += 4) {
          const float4 bb = *reinterpret_cast<const float4*>(br + n);
          Hs[n] = fmaf(coef, bb.x, Hs[n]);
          Hs[n + 1] = fmaf(coef, bb.y, Hs[n + 1]);
          Hs[n + 2] = fmaf(coef, bb.z, Hs[n + 2]);
          Hs[n + 3] = fmaf(coef, bb.w, Hs[n + 3]);
        }
      }
    }
    if (c0 + QC < K) __syncthreads();  // the next chunk rewrites LDS
  }
  if (a.h_final && own) {
    float* hf = a.h_final + ((size_t(b) * H + h) * P + p) * N;
    if constexpr (V4) {
#pragma unroll
      for (int k = 0; k < NMAX; k += 4)
        if (k < N) *reinterpret_cast<float4*>(hf + k) = make_float4(Hs[k], Hs[k + 1], Hs[k + 2], Hs[k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < NMAX; ++k)
        if (k < N) hf[k] = Hs[k];
    }
  }
}

template <typename T, int NMAX, bool V4, bool CONV>
__global__ __launch_bounds__(256) void k_ssd_scan(SsdArgs a) {
  ssd_scan_block<T, NMAX, V4, CONV>(a, blockIdx.x);
}

// Workgroups [0, n_scan) run the scan, the rest the merge of the attention's
// split partials (grid (C * Hkv) x slabs, flattened request-major).  The two
// are independent: the scan needs the projected state, the merge the
// attention's partials, both written by earlier launches on the stream.
template <int NMAX, int LPO, int U>
__global__ __launch_bounds__(256) void k_scan_merge(SsdArgs s, AttnArgs m, int n_scan) {
  const int bid = blockIdx.x;
  if (bid < n_scan) {
    ssd_scan_block<bf16_t, NMAX, true, false>(s, bid);
  } else {
    const int r = bid - n_scan, ch = m.C * m.Hkv;
    attn_merge_block<bf16_t, 128, LPO, U>(m, r % ch, r / ch);
  }
}

size_t ssd_lds_bytes(int P, int N, int Q) {
  (void)P;
  (void)Q;
  if (N <= 16) return SsdLds<16>::floats * sizeof(float);
  if (N <= 32) return SsdLds<32>::floats * sizeof(float);
  if (N <= 64) return SsdLds<64>::floats * sizeof(float);
  return SsdLds<128>::floats * sizeof(float);
}

template <typename T, int NMAX>
static hipError_t launch_n(hipStream_t st, const SsdArgs& a) {
  const int hpw = ssd_heads_per_block(a.H, a.ng, a.P);
  const dim3 grid(a.C * (a.H / hpw)), block(256);
  if constexpr (std::is_same<T, float>::value) {
    if (a.zx) {
      if (a.N % 4 == 0)
        hipLaunchKernelGGL((k_ssd_scan<T, NMAX, true, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((k_ssd_scan<T, NMAX, false, true>), grid, block, 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.N % 4 == 0)
    hipLaunchKernelGGL((k_ssd_scan<T, NMAX, true, false>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_ssd_scan<T, NMAX, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
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

bool scan_merge_fits(int dtype, const SsdArgs& s, const AttnArgs& m) {
  return dtype == 1 && !s.zx && s.N % 4 == 0 && m.D == 128 && m.max_items > m.C;
}

// The merge part takes the configuration k_attn_merge would (LPO lanes per
// output quad, U splits per round of loads, by the largest split count).
template <int NMAX, int LPO, int U>
static hipError_t launch_scan_merge_cfg(hipStream_t st, const SsdArgs& s, const AttnArgs& m) {
  const int n_scan = s.C * (s.H / ssd_heads_per_block(s.H, s.ng, s.P));
  constexpr int OPB = 256 / LPO;
  const int slabs = (m.rows * (128 / 4) + OPB - 1) / OPB;
  const dim3 grid(n_scan + m.C * m.Hkv * slabs), block(256);
  hipLaunchKernelGGL((k_scan_merge<NMAX, LPO, U>), grid, block, 0, st, s, m, n_scan);
  return hipGetLastError();
}

template <int NMAX>
static hipError_t launch_scan_merge_n(hipStream_t st, const SsdArgs& s, const AttnArgs& m) {
  const int ms = m.max_splits;
  if (ms <= 4) return launch_scan_merge_cfg<NMAX, 1, 4>(st, s, m);
  if (ms <= 8) return launch_scan_merge_cfg<NMAX, 1, 8>(st, s, m);
  if (ms <= 16) return launch_scan_merge_cfg<NMAX, 4, 4>(st, s, m);
  return launch_scan_merge_cfg<NMAX, 4, 8>(st, s, m);
}

hipError_t launch_scan_merge(hipStream_t st, const SsdArgs& s, const AttnArgs& m) {
  if (s.N <= 16) return launch_scan_merge_n<16>(st, s, m);
  if (s.N <= 32) return launch_scan_merge_n<32>(st, s, m);
  if (s.N <= 64) return launch_scan_merge_n<64>(st, s, m);
  return launch_scan_merge_n<128>(st, s, m);
}

}  // namespace hspec
