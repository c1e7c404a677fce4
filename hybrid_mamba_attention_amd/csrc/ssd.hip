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

// Static LDS, in floats, for chunks of up to QM positions (16, 32 or 64:
// the whole chunk is staged at once, so the intra-chunk decay matrix spans
// it).  sB / sC rows are padded to NMAX + 4 so the per-thread Cm.B^T dot
// products (rows t and s in different lanes) spread over the banks; every
// other read is a wave-wide broadcast.
template <int NMAX, int QM> struct SsdLds {
  static constexpr int LDB = NMAX + 4;
  static constexpr int oB = 0;                        // sB[QM][LDB]   B_s
  static constexpr int oC = oB + QM * LDB;            // sC[QM][LDB]   Cm_t
  static constexpr int oCB = oC + QM * LDB;           // sCB[QM][QM]   Cm_t . B_s at [t][s]
  static constexpr int oWave = oCB + QM * QM;         // per wave: lam, w, dt, pad [QM]; M[QM][QM]
  static constexpr int WAVE = 4 * QM + QM * QM;
  static constexpr int floats = oWave + 4 * WAVE;
  // Before the first chunk each row block of 64 state rows (one per wave, or
  // one shared by the four waves of a head) is staged here, rows padded to
  // LDH floats: a lane reading its own row, 16 lanes per pass, then hits 16
  // distinct bank quads.  It aliases the arrays above and is only used with
  // 16-byte state rows and states of up to 64.  `total` is the most any
  // layout needs (four blocks).
  static constexpr int LDH = NMAX + 4;
  static constexpr int stage(int blocks) { return NMAX <= 64 ? blocks * 64 * LDH : 0; }
  static constexpr int with_stage(int blocks) { return floats > stage(blocks) ? floats : stage(blocks); }
  static constexpr int total = with_stage(4);
};

// the smallest chunk capacity that holds a chunk
inline int ssd_chunk_cap(int chunk) { return chunk <= 16 ? 16 : chunk <= 32 ? 32 : 64; }

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
// TS = 4 (batches with few heads): the workgroup takes one head (P <= 64) and
// its four waves share it, wave k forming y at positions k, k+4, ... of each
// chunk and a quarter of the head's decay matrix.  Every wave keeps the whole
// state row and updates it after each chunk but the last (the next chunk
// reads all of it); after the last, whose update only feeds h_final, wave k
// updates and writes state columns [k*NMAX/4, (k+1)*NMAX/4).  A position's sum runs over the full row of the masked matrix,
// whose entries past the position are exact zeros, so y has the same bits as
// with one wave per head.
// The scan of workgroup `bid` (a device function so that the drafter layer's
// combined scan + merge launch runs the same code).
// STG: stage the initial state through LDS where it can (see STAGE_H0).
template <typename T, int NMAX, int QM, bool V4, bool CONV, int TS = 1, bool STG = true>
__device__ __forceinline__ void ssd_scan_block(const SsdArgs& a, int bid) {
  using L = SsdLds<NMAX, QM>;
  constexpr int Q = QM, LDB = L::LDB;
  constexpr int E = Q * NMAX / 256;  // B and Cm entries staged per thread
  static_assert(Q * NMAX % 256 == 0 && Q <= 64, "whole staging rounds; one lane per chunk position");
  constexpr bool STAGE_H0 = STG && V4 && NMAX <= 64;
  __shared__ __align__(16) float lds[STAGE_H0 ? L::with_stage(4 / TS) : L::floats];
  const int H = a.H, P = a.P, N = a.N, K = a.K, QC = a.chunk;
  static_assert(TS == 1 || TS == 4, "one wave per head row block, or four per head");
  static_assert(TS == 1 || V4, "the column-split h_final store is the 16-byte one");
  const int RB = (P + 63) >> 6;
  const int HPW = TS == 1 ? ssd_heads_per_block(H, a.ng, P) : 1;
  const int hblocks = H / HPW;
  const int b = bid / hblocks, hfirst = (bid % hblocks) * HPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // (head, row block) of the wave; its position slice (wave-uniform, scalar)
  const int hw = wave / TS, tsw = __builtin_amdgcn_readfirstlane(wave % TS);
  const bool active = hw < HPW * RB;
  const int h = min(hfirst + hw / RB, H - 1), p = (hw % RB) * 64 + lane;
  const bool own = active && p < P;
  const int pc = min(p, P - 1);
  const int grp = hfirst / (H / a.ng);

  float* sB = lds + L::oB;
  float* sC = lds + L::oC;
  float* sCB = lds + L::oCB;
  float* wl = lds + L::oWave + hw * L::WAVE;
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
  // STAGE_H0: the wave's rows [r0, r0 + nr) of the head's state are one
  // contiguous block of nr * N floats, read as 1 KB-contiguous wave loads
  // (each lane's own 128-byte row as 16-byte pieces would make every load
  // touch 64 cache lines) and moved into the lanes' rows through LDS once the
  // first chunk's loads are in flight.  The block is loaded by the GT
  // threads that share it (the wave, or with TS = 4 the head's four waves),
  // piece j of group thread gi being floats 4 * (gi + GT * j) .. + 3; until
  // the staging Hs[4j .. 4j + 3] holds it.
  constexpr int GT = 64 * TS, PPT = NMAX / 4 / TS;  // PPT: pieces per thread
  const int gi = TS == 1 ? lane : tid;
  const int r0 = (hw % RB) * 64, nr = min(64, P - r0);
  if (STAGE_H0 && a.h0) {
    const float* blk = a.h0 + ((size_t(b) * H + h) * P + r0) * N;
    const int lastf = nr * N - 4;  // N % 4 == 0: every piece lies in one row
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(blk + min(4 * (gi + GT * j), lastf));
      Hs[4 * j] = v.x; Hs[4 * j + 1] = v.y; Hs[4 * j + 2] = v.z; Hs[4 * j + 3] = v.w;
    }
  } else if (a.h0) {
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
      if (STAGE_H0 && a.h0) {
        // piece j starts at float f of the block: row f / N, columns f % N
        // .. + 3 (pieces past the block repeat its last one)
        float* st = lds + (TS == 1 ? wave : 0) * 64 * L::LDH;
        const int lastf = nr * N - 4;
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
          const int f = min(4 * (gi + GT * j), lastf);
          const int r = N == NMAX ? f / NMAX : f / N, cc = f - r * N;
          *reinterpret_cast<float4*>(st + r * L::LDH + cc) =
              make_float4(Hs[4 * j], Hs[4 * j + 1], Hs[4 * j + 2], Hs[4 * j + 3]);
        }
        __syncthreads();
        // rows past nr and columns past N hold stale values: the selects below drop them
#pragma unroll
        for (int k = 0; k < NMAX; k += 4) {
          const float4 v = *reinterpret_cast<const float4*>(st + lane * L::LDH + k);
          Hs[k] = v.x; Hs[k + 1] = v.y; Hs[k + 2] = v.z; Hs[k + 3] = v.w;
        }
        __syncthreads();  // the chunk arrays below alias the staging
      }
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
      if (lane < Q && tsw == 0) {
        slam[lane] = v;
        sdt[lane] = dt;
        sw[lane] = lane < q ? __expf(lend - v) * dt : 0.f;
      }
    }
    __syncthreads();
    // head-independent Cm_t . B_s of the group (Q*Q / 256 entries per thread)
#pragma unroll
    for (int i = tid; i < Q * Q; i += 256) {
      const int t = i / Q, s = i % Q;
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
      sCB[i] = d0 + d1;
    }
    __syncthreads();
    // this head's decay-weighted M, masked before the exponential (a quarter
    // of it per wave with TS = 4)
#pragma unroll 4
    for (int j = 0; j < Q * Q / 64 / TS; ++j) {
      const int i = lane + 64 * (j * TS + tsw);
      const int t = i / Q, s = i % Q;
      float v = 0.f;
      if (s <= t && t < q) v = __expf(slam[t] - slam[s]) * sCB[i] * sdt[s];
      sM[i] = v;
    }
    __syncthreads();
    // y[t, p] = exp(lam_t) H_in[p, :] . Cm_t + sum_{s <= t} M[t, s] x[s, p] + D x[t, p]
    if (own && Q > 16) {
      // Chunks of 32 or 64: one position per loop trip, the full row of M
      // (zero past t) against the lane's x values, so the code grows with
      // Q instead of Q^2 (the unrolled triangle took minutes to compile).
#pragma unroll 1
      for (int t = tsw; t < q; t += TS) {
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
        float xt = 0.f;
#pragma unroll
        for (int s = 0; s < Q; s += 4) {
          const float4 m = *reinterpret_cast<const float4*>(mr + s);
          z = fmaf(m.x, xs[s], z);
          z = fmaf(m.y, xs[s + 1], z);
          z = fmaf(m.z, xs[s + 2], z);
          z = fmaf(m.w, xs[s + 3], z);
          xt = s == (t & ~3) ? ((t & 3) == 0 ? xs[s] : (t & 3) == 1 ? xs[s + 1] : (t & 3) == 2 ? xs[s + 2] : xs[s + 3]) : xt;
        }
        yrow[size_t(c0 + t) * HP] = fmaf(Dh, xt, z);
      }
    } else if (own) {
#pragma unroll
      for (int jt = 0; jt < Q / TS; ++jt) {
        const int t = jt * TS + tsw;
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
          if constexpr (TS == 1) {
#pragma unroll
            for (int s = 0; s <= t; s += 4) {
              const float4 m = *reinterpret_cast<const float4*>(mr + s);
              z = fmaf(m.x, xs[s], z);
              if (s + 1 <= t) z = fmaf(m.y, xs[s + 1], z);
              if (s + 2 <= t) z = fmaf(m.z, xs[s + 2], z);
              if (s + 3 <= t) z = fmaf(m.w, xs[s + 3], z);
            }
            yrow[size_t(c0 + t) * HP] = fmaf(Dh, xs[t], z);
          } else {
            // the full row: M[t][s] is an exact zero for s > t
#pragma unroll
            for (int s = 0; s < Q; s += 4) {
              const float4 m = *reinterpret_cast<const float4*>(mr + s);
              z = fmaf(m.x, xs[s], z);
              z = fmaf(m.y, xs[s + 1], z);
              z = fmaf(m.z, xs[s + 2], z);
              z = fmaf(m.w, xs[s + 3], z);
            }
            float xt = xs[jt * TS];
#pragma unroll
            for (int k = 1; k < TS; ++k) xt = tsw == k ? xs[jt * TS + k] : xt;
            yrow[size_t(c0 + t) * HP] = fmaf(Dh, xt, z);
          }
        }
      }
    }
    // state passing: H_out[p, n] = exp(lam_end) H_in[p, n] + sum_s w_s x[s, p] B[s, n]
    // (after the last chunk only h_final needs it; with TS waves per head
    // each then takes its quarter of the columns)
    if (c0 + QC >= K && !a.h_final) break;
    const bool split_n = TS > 1 && c0 + QC >= K;
    constexpr int NQ = NMAX / TS;
    const float dend = __expf(slam[q - 1]);
#pragma unroll
    for (int n = 0; n < NMAX; ++n)
      if (!split_n || n / NQ == tsw) Hs[n] *= dend;
#pragma unroll
    for (int s = 0; s < Q; ++s) {
      if (s < q) {
        const float coef = sw[s] * xs[s];
        const float* br = sB + s * LDB;
#pragma unroll
        for (int n = 0; n < NMAX; n += 4) {
          if (split_n && n / NQ != tsw) continue;
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
        if (k < N && (TS == 1 || k / (NMAX / TS) == tsw))
          *reinterpret_cast<float4*>(hf + k) = make_float4(Hs[k], Hs[k + 1], Hs[k + 2], Hs[k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < NMAX; ++k)
        if (k < N) hf[k] = Hs[k];
    }
  }
}

// Chunks of up to 16 with states of up to 64 are held to two waves per SIMD
// (256 registers): the convolution-fused form at N = 64 took 257 unbounded,
// which halved its occupancy and ran a 2048-head batch in two rounds.
template <typename T, int NMAX, int QM, bool V4, bool CONV, int TS = 1>
__global__ __launch_bounds__(256, (QM == 16 && NMAX <= 64) ? 2 : 1) void k_ssd_scan(SsdArgs a) {
  ssd_scan_block<T, NMAX, QM, V4, CONV, TS>(a, blockIdx.x);
}

// Workgroups [0, n_scan) run the scan, the rest the merge of the attention's
// partials (grid (C * Hkv) x slabs, flattened request-major).  The two
// are independent: the scan needs the projected state, the merge the
// attention's partials, both written by earlier launches on the stream.
// The merge's many short workgroups take the scan's LDS too, so the state is
// staged through LDS only where that does not enlarge it (TS = 4: one block
// per workgroup): with four blocks (36 KB) the uncut batch of 128 requests
// gained 1.3 us of scan and lost as much to the merge's occupancy.
template <int NMAX, int LPO, int U, int TS>
__global__ __launch_bounds__(256) void k_scan_merge(SsdArgs s, AttnArgs m, int n_scan) {
  const int bid = blockIdx.x;
  if (bid < n_scan) {
    ssd_scan_block<bf16_t, NMAX, 16, true, false, TS, (TS > 1)>(s, bid);
  } else {
    const int r = bid - n_scan, ch = m.C * m.Hkv;
    attn_merge_block<bf16_t, 128, LPO, U>(m, r % ch, r / ch);
  }
}

size_t ssd_lds_bytes(int P, int N, int Q) {
  (void)P;
  const int qm = ssd_chunk_cap(Q);
  auto by_n = [&](auto QC) -> size_t {
    constexpr int QM = decltype(QC)::value;
    if (N <= 16) return SsdLds<16, QM>::total * sizeof(float);
    if (N <= 32) return SsdLds<32, QM>::total * sizeof(float);
    if (N <= 64) return SsdLds<64, QM>::total * sizeof(float);
    return SsdLds<128, QM>::total * sizeof(float);
  };
  if (qm == 16) return by_n(std::integral_constant<int, 16>{});
  // chunks of 32 and 64 run with a state capacity of 64
  if (qm == 32) return SsdLds<64, 32>::total * sizeof(float);
  return SsdLds<64, 64>::total * sizeof(float);
}

// Four waves per head (TS = 4) when the batch has too few heads for the
// four-heads form to give every SIMD two waves: at C = 1 (16 heads) that form
// runs 16 waves on the whole chip, each a serial chain over its chunk's
// positions.  States of 17..64 (the model shapes), plain inputs, N % 4 == 0.
// Up to 1024 heads (one wave per SIMD in the four-heads form) it is faster
// (1024 heads: 10.0 against 10.9 us), at 2048 slower (17.2 against 15.7).
static bool ssd_split_positions(const SsdArgs& a) {
  return !a.zx && a.P <= 64 && a.N > 16 && a.N <= 64 && a.N % 4 == 0 && a.chunk <= 16 &&
         int64_t(a.C) * a.H <= 1024;
}

template <typename T, int NMAX>
static hipError_t launch_n(hipStream_t st, const SsdArgs& a) {
  if constexpr (NMAX == 32 || NMAX == 64) {
    if (ssd_split_positions(a)) {
      hipLaunchKernelGGL((k_ssd_scan<T, NMAX, 16, true, false, 4>), dim3(a.C * a.H), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  const int hpw = ssd_heads_per_block(a.H, a.ng, a.P);
  const dim3 grid(a.C * (a.H / hpw)), block(256);
  if constexpr (std::is_same<T, float>::value) {
    if (a.zx) {
      if (a.N % 4 == 0)
        hipLaunchKernelGGL((k_ssd_scan<T, NMAX, 16, true, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((k_ssd_scan<T, NMAX, 16, false, true>), grid, block, 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.N % 4 == 0)
    hipLaunchKernelGGL((k_ssd_scan<T, NMAX, 16, true, false>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_ssd_scan<T, NMAX, 16, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

// Chunks of 32 or 64 positions: the plain scan (no fused convolution), with
// N % 4 == 0 and N <= 64 (ssd_chunk_fits; the host refuses the rest).
template <typename T, int QM>
static hipError_t launch_big_chunk(hipStream_t st, const SsdArgs& a) {
  const int hpw = ssd_heads_per_block(a.H, a.ng, a.P);
  const dim3 grid(a.C * (a.H / hpw)), block(256);
  // one state capacity (64) for all of them: each chunk size unrolls Q^2 / 2
  // multiply-adds per lane, and more instantiations cost minutes of build
  hipLaunchKernelGGL((k_ssd_scan<T, 64, QM, true, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(hipStream_t st, const SsdArgs& a) {
  const int qm = ssd_chunk_cap(a.chunk);
  if (qm == 32) return launch_big_chunk<T, 32>(st, a);
  if (qm == 64) return launch_big_chunk<T, 64>(st, a);
  if (a.N <= 16) return launch_n<T, 16>(st, a);
  if (a.N <= 32) return launch_n<T, 32>(st, a);
  if (a.N <= 64) return launch_n<T, 64>(st, a);
  return launch_n<T, 128>(st, a);
}

bool ssd_chunk_fits(int chunk, int N, bool conv) {
  return chunk <= 16 || (!conv && N % 4 == 0 && N <= 64);
}

hipError_t launch_ssd_scan(hipStream_t st, int dtype, const SsdArgs& a) {
  return dtype == 1 ? launch_t<bf16_t>(st, a) : launch_t<float>(st, a);
}

// States of up to 32: with a 64-wide state the combined grid takes the scan's
// registers for every workgroup and the merge's workgroups wait behind the
// scan's (the 64-head ragged batch: 39.5 us against 22.9 + 11.7 as two
// launches).
bool scan_merge_fits(int dtype, const SsdArgs& s, const AttnArgs& m) {
  return dtype == 1 && !s.zx && s.N % 4 == 0 && s.N <= 32 && s.chunk <= 16 && m.D == 128 && m.w_max > 1;
}

// The merge part takes the configuration k_attn_merge would (LPO lanes per
// output quad and at most U pieces per lane and round of loads).
template <int NMAX, int LPO, int U>
static hipError_t launch_scan_merge_cfg(hipStream_t st, const SsdArgs& s, const AttnArgs& m) {
  constexpr int OPB = 256 / LPO;
  const int slabs = (m.rows * (128 / 4) + OPB - 1) / OPB;
  if constexpr (NMAX == 32) {
    if (ssd_split_positions(s)) {
      const int n_scan = s.C * s.H;
      hipLaunchKernelGGL((k_scan_merge<NMAX, LPO, U, 4>), dim3(n_scan + m.C * m.Hkv * slabs), dim3(256), 0, st,
                         s, m, n_scan);
      return hipGetLastError();
    }
  }
  const int n_scan = s.C * (s.H / ssd_heads_per_block(s.H, s.ng, s.P));
  const dim3 grid(n_scan + m.C * m.Hkv * slabs), block(256);
  hipLaunchKernelGGL((k_scan_merge<NMAX, LPO, U, 1>), grid, block, 0, st, s, m, n_scan);
  return hipGetLastError();
}

template <int NMAX>
static hipError_t launch_scan_merge_n(hipStream_t st, const SsdArgs& s, const AttnArgs& m) {
  if (merge_wide(m)) return launch_scan_merge_cfg<NMAX, 4, 16>(st, s, m);
  return launch_scan_merge_cfg<NMAX, 1, 8>(st, s, m);
}

hipError_t launch_scan_merge(hipStream_t st, const SsdArgs& s, const AttnArgs& m) {
  if (s.N <= 16) return launch_scan_merge_n<16>(st, s, m);
  return launch_scan_merge_n<32>(st, s, m);   // scan_merge_fits: N <= 32
}

}  // namespace hspec
