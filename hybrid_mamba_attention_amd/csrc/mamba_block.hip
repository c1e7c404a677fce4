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
// k_gemm_tn computes C[M,N] = A[M,K] . B[N,K]^T with both operands contiguous
// along K (weights in the [out, in] convention), which is exactly the operand
// layout of the bf16 matrix cores: a lane's eight contraction-adjacent
// elements are one 16-byte row piece.
//   * Workgroup: 4 waves in a 2 x 2 arrangement over a (64*WM) x (64*WN)
//     output tile; each wave owns WM x WN tiles of 32 x 32
//     (v_mfma_f32_32x32x16_bf16, fp32 accumulation in registers).
//   * K advances 64 at a time.  Every thread issues 16-byte loads of A and B
//     row pieces for the stage PF ahead into a register ring; a stage is then
//     written to one of two LDS buffers, one barrier, and the waves run their
//     MFMAs on it.  LDS rows are 128 bytes with the 16-byte piece index XORed
//     by (row % 8), so both the stores and the operand reads are free of bank
//     conflicts.
//   * Rows of A or B past M or N repeat the last row (their results are never
//     stored); contraction indices past K load zeros.
//   * Split-K: blockIdx.y takes one slice of K.  With more than one slice the
//     kernel stores fp32 partials and k_splitk_sum adds them in slice order,
//     so results are repeatable bit for bit.
// fp32 activations take k_gemm_tn_f32, a plain LDS-tiled FMA kernel.
#include <algorithm>

#include "common.h"
#include "kernels.h"

#ifndef HSPEC_GEMM_PF
#define HSPEC_GEMM_PF 2
#endif

namespace hspec {

namespace {

template <typename T> __device__ __forceinline__ void store_out(T* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }

// four consecutive outputs (16-byte aligned fp32, 8-byte aligned bf16)
template <typename T> __device__ __forceinline__ void store_out4(T* p, float4 v);
template <> __device__ __forceinline__ void store_out4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <> __device__ __forceinline__ void store_out4<bf16_t>(bf16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + __expf(-v)); }

// log(1 + e^v); above 20 the correction is below fp32 resolution.
__device__ __forceinline__ float softplus_f(float v) { return v > 20.f ? v : log1pf(__expf(v)); }

}  // namespace

// ---------------------------------------------------------------------------
// bf16 GEMM on matrix cores
// ---------------------------------------------------------------------------

template <int WM, int WN, typename OutT, int PF>
__global__ __launch_bounds__(256) void k_gemm_tn(GemmArgs g) {
  constexpr int BM = 64 * WM, BN = 64 * WN;
  constexpr int LA = BM / 32, LB = BN / 32;        // 16-byte loads per thread per stage
  constexpr int TA = BM * 128, TB = BN * 128;      // bytes of one LDS tile
  static_assert(PF >= 2 && PF % 2 == 0, "even prefetch depth keeps the LDS buffer parity static");
  __shared__ __align__(16) unsigned char lds[2 * (TA + TB)];
  unsigned char* sA = lds;
  unsigned char* sB = lds + 2 * TA;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int tm = blockIdx.x % g.tiles_m, tn = blockIdx.x / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_lo = blockIdx.y * g.kchunk;
  const int k_hi = min(g.K, k_lo + g.kchunk);
  const int nst = (k_hi - k_lo + 63) >> 6;

  // loader: thread -> 16-byte piece lc of rows lr + 32*i
  const int lc = tid & 7, lr = tid >> 3;
  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.a);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.b);
  const bf16_t* pa[LA];
  const bf16_t* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) pa[i] = A + size_t(min(m0 + lr + 32 * i, g.M - 1)) * g.lda;
#pragma unroll
  for (int i = 0; i < LB; ++i) pb[i] = B + size_t(min(n0 + lr + 32 * i, g.N - 1)) * g.ldb;
  uint32_t wpos[LA > LB ? LA : LB];
#pragma unroll
  for (int i = 0; i < (LA > LB ? LA : LB); ++i) {
    const int r = lr + 32 * i;
    wpos[i] = r * 128 + ((lc ^ (r & 7)) << 4);
  }

  // Loads go out unconditionally (a piece past K reads an in-range address);
  // pieces past K are zeroed when the stage is written to LDS, because a
  // select on a value just loaded would wait for that load at issue time.
  u32x4 ra[PF][LA], rb[PF][LB];
  auto issue = [&](int st, u32x4 (&xa)[LA], u32x4 (&xb)[LB]) __attribute__((always_inline)) {
    const int k = k_lo + st * 64 + lc * 8;
    const int kc = k < k_hi ? k : k_lo;       // K % 8 == 0: a piece is all in or all out
#pragma unroll
    for (int i = 0; i < LA; ++i) xa[i] = *reinterpret_cast<const u32x4*>(pa[i] + kc);
#pragma unroll
    for (int i = 0; i < LB; ++i) xb[i] = *reinterpret_cast<const u32x4*>(pb[i] + kc);
  };
  auto commit = [&](int st, int buf, const u32x4 (&xa)[LA], const u32x4 (&xb)[LB]) __attribute__((always_inline)) {
    const bool ok = k_lo + st * 64 + lc * 8 < k_hi;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<u32x4*>(sA + buf * TA + wpos[i]) = ok ? xa[i] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<u32x4*>(sB + buf * TB + wpos[i]) = ok ? xb[i] : u32x4{0, 0, 0, 0};
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // operand rows of this lane (row l%32 of each 32-row tile; piece half l/32)
  const int orow = lane & 31, ohalf = lane >> 5;
  // The operands of k-step ks+1 are read from LDS before the MFMAs of k-step
  // ks are issued, so LDS latency hides behind matrix work.
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* ta = sA + buf * TA;
    const unsigned char* tb = sB + buf * TB;
    Vec8<bf16_t> ao[2][WM], bo[2][WN];
    auto read = [&](int ks, Vec8<bf16_t> (&a)[WM], Vec8<bf16_t> (&b)[WN]) __attribute__((always_inline)) {
      const int pc = 2 * ks + ohalf;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr * 32 * WM + 32 * i + orow;
        a[i].v = *reinterpret_cast<const uint4*>(ta + r * 128 + ((pc ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = wc * 32 * WN + 32 * j + orow;
        b[j].v = *reinterpret_cast<const uint4*>(tb + r * 128 + ((pc ^ (r & 7)) << 4));
      }
    };
    read(0, ao[0], bo[0]);
    static_for<0, 4>([&](auto KS) __attribute__((always_inline)) {
      constexpr int ks = decltype(KS)::value;
      if constexpr (ks + 1 < 4) read(ks + 1, ao[(ks + 1) & 1], bo[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mma32(ao[ks & 1][i], bo[ks & 1][j], acc[i][j]);
    });
  };

  // Stage st: barrier, MFMAs on LDS buffer st&1, then stage st+1 goes from
  // its register slot into buffer (st+1)&1 (last read by stage st-1, which
  // every wave finished before this barrier) and stage st+1+PF is issued
  // into the freed slot.  The wait for stage st+1's loads thus comes after
  // stage st's MFMAs are queued.  Every slot issues its loads, also past the
  // last stage (an in-range, already cached piece that is never used), and
  // stage nst is written to the idle buffer: with no path that skips a load,
  // each wait counts exactly the PF-1 newer stages still in flight.
  static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
    constexpr int pp = decltype(P)::value;
    issue(pp, ra[pp], rb[pp]);
  });
  commit(0, 0, ra[0], rb[0]);
  issue(PF, ra[0], rb[0]);
  const int nfull = nst - nst % PF;
  for (int st0 = 0; st0 < nfull; st0 += PF) {
    static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
      constexpr int pp = decltype(P)::value;
      constexpr int nx = (pp + 1) % PF;
      __syncthreads();
      compute(pp & 1);
      __builtin_amdgcn_sched_barrier(0);   // the loads' wait stays behind the queued MFMAs
      commit(st0 + pp + 1, (pp + 1) & 1, ra[nx], rb[nx]);
      issue(st0 + pp + 1 + PF, ra[nx], rb[nx]);
    });
  }
  static_for<0, PF - 1>([&](auto P) __attribute__((always_inline)) {
    constexpr int pp = decltype(P)::value;
    constexpr int nx = (pp + 1) % PF;
    if (nfull + pp < nst) {   // uniform over the workgroup
      __syncthreads();
      compute(pp & 1);
      commit(nfull + pp + 1, (pp + 1) & 1, ra[nx], rb[nx]);
    }
  });

  // result element r of tile (i, j): column 32j + l%32, row 32i + 8(r/4) + 4(l/32) + r%4
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + wc * 32 * WN + 32 * j + orow;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wr * 32 * WM + 32 * i + 8 * (r >> 2) + 4 * ohalf + (r & 3);
        if (m >= g.M) continue;
        if (g.splits == 1)
          store_out(static_cast<OutT*>(g.c) + size_t(m) * g.ldc + n, acc[i][j][r]);
        else
          g.part[(size_t(blockIdx.y) * g.M + m) * g.N + n] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 GEMM (FMA, 64 x 64 tiles, 4 x 4 outputs per thread)
// ---------------------------------------------------------------------------

template <typename OutT>
__global__ __launch_bounds__(256) void k_gemm_tn_f32(GemmArgs g) {
  __shared__ float sa[16][65], sb[16][65];   // [k][row]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tm = blockIdx.x % g.tiles_m, tn = blockIdx.x / g.tiles_m;
  const int m0 = tm * 64, n0 = tn * 64;
  const int k_lo = blockIdx.y * g.kchunk, k_hi = min(g.K, k_lo + g.kchunk);
  const float* __restrict__ A = static_cast<const float*>(g.a);
  const float* __restrict__ B = static_cast<const float*>(g.b);
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const float* pa = A + size_t(min(m0 + lrow, g.M - 1)) * g.lda;
  const float* pb = B + size_t(min(n0 + lrow, g.N - 1)) * g.ldb;
  float acc[4][4] = {};
  for (int k0 = k_lo; k0 < k_hi; k0 += 16) {
    const int k = k0 + lk;
    const bool ok = k < k_hi;                // K % 8 == 0: four in or four out
    const float4 va = ok ? *reinterpret_cast<const float4*>(pa + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 vb = ok ? *reinterpret_cast<const float4*>(pb + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    sa[lk + 0][lrow] = va.x; sa[lk + 1][lrow] = va.y; sa[lk + 2][lrow] = va.z; sa[lk + 3][lrow] = va.w;
    sb[lk + 0][lrow] = vb.x; sb[lk + 1][lrow] = vb.y; sb[lk + 2][lrow] = vb.z; sb[lk + 3][lrow] = vb.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sb[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      if (g.splits == 1)
        store_out(static_cast<OutT*>(g.c) + size_t(m) * g.ldc + n, acc[i][j]);
      else
        g.part[(size_t(blockIdx.y) * g.M + m) * g.N + n] = acc[i][j];
    }
  }
}

// Sum of the split-K partials in slice order.
template <typename OutT>
__global__ __launch_bounds__(256) void k_splitk_sum(GemmArgs g) {
  const size_t mn = size_t(g.M) * g.N;
  for (size_t e = size_t(blockIdx.x) * 256 + threadIdx.x; e < mn; e += size_t(gridDim.x) * 256) {
    float s = 0.f;
    for (int z = 0; z < g.splits; ++z) s += g.part[z * mn + e];
    const size_t m = e / g.N, n = e % g.N;
    store_out(static_cast<OutT*>(g.c) + m * g.ldc + n, s);
  }
}

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

#ifndef HSPEC_GEMM_FORCE_CFG
#define HSPEC_GEMM_FORCE_CFG -1
#endif
constexpr int kGemmPf = HSPEC_GEMM_PF;

// bf16 tile shapes (WM, WN): cfg 0 = 64 x 128, 1 = 128 x 128, 3 = 64 x 64,
// 4 = 128 x 256, 5 = 256 x 128; cfg 2 is the fp32 kernel.
static void cfg_tile(int cfg, int& bm, int& bn) {
  static const int t[6][2] = {{64, 128}, {128, 128}, {64, 64}, {64, 64}, {128, 256}, {256, 128}};
  bm = t[cfg][0];
  bn = t[cfg][1];
}

static GemmPart gemm_part(int dtype, int M, int n0, int n, int K) {
  GemmPart p{};
  p.n0 = n0;
  p.n = n;
  if (dtype == 1) {
    p.cfg = M <= 64 ? 0 : 1;                 // 64 x 128 or 128 x 128 tiles
    if (HSPEC_GEMM_FORCE_CFG >= 0) p.cfg = HSPEC_GEMM_FORCE_CFG;
    cfg_tile(p.cfg, p.bm, p.bn);
  } else {
    p.cfg = 2;
    p.bm = p.bn = 64;
  }
  p.tiles_m = (M + p.bm - 1) / p.bm;
  p.tiles = p.tiles_m * ((n + p.bn - 1) / p.bn);
  // Slices of K until about 256 workgroups are in flight, each slice at
  // least 256 deep (a multiple of 64).
  const int want = std::max(1, std::min((256 + p.tiles - 1) / p.tiles, K / 256));
  p.kchunk = ((K + want - 1) / want + 63) / 64 * 64;
  p.splits = (K + p.kchunk - 1) / p.kchunk;
  return p;
}

// A ragged last column of tiles that would start a second round of
// workgroups on its own (the input projection at 2048 rows: 256 whole tiles
// plus 16 tiles of 80 columns) becomes a launch of its own, sliced along K,
// so the whole tiles fill the 256 CUs in one round (measured 84 -> 60 us
// for the 2048 x 2048 part).
GemmPlan gemm_plan(int dtype, int M, int N, int K) {
  GemmPlan p{};
  p.nparts = 1;
  p.part[0] = gemm_part(dtype, M, 0, N, K);
  const GemmPart& a = p.part[0];
  const int tail = N % a.bn, n_main = N - tail;
  if (dtype == 1 && tail && n_main && a.splits == 1) {
    const int rounds_all = (a.tiles + 255) / 256;
    const int rounds_main = (a.tiles_m * (n_main / a.bn) + 255) / 256;
    if (rounds_main < rounds_all) {
      p.part[0] = gemm_part(dtype, M, 0, n_main, K);
      p.part[1] = gemm_part(dtype, M, n_main, tail, K);
      p.nparts = 2;
    }
  }
  for (int i = 0; i < p.nparts; ++i)
    if (p.part[i].splits > 1)
      p.part_floats = std::max(p.part_floats, size_t(p.part[i].splits) * M * p.part[i].n);
  return p;
}

template <typename OutT>
static hipError_t launch_gemm_part(hipStream_t st, GemmArgs g, const GemmPart& p) {
  g.b = static_cast<const char*>(g.b) + size_t(p.n0) * g.ldb * (p.cfg == 2 ? 4 : 2);
  g.c = static_cast<OutT*>(g.c) + p.n0;
  g.N = p.n;
  g.tiles_m = p.tiles_m;
  g.splits = p.splits;
  g.kchunk = p.kchunk;
  const dim3 grid(p.tiles, p.splits);
  switch (p.cfg) {
    case 0: hipLaunchKernelGGL((k_gemm_tn<1, 2, OutT, kGemmPf>), grid, dim3(256), 0, st, g); break;
    case 1: hipLaunchKernelGGL((k_gemm_tn<2, 2, OutT, kGemmPf>), grid, dim3(256), 0, st, g); break;
    case 3: hipLaunchKernelGGL((k_gemm_tn<1, 1, OutT, kGemmPf>), grid, dim3(256), 0, st, g); break;
    case 4: hipLaunchKernelGGL((k_gemm_tn<2, 4, OutT, kGemmPf>), grid, dim3(256), 0, st, g); break;
    case 5: hipLaunchKernelGGL((k_gemm_tn<4, 2, OutT, kGemmPf>), grid, dim3(256), 0, st, g); break;
    default: hipLaunchKernelGGL((k_gemm_tn_f32<OutT>), grid, dim3(256), 0, st, g); break;
  }
  if (p.splits > 1) {
    const size_t mn = size_t(g.M) * g.N;
    const unsigned blocks = unsigned(std::min<size_t>((mn + 255) / 256, 4096));
    hipLaunchKernelGGL((k_splitk_sum<OutT>), dim3(blocks), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

template <typename OutT>
static hipError_t launch_gemm_out(hipStream_t st, const GemmArgs& g, const GemmPlan& p) {
  for (int i = 0; i < p.nparts; ++i) {
    const hipError_t e = launch_gemm_part<OutT>(st, g, p.part[i]);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_tn(hipStream_t st, int dtype, int out_f32, const GemmArgs& g, const GemmPlan& p) {
  if (out_f32 || dtype == 0) return launch_gemm_out<float>(st, g, p);
  return launch_gemm_out<bf16_t>(st, g, p);
}

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
