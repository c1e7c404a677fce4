// Matrix-core GEMM shared by the Mamba-2 block's projections and the
// drafter-side KV injection (the contrast workload).
//
// k_gemm_tn computes C[M,N] = A[M,K] . B[N,K]^T with both operands contiguous
// along K (weights in the [out, in] convention), which is exactly the operand
// layout of the bf16 matrix cores: a lane's eight contraction-adjacent
// elements are one 16-byte row piece.
//   * Workgroup: NWR x 2 waves over a (32*WM*NWR) x (64*WN) output tile;
//     each wave owns WM x WN tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16, fp32
//     accumulation in registers).  64 x 128 tiles: 4 waves (one per SIMD).
//     128 x 128 tiles: 8 waves of 32 x 64 outputs, two per SIMD, so one
//     wave's MFMAs run while the other waits on LDS, its loads or the
//     barrier; at 2048 rows that took the 2048 x 2048 x 4096 part of the
//     Mamba-2 input projection from 56 to 45 us and the block from 132 to
//     118 us against 4 waves of 64 x 64 (a 4-stage load ring on top: 122 us).
//   * K advances 64 at a time.  Every thread issues 16-byte loads of A and B
//     row pieces for the stage PF ahead into a register ring; a stage is then
//     written to one of two LDS buffers, one barrier, and the waves run their
//     MFMAs on it.  LDS rows are 128 bytes with the 16-byte piece index XORed
//     by ((row / 2) % 8): 16 lanes of a 16-byte read (32 consecutive rows per
//     half-wave) then cover the 64 banks once, and so do the stores (two rows
//     of eight pieces).  XOR by (row % 8) suits 32 banks and measured 2-way
//     conflicts on every operand read here.
//   * Rows of A or B past M or N repeat the last row (their results are never
//     stored); contraction indices past K load zeros.
//   * Split-K: blockIdx.y takes one slice of K.  With more than one slice the
//     kernel stores fp32 partials and k_splitk_sum adds them in slice order,
//     so results are repeatable bit for bit.
// fp32 activations take k_gemm_tn_f32, a plain LDS-tiled FMA kernel.
// Epilogue: the result goes to a row-major output, or (KV injection) each
// row m = request b * n_new + i is written as K | V rows of token position
// start[b] + i into paged pools through the page table.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hspec {

// Paged destination of output row m (-1: the position has no page, so the
// row is not written), and of output column n (which pool, offset).
__device__ __forceinline__ int64_t scatter_row(const KvScatter& s, int m) {
  const int b = m / s.n_new, p = s.start[b] + (m - b * s.n_new);
  if (p < 0 || (p >> s.lpt) >= s.max_pages) return -1;
  const int page = s.page_table[size_t(b) * s.max_pages + (p >> s.lpt)];
  if (page < 0 || page >= s.num_pages) return -1;
  return int64_t(page) * s.ps + int64_t(p & ((1 << s.lpt) - 1)) * s.ts;
}
// n: column of this launch (the projection column is s.col0 + n)
template <typename OutT>
__device__ __forceinline__ OutT* scatter_col(const KvScatter& s, int n) {
  n += s.col0;
  const bool v = n >= s.HD;
  const int nn = v ? n - s.HD : n;
  return static_cast<OutT*>(v ? s.v_cache : s.k_cache) + int64_t(nn / s.D) * s.hs + nn % s.D;
}

// ---------------------------------------------------------------------------
// bf16 GEMM on matrix cores
// ---------------------------------------------------------------------------

template <int WM, int WN, typename OutT, int PF, int NWR = 2>
__global__ __launch_bounds__(128 * NWR) void k_gemm_tn(GemmArgs g) {
  constexpr int NT = 128 * NWR;                    // threads
  constexpr int RPP = NT / 8;                      // rows one load pass covers
  constexpr int BM = 32 * WM * NWR, BN = 64 * WN;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "whole load passes");
  constexpr int LA = BM / RPP, LB = BN / RPP;      // 16-byte loads per thread per stage
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

  // loader: thread -> 16-byte piece lc of rows lr + RPP*i
  const int lc = tid & 7, lr = tid >> 3;
  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.a);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.b);
  const bf16_t* pa[LA];
  const bf16_t* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) pa[i] = A + size_t(min(m0 + lr + RPP * i, g.M - 1)) * g.lda;
#pragma unroll
  for (int i = 0; i < LB; ++i) pb[i] = B + size_t(min(n0 + lr + RPP * i, g.N - 1)) * g.ldb;
  uint32_t wpos[LA > LB ? LA : LB];
#pragma unroll
  for (int i = 0; i < (LA > LB ? LA : LB); ++i) {
    const int r = lr + RPP * i;
    wpos[i] = r * 128 + ((lc ^ ((r >> 1) & 7)) << 4);
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
  // ks are issued, so LDS latency hides behind matrix work.  `mid` (the next
  // stage's LDS write and loads) runs after the third k-step's MFMAs, where
  // its instructions interleave with the remaining matrix work instead of
  // following it with the matrix pipe idle.
  auto compute = [&](int buf, auto&& mid) __attribute__((always_inline)) {
    const unsigned char* ta = sA + buf * TA;
    const unsigned char* tb = sB + buf * TB;
    Vec8<bf16_t> ao[2][WM], bo[2][WN];
    auto read = [&](int ks, Vec8<bf16_t> (&a)[WM], Vec8<bf16_t> (&b)[WN]) __attribute__((always_inline)) {
      const int pc = 2 * ks + ohalf;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr * 32 * WM + 32 * i + orow;
        a[i].v = *reinterpret_cast<const uint4*>(ta + r * 128 + ((pc ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = wc * 32 * WN + 32 * j + orow;
        b[j].v = *reinterpret_cast<const uint4*>(tb + r * 128 + ((pc ^ ((r >> 1) & 7)) << 4));
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
      if constexpr (ks == 2) mid();
    });
  };

  // Stage st: barrier, MFMAs on LDS buffer st&1; during its last k-steps,
  // stage st+1 goes from its register slot into buffer (st+1)&1 (last read by
  // stage st-1, which every wave finished before this barrier) and stage
  // st+1+PF is issued into the freed slot.  The wait for stage st+1's loads
  // thus comes after most of stage st's MFMAs are queued.  Every slot issues its loads, also past the
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
      compute(pp & 1, [&]() __attribute__((always_inline)) {
        commit(st0 + pp + 1, (pp + 1) & 1, ra[nx], rb[nx]);
        issue(st0 + pp + 1 + PF, ra[nx], rb[nx]);
      });
    });
  }
  static_for<0, PF - 1>([&](auto P) __attribute__((always_inline)) {
    constexpr int pp = decltype(P)::value;
    constexpr int nx = (pp + 1) % PF;
    if (nfull + pp < nst) {   // uniform over the workgroup
      __syncthreads();
      compute(pp & 1, [] {});
      commit(nfull + pp + 1, (pp + 1) & 1, ra[nx], rb[nx]);
    }
  });

  // result element r of tile (i, j): column 32j + l%32, row 32i + 8(r/4) + 4(l/32) + r%4
  if (g.scatter && g.splits == 1) {
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      int64_t roff[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wr * 32 * WM + 32 * i + 8 * (r >> 2) + 4 * ohalf + (r & 3);
        roff[r] = m < g.M ? scatter_row(g.sc, m) : -1;
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int n = n0 + wc * 32 * WN + 32 * j + orow;
        if (n >= g.N) continue;
        OutT* col = scatter_col<OutT>(g.sc, n);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (roff[r] >= 0) store_out(col + roff[r], acc[i][j][r]);
      }
    }
    return;
  }
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
      if (g.splits == 1 && g.scatter) {
        const int64_t ro = scatter_row(g.sc, m);
        if (ro >= 0) store_out(scatter_col<OutT>(g.sc, n) + ro, acc[i][j]);
      } else if (g.splits == 1)
        store_out(static_cast<OutT*>(g.c) + size_t(m) * g.ldc + n, acc[i][j]);
      else
        g.part[(size_t(blockIdx.y) * g.M + m) * g.N + n] = acc[i][j];
    }
  }
}

// Sum of the split-K partials in slice order, V consecutive columns per
// thread (V = 4 needs N % 4 == 0; the head size, a multiple of 8, keeps four
// scatter columns in one head).  The slices are loaded eight at a time, all
// issued before the first add (clamped slice index; the sum skips the
// repeats): a load per loop trip would wait out one memory round trip per
// slice, which dominated this kernel at small M.
template <typename OutT, int V>
__global__ __launch_bounds__(256) void k_splitk_sum(GemmArgs g) {
  using VecF = typename std::conditional<V == 4, float4, float>::type;
  const size_t mn = size_t(g.M) * g.N;
  const size_t nq = mn / V;
  const int ns = g.splits;
  for (size_t q = size_t(blockIdx.x) * 256 + threadIdx.x; q < nq; q += size_t(gridDim.x) * 256) {
    const size_t e = q * V;
    float s[V];
#pragma unroll
    for (int v = 0; v < V; ++v) s[v] = 0.f;
    for (int z0 = 0; z0 < ns; z0 += 8) {
      VecF x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        x[u] = *reinterpret_cast<const VecF*>(g.part + size_t(min(z0 + u, ns - 1)) * mn + e);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (z0 + u < ns) {   // uniform
          const float* xv = reinterpret_cast<const float*>(&x[u]);
#pragma unroll
          for (int v = 0; v < V; ++v) s[v] += xv[v];
        }
      }
    }
    const size_t m = e / g.N, n = e % g.N;
    OutT* dst;
    if (g.scatter) {
      const int64_t ro = scatter_row(g.sc, int(m));
      if (ro < 0) continue;
      dst = scatter_col<OutT>(g.sc, int(n)) + ro;
    } else {
      dst = static_cast<OutT*>(g.c) + m * g.ldc + n;
    }
    if constexpr (V == 4) {
      store_out4(dst, make_float4(s[0], s[1], s[2], s[3]));
    } else {
      store_out(dst, s[0]);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Stages of loads in flight per thread.  Four (checked in the ISA: the
// steady loop then waits at vmcnt(24)) measured no faster than two.
constexpr int kGemmPf = 2;

// bf16 tile shapes: cfg 0 = 64 x 128 (4 waves), 1 = 128 x 128 (8 waves);
// cfg 2 is the fp32 kernel (64 x 64).
static void cfg_tile(int cfg, int& bm, int& bn) {
  static const int t[3][2] = {{64, 128}, {128, 128}, {64, 64}};
  bm = t[cfg][0];
  bn = t[cfg][1];
}

static GemmPart gemm_part(int dtype, int M, int n0, int n, int K) {
  GemmPart p{};
  p.n0 = n0;
  p.n = n;
  if (dtype == 1) {
    p.cfg = M <= 64 ? 0 : 1;                 // 64 x 128 or 128 x 128 tiles
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
  g.sc.col0 = p.n0;   // scatter targets are looked up by projection column
  g.N = p.n;
  g.tiles_m = p.tiles_m;
  g.splits = p.splits;
  g.kchunk = p.kchunk;
  const dim3 grid(p.tiles, p.splits);
  switch (p.cfg) {
    case 0: hipLaunchKernelGGL((k_gemm_tn<1, 2, OutT, kGemmPf>), grid, dim3(256), 0, st, g); break;
    case 1: hipLaunchKernelGGL((k_gemm_tn<1, 2, OutT, kGemmPf, 4>), grid, dim3(512), 0, st, g); break;
    default: hipLaunchKernelGGL((k_gemm_tn_f32<OutT>), grid, dim3(256), 0, st, g); break;
  }
  if (p.splits > 1) {
    // four columns per thread: whole 16-byte partial pieces, and output
    // columns that stay in one row (or one head of one pool) at 4-element
    // aligned addresses
    auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    const bool v4 = g.N % 4 == 0 &&
                    (g.scatter ? g.sc.D % 4 == 0 && al16(g.sc.k_cache) && al16(g.sc.v_cache)
                               : g.ldc % 4 == 0 && al16(g.c));
    const size_t nq = size_t(g.M) * g.N / (v4 ? 4 : 1);
    const unsigned blocks = unsigned(std::min<size_t>((nq + 255) / 256, 4096));
    if (v4)
      hipLaunchKernelGGL((k_splitk_sum<OutT, 4>), dim3(blocks), dim3(256), 0, st, g);
    else
      hipLaunchKernelGGL((k_splitk_sum<OutT, 1>), dim3(blocks), dim3(256), 0, st, g);
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

}  // namespace hspec
