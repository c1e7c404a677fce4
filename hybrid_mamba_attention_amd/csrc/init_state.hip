// a1: initial Mamba-2 state h0 = u . W_init (H-Spec, Abstract: the Mamba
// module starts from a projection of the target's last-token hidden state).
//
// A skinny GEMM: M = C requests (1..128), N = S = H*P*N state entries
// (4096..131072), K = d_model.  Every call streams all of W_init (256 MiB to
// 1.25 GiB in bf16) once, so the kernel is HBM-bound at every C: its job is
// to keep enough W bytes in flight while the matrix cores do C flops per
// weight element.
//
// Two kernels.  k_init_wide (below) takes every bf16 call with d_model % 64
// == 0 and S % 128 == 0 -- all the model shapes.  k_init_state is the general
// one (fp32, or any d_model % 32 == 0 and S % 64 == 0):
//
// Workgroup = 16*NCL output columns x (up to) 16*MT rows; its 4 waves split
// the d_model contraction four ways (k-steps of 32 rows dealt round-robin)
// and sum their tiles through LDS at the end.  Per k-step a lane reads 8 W
// rows x NCL adjacent columns (16 lanes cover one 16*NCL-column row segment)
// off a scalar column base, transposes them in registers into NCL matrix-core
// B operands (output column n0 + NCL*(lane%16) + c of MFMA c), and takes its
// u rows as A operands.  PF k-steps of W, and of the u rows that go with them,
// are kept in flight per wave.  The u rows of a k-step are issued together with
// its W rows: vector-memory loads retire in issue order, so a u load issued
// later than a younger W load would make the matrix cores wait for that W load
// as well, and the ring would hide only one k-step of HBM latency.
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
  // lane's u rows (A operand row li of each m-tile).  Rows past the last
  // request are clamped to a real row: an MFMA output row depends only on the
  // A row of the same index, and output rows >= C are never stored, so the
  // loads stay unconditional (a branch per load would break the prefetch ring
  // into copies that drain the memory pipeline every iteration).
  const T* urow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) urow[m] = u + size_t(min(m0 + m * 16 + li, C - 1)) * d + lg * 8;

  const int nk = d >> 5;
  const int nmine = nk > wave ? (nk - wave + 3) >> 2 : 0;  // k-steps wave, wave+4, ...
  WRow<T, NCL> ring[PF][8];
  Vec8<T> aop[PF][MT];
  // k-step i of this wave into ring slot `slot`; i is clamped to the last
  // k-step, so the drain re-reads it (from L2) instead of branching.
  auto issue = [&](int i, WRow<T, NCL> (&dst)[8], Vec8<T> (&adst)[MT]) __attribute__((always_inline)) {
    const int ks = wave + 4 * min(i, nmine - 1);
    const char* base = wcol + size_t(ks) * kstep_b;
#pragma unroll
    for (int e = 0; e < 8; ++e) wload(dst[e], base + roff[e]);
#pragma unroll
    for (int m = 0; m < MT; ++m) load8(adst[m], urow[m] + ks * 32);
  };
  auto step = [&](WRow<T, NCL> (&w)[8], Vec8<T> (&ap)[MT]) __attribute__((always_inline)) {
    Vec8<T> bop[NCL];
#pragma unroll
    for (int c = 0; c < NCL; ++c) wtrans<NCL>(bop[c], w, c);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < NCL; ++c) acc[m][c] = mma8(ap[m], bop[c], acc[m][c]);
  };
  if (nmine > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) issue(p, ring[p], aop[p]);
    const int nfull = nmine - nmine % PF;
    for (int i0 = 0; i0 < nfull; i0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        step(ring[p], aop[p]);
        issue(i0 + p + PF, ring[p], aop[p]);
      }
    }
#pragma unroll
    for (int p = 0; p < PF - 1; ++p)
      if (p < nmine - nfull) step(ring[p], aop[p]);
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

// Wide variant for bf16 with d_model % 64 == 0 and S % 128 == 0: a workgroup
// covers 128 columns and up to 128 rows with 32x32x16 matrix-core tiles (one
// wave keeps those at the matrix-core peak; the 16x16x32 form needs several
// waves per SIMD to get there, and at C = 128 one wave per SIMD is all the
// accumulators allow).  Its 4 waves are 2 column halves x 2 k-halves (wave kh
// takes k-step 2j+kh of step j), so every u element a workgroup needs is
// fetched once per workgroup -- as full 128-byte rows of the 64-wide k slice
// of step j, staged through LDS -- instead of once per wave as half lines.
//
// Columns: lane (c, g) = (lane % 32, lane / 32) of wave half cg computes
// columns n0 + 2c and n0 + 2c + 1 (n-tiles 0 and 1) and holds, per k-step,
// rows 8g .. 8g+7 and 16+8g .. 16+8g+7 of those two columns as one dword per
// row: 128 contiguous bytes per row across the 32 lanes of a half-wave.
//
// Per step j: barrier; build the B operands of step j; read its A operands
// from the LDS slice buffer j & 1; MFMAs; issue the W rows and u slice of
// step j+PF into the register ring slot just freed (before the MFMAs at 128
// rows, see EARLY below); write the u slice of step j+1 into LDS
// buffer (j+1) & 1.  The u slice is loaded PF steps ahead like W, because
// loads retire in order and waiting on a later-issued u load would also wait
// on every W load issued before it.
template <int MT>  // 32-row m-tiles
struct WideCfg {
  static constexpr int ROWS = 32 * MT;                 // u rows staged per workgroup
  static constexpr int NU = ROWS / 32;                 // 16-byte u pieces per thread per step
  static constexpr int TILE = ROWS * 128;              // bytes of one staged 64-wide u slice
  static constexpr int RED = 2 * MT * 2 * 16 * 64 * 4; // k-half-1 partial tiles of 2 waves
  static constexpr int LDS = 2 * TILE > RED ? 2 * TILE : RED;
};

// EARLY: a step issues the loads of step j+PF as soon as the B operands of
// step j are built, before its MFMAs.  At 128 rows a wave's 16 MFMAs would
// otherwise hold the next loads back by ~500 cycles every step (C = 128:
// 60-63 -> 57.5 us); at 32 and 64 rows issuing after the MFMAs is faster.
//
// KS = false (wide states, enough column blocks to fill the chip twice): a
// workgroup covers 256 columns, one 64-column quarter per wave, and every
// wave takes both 32-row k-steps of each 64-row step (NKK = 2).  The u slice
// a workgroup stages then serves twice the W columns, halving the u bytes
// read per W byte, and the k-halves' sum through LDS goes away.
template <int MT, int PF, bool EARLY, bool KS = true>
__global__ __launch_bounds__(256) void k_init_wide(InitArgs a) {
  using Cfg = WideCfg<MT>;
  static_assert(PF >= 2, "the u slice of step j+1 must already be in flight");
  constexpr int NKK = KS ? 1 : 2;        // 32-row k-steps of a 64-row step per wave
  constexpr int BW = KS ? 128 : 256;     // columns per workgroup
  constexpr int LDSB = KS ? Cfg::LDS : 2 * Cfg::TILE;
  __shared__ __align__(16) char lds[LDSB];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 31, g = lane >> 5;
  const int cg = KS ? (wave & 1) : wave, kh = KS ? (wave >> 1) : 0;
  const int C = a.C, d = a.d, S = a.S;
  // 1-D grid of (S/BW) column blocks x MB row blocks.  When the column
  // blocks split evenly over the 8 XCDs, the row blocks of one column block
  // are dispatched back to back on one XCD (blocks L and L+8 share an XCD),
  // so they run together and all but the first read their W from that L2.
  const int MB = (C + Cfg::ROWS - 1) / Cfg::ROWS;
  const int nb = S / BW, L = blockIdx.x;
  int cb, mb;
  if ((nb & 7) == 0) {
    cb = (L / (8 * MB)) * 8 + (L & 7);
    mb = (L >> 3) % MB;
  } else {
    cb = L / MB;
    mb = L % MB;
  }
  const int m0 = mb * Cfg::ROWS;
  const int n0 = cb * BW + cg * 64;
  const int ns = d >> 6;
  const bf16_t* __restrict__ u = static_cast<const bf16_t*>(a.u);
  const char* __restrict__ wk = static_cast<const char*>(a.w) + (size_t(kh) * 32 * S + n0) * 2;
  const size_t step_b = size_t(64) * S * 2;  // bytes between the same wave's consecutive k-steps
  const size_t half_b = size_t(16) * S * 2;  // second half (rows 16..31) of a k-step

  f32x16 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

  uint32_t roff[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) roff[e] = uint32_t((g * 8 + e) * S + 2 * c) * 2;
  // u pieces: piece q = row * 8 + slot holds the 16 bytes of logical segment
  // slot ^ ((row / 2) & 7) of that row's 64-wide slice.  16-byte LDS reads are
  // served as 64 banks: the 16 A-operand reads of 16 consecutive rows (two
  // rows per 256 bytes) then hit 16 different bank groups; XOR by (row & 7)
  // put rows r and r + 8 on the same banks.
  const bf16_t* usrc[Cfg::NU];
  uint32_t udst[Cfg::NU];
#pragma unroll
  for (int t = 0; t < Cfg::NU; ++t) {
    const int q = int(threadIdx.x) + 256 * t;
    const int row = q >> 3, slot = q & 7;
    usrc[t] = u + size_t(min(m0 + row, C - 1)) * d + 8 * (slot ^ ((row >> 1) & 7));
    udst[t] = uint32_t(q) * 16;
  }
  // A operand of m-tile m, 32-row k-step kk, k-half h: row 32m + c, logical
  // segment k*4 + 2h + g of the slice, k = kh with the k split, kk without
  uint32_t aoff[MT][NKK][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        aoff[m][kk][h] = uint32_t(m * 32 + c) * 128 +
                         uint32_t((((KS ? kh : kk) * 4 + 2 * h + g) ^ ((c >> 1) & 7)) << 4);

  // per 32-row k-step kk: rows 8g+e (e < 8) and 16+8g+e (e >= 8) at 16kk + e, columns 2c, 2c+1
  uint32_t ring[PF][16 * NKK];
  u32x4 uring[PF][Cfg::NU];
  auto issue = [&](int j, uint32_t (&w)[16 * NKK], u32x4 (&ud)[Cfg::NU]) __attribute__((always_inline)) {
    const int jj = min(j, ns - 1);  // past the end: re-read the last step, never used
    const char* base = wk + size_t(jj) * step_b;
#pragma unroll
    for (int t = 0; t < Cfg::NU; ++t) ud[t] = *reinterpret_cast<const u32x4*>(usrc[t] + 64 * jj);
    // W is read exactly once per call: nontemporal loads
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const char* kb = base + size_t(kk) * 2 * half_b;  // rows 32kk.. of the step
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[16 * kk + e] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + roff[e]));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[16 * kk + 8 + e] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + half_b + roff[e]));
    }
  };
  auto put_u = [&](int buf, const u32x4 (&ud)[Cfg::NU]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < Cfg::NU; ++t) *reinterpret_cast<u32x4*>(lds + buf * Cfg::TILE + udst[t]) = ud[t];
  };
  auto bops = [&](const uint32_t (&w)[16 * NKK], Vec8<bf16_t> (&bop)[NKK][2][2]) __attribute__((always_inline)) {
    // B operand (k-step kk, k-half h, n-tile t): element e = W[32kk + 16h + 8g + e][n0 + 2c + t]
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t sel = t ? 0x07060302u : 0x05040100u;
          const uint32_t* r = w + 16 * kk + 8 * h;
          bop[kk][h][t].v.x = __builtin_amdgcn_perm(r[1], r[0], sel);
          bop[kk][h][t].v.y = __builtin_amdgcn_perm(r[3], r[2], sel);
          bop[kk][h][t].v.z = __builtin_amdgcn_perm(r[5], r[4], sel);
          bop[kk][h][t].v.w = __builtin_amdgcn_perm(r[7], r[6], sel);
        }
  };
  auto mmas = [&](int buf, const Vec8<bf16_t> (&bop)[NKK][2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Vec8<bf16_t> ap;
          ap.v = *reinterpret_cast<const uint4*>(lds + buf * Cfg::TILE + aoff[m][kk][h]);
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[m][t] = mma32(ap, bop[kk][h][t], acc[m][t]);
        }
  };
  static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
    issue(decltype(P)::value, ring[decltype(P)::value], uring[decltype(P)::value]);
  });
  put_u(0, uring[0]);
  // step j: W in ring[j % PF], u slice j+1 in uring[(j + 1) % PF], A of step j
  // in LDS buffer j & 1
  auto step = [&](int j, auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    __syncthreads();
    Vec8<bf16_t> bop[NKK][2][2];
    bops(ring[p], bop);
    if constexpr (EARLY) {
      issue(j + PF, ring[p], uring[p]);
      __builtin_amdgcn_sched_barrier(0);
      mmas(j & 1, bop);
    } else {
      mmas(j & 1, bop);
      issue(j + PF, ring[p], uring[p]);
    }
    put_u((j + 1) & 1, uring[(p + 1) % PF]);
  };
  const int nfull = ns - ns % PF;
  for (int j0 = 0; j0 < nfull; j0 += PF)
    static_for<0, PF>([&](auto P) __attribute__((always_inline)) { step(j0 + decltype(P)::value, P); });
  static_for<0, PF - 1>([&](auto P) __attribute__((always_inline)) {
    const int j = nfull + decltype(P)::value;
    if (j < ns) step(j, P);  // block-uniform; only the last few steps
  });

  if constexpr (!KS) {
    // no k split: every wave holds final values
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (row < C)
          *reinterpret_cast<float2*>(a.h0 + size_t(row) * S + n0 + 2 * c) = make_float2(acc[m][0][i], acc[m][1][i]);
      }
  } else {
    // k-half 1 hands its partial tile to k-half 0 through LDS
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds) + cg * (MT * 2 * 16 * 64);
    if (kh == 1) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) red[((m * 2 + t) * 16 + i) * 64 + lane] = acc[m][t][i];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v0 = acc[m][0][i] + red[((m * 2 + 0) * 16 + i) * 64 + lane];
        const float v1 = acc[m][1][i] + red[((m * 2 + 1) * 16 + i) * 64 + lane];
        const int row = m0 + m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (row < C) *reinterpret_cast<float2*>(a.h0 + size_t(row) * S + n0 + 2 * c) = make_float2(v0, v1);
      }
  }
}

template <typename T, int MT, int NCL, int PF>
static hipError_t launch_cfg(hipStream_t st, const InitArgs& a) {
  const int mblocks = (a.C + MT * 16 - 1) / (MT * 16);
  hipLaunchKernelGGL((k_init_state<T, MT, NCL, PF>), dim3(a.S / (16 * NCL), mblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int MT, int PF>
static hipError_t launch_wide(hipStream_t st, const InitArgs& a) {
  const int mb = (a.C + 32 * MT - 1) / (32 * MT);
  // 256-column blocks without the k split when they still give every CU two
  // workgroups (up to 64 rows, where two of them fit a CU at once)
  if constexpr (MT <= 2) {
    if (a.S % 256 == 0 && int64_t(a.S / 256) * mb >= 512) {
      hipLaunchKernelGGL((k_init_wide<MT, PF, (MT >= 4), false>), dim3((a.S / 256) * mb), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_init_wide<MT, PF, (MT >= 4)>), dim3((a.S / 128) * mb), dim3(256), 0, st, a);
  return hipGetLastError();
}

static bool init_uses_wide(int dtype, int d, int S) { return dtype == 1 && d % 64 == 0 && S % 128 == 0; }

hipError_t launch_init_state(hipStream_t st, int dtype, const InitArgs& a) {
  if (init_uses_wide(dtype, a.d, a.S)) {
    if (a.C <= 32) return launch_wide<1, 3>(st, a);
    if (a.C <= 64) return launch_wide<2, 3>(st, a);
    return launch_wide<4, 3>(st, a);
  }
  if (dtype == 1) {
    if (a.C <= 16) return launch_cfg<bf16_t, 1, 4, 4>(st, a);
    if (a.C <= 32) return launch_cfg<bf16_t, 2, 4, 3>(st, a);
    if (a.C <= 64) return launch_cfg<bf16_t, 4, 4, 3>(st, a);
    return launch_cfg<bf16_t, 8, 4, 3>(st, a);
  }
  if (a.C <= 16) return launch_cfg<float, 1, 4, 4>(st, a);
  if (a.C <= 32) return launch_cfg<float, 2, 4, 4>(st, a);
  if (a.C <= 64) return launch_cfg<float, 4, 4, 2>(st, a);
  return launch_cfg<float, 8, 4, 2>(st, a);
}

}  // namespace hspec
