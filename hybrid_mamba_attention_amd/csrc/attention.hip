// a0 / a3 / a4: block-query attention over the target's paged KV cache, read
// in place (H-Spec, Abstract: attention modules reuse the target KV where it
// lies; there is no drafter-side KV cache).
//
// a0  k_split_plan       one workgroup turns ctx_lens into the int32 split plan
// a3  k_block_attn       one workgroup per (work item = request x split, kv head)
// a4  k_attn_merge       log-sum-exp merge of the splits of multi-split requests
//
// k_block_attn, per workgroup of NW waves (one work item, one kv head j):
//   * The G*K query rows of kv head j (row r -> block position r / G, head
//     j*G + r % G) are split over the waves, RT tiles of 16 rows each, and
//     held in registers as matrix-core operands for the whole kernel.
//   * The item's pages stream through LDS 32 tokens (two pages) at a time:
//     every thread loads 16-byte pieces of K and V rows for the next stage
//     (16 threads cover a 256-byte row, the physical page comes from the page
//     table) while the waves compute on the current stage; one barrier per
//     stage.  LDS rows are XOR-swizzled by 16-byte chunk so that operand reads
//     are bank-conflict free.
//   * The draft block's own K keys and values ("transient intra-block KV")
//     are the last stages of the last split: they pass through the same LDS
//     buffers and are never written anywhere.
//   * S^T = K . Q^T on MFMA: lane l then holds the scores of query row l%16
//     for tokens 4*(l/16)+r of each page, so a row's softmax statistics stay
//     in the lane (two xor-shuffles give the row max, the sum is deferred).
//   * O^T += V^T . P^T on MFMA: each lane reads 8 token rows x D/16 values of
//     V and transposes them in registers; P^T is the lane's own probabilities.
//   * Each wave owns its rows across all the item's tokens, so nothing is
//     merged inside the workgroup: a single-split request writes its
//     normalised output, otherwise fp32 (m, l, O) partials go to the workspace.
#include "common.h"
#include "kernels.h"

namespace hspec {

// ---------------------------------------------------------------------------
// a0: split plan.  Layout documented in include/hspec.h.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_split_plan(const int32_t* __restrict__ ctx_lens, int C,
                                                     int max_ctx, int pps, int M,
                                                     int32_t* __restrict__ plan) {
  __shared__ int s_scan[1024];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  int32_t* n_splits = plan + 4;
  int32_t* first = plan + 4 + C;
  int32_t* req = plan + 4 + 2 * C;
  int32_t* spl = req + M;
  for (int base = 0; base < C; base += 1024) {
    const int b = base + tid;
    int ns = 0;
    if (b < C) {
      const int ctx = min(max(ctx_lens[b], 0), max_ctx);
      const int np = (ctx + 15) >> 4;
      ns = max(1, (np + pps - 1) / pps);
    }
    s_scan[tid] = ns;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int excl = s_carry + s_scan[tid] - ns;
    if (b < C) {
      n_splits[b] = ns;
      first[b] = excl;
      for (int s = 0; s < ns; ++s) {
        if (excl + s < M) {
          req[excl + s] = b;
          spl[excl + s] = s;
        }
      }
    }
    __syncthreads();
    if (tid == 1023) s_carry += s_scan[1023];
    __syncthreads();
  }
  const int total = min(s_carry, M);
  for (int i = total + tid; i < M; i += 1024) {
    req[i] = -1;
    spl[i] = -1;
  }
  if (tid == 0) {
    plan[0] = total;
    plan[1] = pps;
    plan[2] = C;
    plan[3] = M;
  }
}

// ---------------------------------------------------------------------------
// register tiles
// ---------------------------------------------------------------------------

// D/16 consecutive elements of one V row.
template <typename T, int DPL> struct VRow;
template <> struct VRow<bf16_t, 8> { uint4 v; };
template <> struct VRow<bf16_t, 4> { uint2 v; };
template <> struct VRow<float, 8> { float v[8]; };
template <> struct VRow<float, 4> { float v[4]; };

// Element cc of row r as raw 16-bit bf16 (bf16 only).
__device__ __forceinline__ uint32_t vbits(const VRow<bf16_t, 8>& r, int cc) {
  return half_of(dword_of(r.v, cc >> 1), cc & 1);
}
__device__ __forceinline__ uint32_t vbits(const VRow<bf16_t, 4>& r, int cc) {
  return half_of((cc >> 1) ? r.v.y : r.v.x, cc & 1);
}

// V^T operand for output column group cc: element e = V[token e][cc].
template <int DPL>
__device__ __forceinline__ void vtrans(Vec8<bf16_t>& o, const VRow<bf16_t, DPL> (&v)[8], int cc) {
  o.v.x = vbits(v[0], cc) | (vbits(v[1], cc) << 16);
  o.v.y = vbits(v[2], cc) | (vbits(v[3], cc) << 16);
  o.v.z = vbits(v[4], cc) | (vbits(v[5], cc) << 16);
  o.v.w = vbits(v[6], cc) | (vbits(v[7], cc) << 16);
}
template <int DPL>
__device__ __forceinline__ void vtrans(Vec8<float>& o, const VRow<float, DPL> (&v)[8], int cc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = v[e].v[cc];
}

// P^T operand: element e = probability of token e of the lane's 8 (see file head).
__device__ __forceinline__ void pack_p(Vec8<bf16_t>& o, const float (&p)[8]) {
  o.v.x = pack_bf16x2(p[0], p[1]);
  o.v.y = pack_bf16x2(p[2], p[3]);
  o.v.z = pack_bf16x2(p[4], p[5]);
  o.v.w = pack_bf16x2(p[6], p[7]);
}
__device__ __forceinline__ void pack_p(Vec8<float>& o, const float (&p)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = p[e];
}

template <typename T, int D, int RT> struct Acc {
  f32x4 o[RT][D / 16];
  float m[RT], l[RT];
};

// Geometry of one 32-token stage in LDS: rows of D elements cut into 16-byte
// chunks; chunk c of row r sits at position c ^ (r % SWZ) so that the 16
// lanes that read one chunk column of 16 different rows hit distinct banks.
template <typename T, int D> struct StageGeom {
  static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                 // chunks per row
  static constexpr int SWZ = CPR < 16 ? CPR : 16;
  static constexpr int ROWS = 32;                     // two pages
  static constexpr int TILE = ROWS * CPR;             // uint4 per tensor per stage
  __device__ static int pos(int row, int chunk) { return row * CPR + (chunk ^ (row % SWZ)); }
};

template <typename T, int D, int NW> struct AttnLds {
  using G = StageGeom<T, D>;
  static constexpr size_t bytes = size_t(2) * 2 * G::TILE * 16;  // {K,V} x double buffer
};

// Read 8 consecutive elements (chunk-aligned start `e0`) of LDS row `row`.
template <typename T, int D>
__device__ __forceinline__ void lds_read8(Vec8<T>& out, const uint4* tile, int row, int e0) {
  using G = StageGeom<T, D>;
  if constexpr (sizeof(T) == 2) {
    out.v = tile[G::pos(row, e0 / G::EPC)];
  } else {
    const uint4 a = tile[G::pos(row, e0 / G::EPC)];
    const uint4 b = tile[G::pos(row, e0 / G::EPC + 1)];
    out.v[0] = __uint_as_float(a.x); out.v[1] = __uint_as_float(a.y);
    out.v[2] = __uint_as_float(a.z); out.v[3] = __uint_as_float(a.w);
    out.v[4] = __uint_as_float(b.x); out.v[5] = __uint_as_float(b.y);
    out.v[6] = __uint_as_float(b.z); out.v[7] = __uint_as_float(b.w);
  }
}

// Read the D/16 elements starting at e0 of LDS row `row` as a V row.
template <typename T, int D>
__device__ __forceinline__ void lds_read_v(VRow<T, D / 16>& out, const uint4* tile, int row, int e0) {
  using G = StageGeom<T, D>;
  constexpr int DPL = D / 16;
  if constexpr (sizeof(T) == 2 && DPL == 8) {
    out.v = tile[G::pos(row, e0 / G::EPC)];
  } else if constexpr (sizeof(T) == 2) {  // 4 bf16 = half a chunk
    const uint2* h = reinterpret_cast<const uint2*>(tile + G::pos(row, e0 / G::EPC));
    out.v = h[(e0 % G::EPC) / 4];
  } else {
#pragma unroll
    for (int c = 0; c < DPL / 4; ++c) {
      const uint4 a = tile[G::pos(row, e0 / 4 + c)];
      out.v[4 * c + 0] = __uint_as_float(a.x);
      out.v[4 * c + 1] = __uint_as_float(a.y);
      out.v[4 * c + 2] = __uint_as_float(a.z);
      out.v[4 * c + 3] = __uint_as_float(a.w);
    }
  }
}

template <typename T, int D, int RT, int NW>
__global__ __launch_bounds__(64 * NW) void k_block_attn(AttnArgs a) {
  using Gm = StageGeom<T, D>;
  constexpr int NT = 64 * NW;
  constexpr int DS = D / 32, DPL = D / 16, EPC = Gm::EPC, CPR = Gm::CPR;
  constexpr int RPR = NT / CPR;                          // rows one load round covers
  constexpr int ROUNDS = RPR >= 32 ? 1 : 32 / RPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const int Hkv = a.Hkv;
  const int item = blockIdx.x / Hkv, j = blockIdx.x % Hkv;
  const int32_t* plan = a.plan;
  if (item >= plan[0]) return;  // uniform over the workgroup
  const int C = a.C, K = a.K, G = a.G, rows = a.rows;
  const int pps = plan[1];
  const int b = plan[4 + 2 * C + item];
  const int split = plan[4 + 2 * C + a.max_items + item];
  const int nsplit = plan[4 + b];
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int npages = (ctx + 15) >> 4;
  const int p_lo = split * pps;
  const int ncache = max(0, min(npages, p_lo + pps) - p_lo);
  const int nblk = (split == nsplit - 1) ? (K + 15) >> 4 : 0;
  const int nstage = (ncache + nblk + 1) >> 1;

  extern __shared__ __align__(16) unsigned char smem[];
  uint4* sK = reinterpret_cast<uint4*>(smem);           // [2][TILE]
  uint4* sV = sK + 2 * Gm::TILE;                        // [2][TILE]

  // this wave's query rows as B operands (row li of tile rt, d group lg + 4*ds)
  const T* __restrict__ q = static_cast<const T*>(a.q);
  Vec8<T> qv[RT][DS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + li;
    if (row < rows) {
      const int t = row / G, gg = row % G;
      const T* qp = q + ((size_t(b) * K + t) * a.Hq + j * G + gg) * D;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) load8(qv[rt][ds], qp + (lg + 4 * ds) * 8);
    } else {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) zero8(qv[rt][ds]);
    }
  }

  Acc<T, D, RT> acc;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    acc.m[rt] = -INFINITY;
    acc.l[rt] = 0.f;
#pragma unroll
    for (int cc = 0; cc < DPL; ++cc) acc.o[rt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale_log2;

  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const T* __restrict__ kbk = static_cast<const T*>(a.k_blk);
  const T* __restrict__ vbk = static_cast<const T*>(a.v_blk);
  const int32_t* __restrict__ pt = a.page_table + size_t(b) * a.max_pages;
  const int64_t head_off = int64_t(j) * a.head_stride;
  const int64_t blk_ts = int64_t(Hkv) * D;

  // page vp of this work item: context pages first, then the block's own
  // keys/values (last split only).  Returns element offsets and valid tokens.
  auto page_desc = [&](int vp, const T*& kb, const T*& vb, int64_t& ts, int& valid) {
    kb = kc;
    vb = vc;
    ts = a.token_stride;
    valid = 0;
    if (vp < ncache) {
      const int pg = p_lo + vp;
      const int phys = pt[pg];
      if (phys >= 0 && phys < a.num_pages) {
        const int64_t off = int64_t(phys) * a.page_stride + head_off;
        kb = kc + off;
        vb = vc + off;
        valid = min(16, ctx - pg * 16);
      }
    } else if (vp < ncache + nblk) {
      const int bp = vp - ncache;
      const size_t off = ((size_t(b) * K + bp * 16) * Hkv + j) * D;
      kb = kbk + off;
      vb = vbk + off;
      ts = blk_ts;
      valid = min(16, K - bp * 16);
    }
  };

  // loader role: thread -> (row0 + r*RPR, chunk)
  const int lchunk = threadIdx.x % CPR;
  const int lrow0 = threadIdx.x / CPR;
  uint4 stk[ROUNDS], stv[ROUNDS];
  auto issue = [&](int st) {
    const T *kb0, *vb0, *kb1, *vb1;
    int64_t ts0, ts1;
    int n0, n1;
    page_desc(2 * st, kb0, vb0, ts0, n0);
    page_desc(2 * st + 1, kb1, vb1, ts1, n1);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int row = lrow0 + r * RPR;
      const int tt = row >> 4, slot = row & 15;
      const T* kb = tt ? kb1 : kb0;
      const T* vb = tt ? vb1 : vb0;
      const int64_t ts = tt ? ts1 : ts0;
      const int nv = tt ? n1 : n0;
      if (row < 32 && slot < nv) {
        const int64_t off = slot * ts + lchunk * EPC;
        stk[r] = *reinterpret_cast<const uint4*>(kb + off);
        stv[r] = *reinterpret_cast<const uint4*>(vb + off);
      } else {
        stk[r] = make_uint4(0, 0, 0, 0);
        stv[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int row = lrow0 + r * RPR;
      if (row < 32) {
        sK[buf * Gm::TILE + Gm::pos(row, lchunk)] = stk[r];
        sV[buf * Gm::TILE + Gm::pos(row, lchunk)] = stv[r];
      }
    }
  };

  if (nstage > 0) issue(0);
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    commit(buf);
    int valid[2];
    {
      const T *x0, *x1;
      int64_t y;
      page_desc(2 * st, x0, x1, y, valid[0]);
      page_desc(2 * st + 1, x0, x1, y, valid[1]);
    }
    if (st + 1 < nstage) issue(st + 1);
    __syncthreads();

    const uint4* tk = sK + buf * Gm::TILE;
    const uint4* tv = sV + buf * Gm::TILE;
    // S^T = K . Q^T: A operand = token li of page tt, d group lg + 4*ds
    Vec8<T> kop[2][DS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) lds_read8<T, D>(kop[tt][ds], tk, tt * 16 + li, (lg + 4 * ds) * 8);
    float p[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) s[tt] = mma8(kop[tt][ds], qv[rt][ds], s[tt]);
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = e >> 2, r = e & 3;
        sv[e] = (4 * lg + r < valid[tt]) ? s[tt][r] : -INFINITY;
        mx = fmaxf(mx, sv[e]);
      }
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
      const float mnew = fmaxf(acc.m[rt], mx);
      const float mu = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2((acc.m[rt] - mu) * c2);
      const float nb = -mu * c2;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[rt][e] = fast_exp2(fmaf(sv[e], c2, nb));
        ls += p[rt][e];
      }
      acc.l[rt] = acc.l[rt] * alpha + ls;
      acc.m[rt] = mnew;
#pragma unroll
      for (int cc = 0; cc < DPL; ++cc) acc.o[rt][cc] *= alpha;
    }
    // O^T += V^T . P^T: lane reads 8 token rows x D/16 values, transposes in registers
    VRow<T, DPL> vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) lds_read_v<T, D>(vr[e], tv, (e >> 2) * 16 + 4 * lg + (e & 3), li * DPL);
    Vec8<T> vt[DPL];
#pragma unroll
    for (int cc = 0; cc < DPL; ++cc) vtrans<DPL>(vt[cc], vr, cc);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      Vec8<T> pv;
      pack_p(pv, p[rt]);
#pragma unroll
      for (int cc = 0; cc < DPL; ++cc) acc.o[rt][cc] = mma8(vt[cc], pv, acc.o[rt][cc]);
    }
  }

  // store: lane holds row li of each tile and d = (4*lg + r)*DPL + cc
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float lsum = wave_xor_sum(acc.l[rt], 16);
    lsum = wave_xor_sum(lsum, 32);
    const int row = (wave * RT + rt) * 16 + li;
    if (row >= rows) continue;
    if (nsplit == 1) {
      const int t = row / G, gg = row % G;
      T* o = static_cast<T*>(a.out) + ((size_t(b) * K + t) * a.Hq + j * G + gg) * D;
      const float inv = 1.f / lsum;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        T* dst = o + (4 * lg + r) * DPL;
        if constexpr (sizeof(T) == 2) {
          if constexpr (DPL == 8) {
            uint4 w;
            w.x = pack_bf16x2(acc.o[rt][0][r] * inv, acc.o[rt][1][r] * inv);
            w.y = pack_bf16x2(acc.o[rt][2][r] * inv, acc.o[rt][3][r] * inv);
            w.z = pack_bf16x2(acc.o[rt][4][r] * inv, acc.o[rt][5][r] * inv);
            w.w = pack_bf16x2(acc.o[rt][6][r] * inv, acc.o[rt][7][r] * inv);
            *reinterpret_cast<uint4*>(dst) = w;
          } else {
            uint2 w;
            w.x = pack_bf16x2(acc.o[rt][0][r] * inv, acc.o[rt][1][r] * inv);
            w.y = pack_bf16x2(acc.o[rt][2][r] * inv, acc.o[rt][3][r] * inv);
            *reinterpret_cast<uint2*>(dst) = w;
          }
        } else {
#pragma unroll
          for (int cc = 0; cc < DPL; cc += 4)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + cc) =
                make_float4(acc.o[rt][cc][r] * inv, acc.o[rt][cc + 1][r] * inv,
                            acc.o[rt][cc + 2][r] * inv, acc.o[rt][cc + 3][r] * inv);
        }
      }
    } else {
      const size_t prow = (size_t(item) * Hkv + j) * rows + row;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = po + (4 * lg + r) * DPL;
#pragma unroll
        for (int cc = 0; cc < DPL; cc += 4)
          *reinterpret_cast<float4*>(dst + cc) =
              make_float4(acc.o[rt][cc][r], acc.o[rt][cc + 1][r], acc.o[rt][cc + 2][r], acc.o[rt][cc + 3][r]);
      }
      if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(acc.m[rt], lsum);
    }
  }
}

// ---------------------------------------------------------------------------
// a4: merge of split partials (requests with more than one split only)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int Hkv = a.Hkv;
  const int b = blockIdx.x / Hkv, j = blockIdx.x % Hkv;
  const int32_t* plan = a.plan;
  const int C = a.C;
  const int ns = plan[4 + b];
  if (ns <= 1) return;
  const int first = plan[4 + C + b];
  const int rows = a.rows, G = a.G, K = a.K;
  const float c2 = a.scale_log2;
  for (int idx = threadIdx.x; idx < rows * (D / 4); idx += 256) {
    const int row = idx / (D / 4), d4 = idx % (D / 4);
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
      M = fmaxf(M, a.part_ml[((size_t(first + s) * Hkv + j) * rows + row) * 2]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    float4 accv = make_float4(0, 0, 0, 0);
    float Ls = 0.f;
    for (int s = 0; s < ns; ++s) {
      const size_t prow = (size_t(first + s) * Hkv + j) * rows + row;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + prow * 2);
      const float f = fast_exp2((ml.x - mu) * c2);
      const float4 v = reinterpret_cast<const float4*>(a.part_o + prow * D)[d4];
      accv.x += f * v.x;
      accv.y += f * v.y;
      accv.z += f * v.z;
      accv.w += f * v.w;
      Ls += f * ml.y;
    }
    const float inv = 1.f / Ls;
    const int t = row / G, gg = row % G;
    T* o = static_cast<T*>(a.out) + ((size_t(b) * K + t) * a.Hq + j * G + gg) * D + d4 * 4;
    if constexpr (sizeof(T) == 2) {
      uint2 w;
      w.x = pack_bf16x2(accv.x * inv, accv.y * inv);
      w.y = pack_bf16x2(accv.z * inv, accv.w * inv);
      *reinterpret_cast<uint2*>(o) = w;
    } else {
      *reinterpret_cast<float4*>(o) = make_float4(accv.x * inv, accv.y * inv, accv.z * inv, accv.w * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
// (RT row tiles per wave, NW waves) for a query-row count: every wave reads the
// whole stage from LDS, so fewer, wider waves cut LDS traffic per HBM byte.
template <typename T, int D, int RT, int NW>
static hipError_t launch_attn_cfg(hipStream_t st, const AttnArgs& a) {
  const size_t lds = AttnLds<T, D, NW>::bytes;
  auto kern = k_block_attn<T, D, RT, NW>;
  hipLaunchKernelGGL(kern, dim3(a.max_items * a.Hkv), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(hipStream_t st, const AttnArgs& a) {
  if (a.rows <= 16) return launch_attn_cfg<T, D, 1, 1>(st, a);
  if (a.rows <= 32) return launch_attn_cfg<T, D, 1, 2>(st, a);
  if (a.rows <= 64) return launch_attn_cfg<T, D, 1, 4>(st, a);
  if (a.rows <= 128) return launch_attn_cfg<T, D, 2, 4>(st, a);
  return launch_attn_cfg<T, D, 4, 4>(st, a);
}

size_t attn_lds_bytes(int dtype, int D, int rows, int K) {
  (void)rows;
  (void)K;
  if (dtype == 1) return D == 64 ? AttnLds<bf16_t, 64, 4>::bytes : AttnLds<bf16_t, 128, 4>::bytes;
  return D == 64 ? AttnLds<float, 64, 4>::bytes : AttnLds<float, 128, 4>::bytes;
}

hipError_t launch_block_attn(hipStream_t st, int dtype, const AttnArgs& a, int pps) {
  hipLaunchKernelGGL(k_split_plan, dim3(1), dim3(1024), 0, st, a.ctx_lens, a.C, a.max_ctx, pps,
                     a.max_items, const_cast<int32_t*>(a.plan));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1) {
    e = a.D == 64 ? launch_attn_d<bf16_t, 64>(st, a) : launch_attn_d<bf16_t, 128>(st, a);
  } else {
    e = a.D == 64 ? launch_attn_d<float, 64>(st, a) : launch_attn_d<float, 128>(st, a);
  }
  if (e != hipSuccess) return e;
  if (a.max_items > a.C) {  // some request may have several splits
    if (dtype == 1) {
      if (a.D == 64) hipLaunchKernelGGL((k_attn_merge<bf16_t, 64>), dim3(a.C * a.Hkv), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((k_attn_merge<bf16_t, 128>), dim3(a.C * a.Hkv), dim3(256), 0, st, a);
    } else {
      if (a.D == 64) hipLaunchKernelGGL((k_attn_merge<float, 64>), dim3(a.C * a.Hkv), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((k_attn_merge<float, 128>), dim3(a.C * a.Hkv), dim3(256), 0, st, a);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace hspec
