// a0 / a3 / a4: block-query attention over the target's paged KV cache, read
// in place (H-Spec, Abstract: attention modules reuse the target KV where it
// lies; there is no drafter-side KV cache).
//
// a3  k_block_attn       one workgroup per (work range, kv head), or per (work
//                        range, pair of adjacent kv heads) with long ranges;
//                        one more workgroup writes the int32 work plan (a0)
// a4  k_attn_merge       log-sum-exp merge of the pieces of requests that
//                        span more than one range
//
// Work plan (a0).  Each request's keys are its context, in slabs of 16
// tokens, followed by its K block keys (nbk slabs), counted in granules of
// `gran` slabs (max(2, slabs per page), from the request's start, so a
// granule boundary starts a page and an even slab).  Automatic ranges also
// charge each request `seg` units of fixed cost placed before its keys (the
// segment's prologue, general-path tail and store); the batch's units,
// request after request, are cut into W nearly equal ranges (B_w =
// floor(w * T / W)); a workgroup takes its range's slabs request by request
// (segments).  Long and short requests thus cost the same wall time: ragged
// batches keep every workgroup busy for about the same time.  Every
// workgroup derives the plan from ctx_lens itself (a block scan over the
// requests); a segment that is a whole request writes its normalised output,
// one that is a piece of a longer request writes fp32 (m, l, O) to slot
// 2w + k of the workspace (k = 0 for the segment starting at the range's
// first granule, 1 for the one starting later), and k_attn_merge combines
// the pieces.  The plan in the workspace lists the same decomposition for
// the merge, callers and tests.
//
// k_block_attn, per workgroup of NW waves (one range, HP = 1 or 2 kv heads):
//   * The G*K query rows of kv head j (row r -> block position r / G, head
//     j*G + r % G) are split over NW/HP waves, RT tiles of 16 rows each, and
//     held in registers as matrix-core operands for a whole segment.  With
//     HP = 2 (NHD pools, ranges of 32+ slabs) a stage row is the 2D-wide
//     piece of both heads, 512 bytes for bf16 D = 128, and each half of the
//     waves computes on its own head's columns.
//   * A segment's slabs stream through LDS 32 tokens (two slabs) at a time:
//     every thread loads 16-byte pieces of K and V rows for the next stage
//     (16 threads cover a 256-byte row, 32 a 512-byte head-pair row; the
//     physical page comes from the page table) while the waves compute on the
//     current stage; one barrier per stage.  LDS rows are XOR-swizzled by
//     16-byte chunk so that operand reads are bank-conflict free.
//   * The draft block's own K keys and values ("transient intra-block KV")
//     are the last slabs of a request's keys: they pass through the same LDS
//     buffers and are never written anywhere.  With the block-causal mask,
//     those stages also drop block key s for query rows at block position
//     t < s; context pages are never masked.
//   * S^T = K . Q^T on MFMA: lane l then holds the scores of query row l%16
//     for tokens 4*(l/16)+r of each page, so a row's softmax statistics stay
//     in the lane (two xor-shuffles give the row max, the sum is deferred).
//   * O^T += V^T . P^T on MFMA: each lane reads 8 token rows x D/16 values of
//     V and transposes them in registers; P^T is the lane's own probabilities.
//   * Each wave owns its rows across all of a segment's tokens, so nothing is
//     merged inside the workgroup.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "merge.h"

namespace hspec {

// 16 bytes of a K/V row, which each call reads exactly once: a nontemporal
// load.  Measured on a 4 GiB stream, nontemporal 16-byte loads sustain ~3%
// more than plain ones, and in this kernel they cut the C = 128 time by 13%
// (the cache lines of a one-time stream stop displacing everything else).
__device__ __forceinline__ uint4 ld_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// a0: the work plan (include/hspec.h documents the layout)
// ---------------------------------------------------------------------------

__device__ __forceinline__ int ctx_of(const AttnArgs& a, int b) { return min(max(a.ctx_lens[b], 0), a.max_ctx); }

// Granules of a request's keys: ceil(ctx / 16) context slabs, then the block's.
__device__ __forceinline__ int req_granules(const AttnArgs& a, int ctx) {
  return (((ctx + 15) >> 4) + a.nbk + a.gran - 1) / a.gran;
}

// Ranges for a batch of T granules (T >= C >= 1, so W <= T: no range is
// empty): fixed ranges of range_gran granules (the last one shorter), or W
// nearly equal ranges of at least min_gran granules each (one range when
// the batch has fewer).  The host sizes w_max for the fixed form's count.
__device__ __forceinline__ int range_count(const AttnArgs& a, int T) {
  const int W = a.range_gran > 0 ? (T + a.range_gran - 1) / a.range_gran : T / a.min_gran;
  return max(1, min(W, a.w_max));
}
// B_w, the first granule of range w (B_W = T)
__device__ __forceinline__ int range_bound(const AttnArgs& a, int w, int T, int W) {
  return a.range_gran > 0 ? int(min(int64_t(w) * a.range_gran, int64_t(T))) : int(int64_t(w) * T / W);
}
// The range holding granule x < T: the largest w with B_w <= x.
__device__ __forceinline__ int range_of(const AttnArgs& a, int x, int T, int W) {
  if (a.range_gran > 0) return x / a.range_gran;
  return int((int64_t(x + 1) * W + T - 1) / T) - 1;   // floor(w*T/W) <= x  <=>  w < (x+1)*W/T
}

// Inclusive prefix sum of v over the workgroup's NT threads (NT / 64 waves;
// lds[0 .. NT/64) is scratch); *total receives the sum.  Every thread calls it.
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int t = lds[i];
    before += i < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return x + before;
}

// The batch's total units T = sum (seg + G_b) (every thread; lds as
// block_incl_scan).  g0 receives this thread's request granules G_b of the
// first chunk (requests 0 .. NT-1), which a second pass over a batch of
// C <= NT then reuses.
template <int NT>
__device__ __forceinline__ int batch_granules(const AttnArgs& a, int* lds, int* g0) {
  int part = 0;
  *g0 = 0;
  for (int base = 0; base < a.C; base += NT) {
    const int b = base + int(threadIdx.x);
    const int gb = b < a.C ? req_granules(a, ctx_of(a, b)) : 0;
    if (base == 0) *g0 = gb;
    part += b < a.C ? gb + a.seg : 0;
  }
  int T;
  block_incl_scan<NT>(part, lds, &T);
  return T;
}

// Written by the grid's last workgroup, which does nothing else: W, the
// units S_b where the requests' keys start, each request's first range and
// piece count, and the range bounds B_0 .. B_W (-1 past W up to the capacity).
template <int NT>
__device__ void write_plan(const AttnArgs& a, int* lds) {
  const int tid = threadIdx.x, C = a.C;
  int32_t* plan = a.plan;
  int g0;
  const int T = batch_granules<NT>(a, lds, &g0);
  const int W = range_count(a, T);
  int carry = 0;
  for (int base = 0; base < C; base += NT) {
    const int b = base + tid;
    const int gb = base == 0 ? g0 : (b < C ? req_granules(a, ctx_of(a, b)) : 0);
    int tot;
    const int incl = carry + block_incl_scan<NT>(b < C ? gb + a.seg : 0, lds, &tot);
    if (b < C) {
      const int S = incl - gb;   // the fixed cost comes first
      const int wf = range_of(a, S, T, W), wl = range_of(a, incl - 1, T, W);
      plan[4 + b] = S;
      plan[4 + C + b] = wf;
      plan[4 + 2 * C + b] = wl - wf + 1;
    }
    carry += tot;
  }
  int32_t* bounds = plan + 4 + 3 * C;
  for (int w = tid; w <= a.w_max; w += NT) bounds[w] = w <= W ? range_bound(a, w, T, W) : -1;
  if (tid == 0) {
    plan[0] = W;
    plan[1] = a.gran;
    plan[2] = C;
    plan[3] = a.w_max;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (no LDS, no barrier).
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Where range w starts: the request b whose units (fixed cost, then keys)
// hold the range's first unit B0, the unit S where that request's keys start
// and its context length (uniform over the workgroup; b = -1 when w >= W).
struct RangeStart {
  int W, T, B0, B1, b, S, ctx;
};
template <int NT>
__device__ RangeStart find_range(const AttnArgs& a, int w, int* lds) {
  const int tid = threadIdx.x, C = a.C;
  RangeStart r;
  if (C <= 64) {
    // One wave holds the whole batch: every wave scans it on its own, with
    // lane ops only, so no barrier and no LDS round trip delays the stream.
    const int lane = tid & 63;
    const int ctx = lane < C ? ctx_of(a, lane) : 0;
    const int gb = lane < C ? req_granules(a, ctx) : 0;
    const int gv = lane < C ? gb + a.seg : 0;
    const int incl = wave_incl_scan(gv);
    r.T = __builtin_amdgcn_readlane(incl, 63);
    r.W = range_count(a, r.T);
    r.b = -1;
    r.S = 0;
    r.ctx = 0;
    if (w >= r.W) return r;
    r.B0 = range_bound(a, w, r.T, r.W);
    r.B1 = range_bound(a, w + 1, r.T, r.W);
    const uint64_t hit = __ballot(lane < C && incl - gv <= r.B0 && r.B0 < incl);
    if (hit == 0) return r;   // cannot happen: B0 < T lies in some request
    const int fb = __ffsll(static_cast<long long>(hit)) - 1;   // exactly one lane
    r.b = fb;
    r.S = __builtin_amdgcn_readlane(incl - gb, fb);
    r.ctx = __builtin_amdgcn_readlane(ctx, fb);
    return r;
  }
  int g0;
  r.T = batch_granules<NT>(a, lds, &g0);
  r.W = range_count(a, r.T);
  r.b = -1;
  r.S = 0;
  if (w >= r.W) return r;
  r.B0 = range_bound(a, w, r.T, r.W);
  r.B1 = range_bound(a, w + 1, r.T, r.W);
  r.ctx = 0;
  int* found = lds + 16;   // past block_incl_scan's scratch
  if (tid == 0) found[0] = -1;
  int carry = 0;
  for (int base = 0; base < C; base += NT) {
    const int b = base + tid;
    const int gb = base == 0 ? g0 : (b < C ? req_granules(a, ctx_of(a, b)) : 0);
    const int gv = b < C ? gb + a.seg : 0;
    int tot;
    const int incl = carry + block_incl_scan<NT>(gv, lds, &tot);  // (its barriers order found[0] = -1)
    if (b < C && incl - gv <= r.B0 && r.B0 < incl) {   // exactly one thread of the batch
      found[0] = b;
      found[1] = incl - gb;
    }
    __syncthreads();
    const int fb = found[0];
    if (fb >= 0) {
      r.b = __builtin_amdgcn_readfirstlane(fb);
      r.S = __builtin_amdgcn_readfirstlane(found[1]);
      break;
    }
    carry += tot;
  }
  r.ctx = r.b >= 0 ? ctx_of(a, r.b) : 0;
  return r;
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

// V^T operand for output column group cc: element e = V[token e][cc].  For
// bf16 each dword pairs the same column of two tokens: one v_perm_b32.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {  // a.lo | b.lo << 16
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {  // a.hi | b.hi << 16
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
template <int DPL>
__device__ __forceinline__ void vtrans(Vec8<bf16_t>& o, const VRow<bf16_t, DPL> (&v)[8], int cc) {
  auto dw = [&](int e) -> uint32_t {
    if constexpr (DPL == 8) return dword_of(v[e].v, cc >> 1);
    else return (cc >> 1) ? v[e].v.y : v[e].v.x;
  };
  if (cc & 1) {
    o.v.x = pair_hi(dw(0), dw(1)); o.v.y = pair_hi(dw(2), dw(3));
    o.v.z = pair_hi(dw(4), dw(5)); o.v.w = pair_hi(dw(6), dw(7));
  } else {
    o.v.x = pair_lo(dw(0), dw(1)); o.v.y = pair_lo(dw(2), dw(3));
    o.v.z = pair_lo(dw(4), dw(5)); o.v.w = pair_lo(dw(6), dw(7));
  }
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

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48 hold the same query row): gfx950 lane-swap instructions, no LDS.
__device__ __forceinline__ float group4_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <typename T, int D, int RT> struct Acc {
  f32x4 o[RT][D / 16];
  float m2[RT], l[RT];  // running max in log2 units (score * scale * log2 e), running sum
};

// Geometry of one 32-token stage in LDS: rows of D elements cut into 16-byte
// chunks; chunk c of row r sits at position c ^ (r % SWZ) so that the 16
// lanes that read one chunk column of 16 different rows hit distinct banks.
template <typename T, int D> struct StageGeom {
  static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                 // chunks per row
  static constexpr int SWZ = CPR < 16 ? CPR : 16;
  static constexpr int ROWS = 32;                     // two pages
  static constexpr int TILE = ROWS * CPR;             // 16-byte chunks per tensor per stage
  __host__ __device__ static constexpr int pos(int row, int chunk) { return row * CPR + (chunk ^ (row % SWZ)); }
};

// The 16-byte d-chunk of its head that V-operand lane li reads (bf16,
// D = 128, where each lane reads one chunk of each token row).
// ds_read_b128 serves a wave in four passes of 16 lanes: the lanes that share
// bit 5 and the parity of bits 2..4 (lanes 0-3, 12-15, 20-23 and 24-27 form
// one pass, as an LDS access-pattern probe of this GPU measures).  A V read
// puts lane groups lg = 2m and 2m+1 (token rows 4lg + e) in each pass; with
// chunk li, the row swizzle maps the two groups' lanes onto the same eight
// bank groups (a 2-way conflict on every V read).  Here lanes 0-3 and 12-15
// read chunks 0-7 and lanes 4-11 chunks 8-15, so the two groups of a pass
// cover all sixteen bank groups.  The stage layout is unchanged; the output
// rows follow the same permutation (d = vchunk(i) * 8 + cc).
__host__ __device__ constexpr int vchunk(int i) {
  return (i & 3) | ((((i >> 2) ^ (i >> 3)) & 1) << 3) | (((i >> 3) & 1) << 2);
}

template <typename T, int D> struct AttnLds {
  using G = StageGeom<T, D>;
  static constexpr size_t bytes = size_t(2) * 2 * G::TILE * 16;  // {K,V} x double buffer
};

// Rescale threshold (log2 units): the running max is only moved when a new
// score exceeds it by more than this, so probabilities stay <= 2^8 and the
// accumulators are rescaled rarely.
constexpr float kRescaleLog2 = 8.f;

// bf16 with two row tiles per wave (128 query rows per head) is held to two
// waves per SIMD: it needs 259 registers unbounded, 256 with three spilled
// (workload 4: 665 -> 559 us).  fp32 would spill hundreds, so it is not bound.
template <typename T, int D, int RT, int NW, int PF, int HP>
__global__ __launch_bounds__(64 * NW, (RT == 2 && sizeof(T) == 2) ? 2 : 1) void k_block_attn(AttnArgs a) {
  // HP kv heads per workgroup (1 or 2): with 2, heads j0 and j0+1 are
  // adjacent in every token row (head stride D), so a stage's rows are 2D
  // elements (one 512-byte piece per token for bf16, D = 128) and the waves
  // split by head, NW/2 per head.
  using Gm = StageGeom<T, HP * D>;
  constexpr int WPH = NW / HP;  // waves per head
  static_assert(HP == 1 || HP == 2, "one or two kv heads per workgroup");
  constexpr int NT = 64 * NW;
  constexpr int DS = D / 32, DPL = D / 16, EPC = Gm::EPC, CPR = Gm::CPR;
  constexpr int TPR = NT / CPR;                          // loader thread rows
  // Page split: with 32 thread rows (8 waves on 256-byte rows, or 4 on
  // 128-byte rows) rows 0-15 load the stage's first page and rows 16-31 its
  // second, one 16-byte piece per tensor each, so every thread loads and the
  // hot path applies.  Otherwise a round of thread rows covers RPP rows of
  // each page.
  constexpr bool PS = TPR == 32;
  constexpr int RPP = PS ? 16 : (TPR < 16 ? TPR : 16);   // page rows one load round covers
  constexpr int RND = 16 / RPP;                          // load rounds per page
  constexpr int NLD = PS ? 1 : 2 * RND;                  // 16-byte loads per tensor per stage
  constexpr int TILE_B = Gm::TILE * 16;
  static_assert(PF % 2 == 0, "even prefetch depth keeps the LDS buffer parity static");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;

  extern __shared__ __align__(16) unsigned char smem[];
  // The grid's last workgroup writes the work plan (a0) and nothing else, so
  // the plan runs beside the ranges instead of after one of them.
  if (blockIdx.x == gridDim.x - 1) {
    write_plan<NT>(a, reinterpret_cast<int*>(smem));
    return;
  }

  const int Hkv = a.Hkv;
  const int w = blockIdx.x / (Hkv / HP), j0 = (blockIdx.x % (Hkv / HP)) * HP;
  // this wave's kv head and its first row tile among that head's G*K rows
  const int hl = wave / WPH, j = j0 + hl, wt = (wave % WPH) * RT;
  const int K = a.K, G = a.G, rows = a.rows;
  // This wave's query rows as B operands (row li of tile rt, d group lg + 4*ds);
  // rows past G*K repeat the last row (their outputs are never stored).
  const T* __restrict__ q = static_cast<const T*>(a.q);
  Vec8<T> qv[RT][DS];
  auto load_q = [&](int bq) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = min((wt + rt) * 16 + li, rows - 1);
      const int t = row / G, gg = row % G;
      const T* qp = q + ((size_t(bq) * K + t) * a.Hq + j * G + gg) * D;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) load8(qv[rt][ds], qp + (lg + 4 * ds) * 8);
    }
  };
  // With one request its query rows are known before the plan: their loads
  // go out with the plan's, so the two round trips overlap.
  const bool q_early = a.C == 1;
  if (q_early) load_q(0);
  const RangeStart rs = find_range<NT>(a, w, reinterpret_cast<int*>(smem));
  if (rs.b < 0) return;   // no such range for this batch (uniform)

  // The kernel walks a request's keys in slabs of 16 tokens; a page holds
  // 2^lsp slabs (page size 16 << lsp), so slab q lies in page q >> lsp at
  // token offset 16 * (q & (2^lsp - 1)).  Segments start on granule
  // boundaries, which start a page and an even slab.
  const int lsp = a.lsp, smask = (1 << lsp) - 1;
  unsigned char* sK = smem;                    // [2][TILE_B]
  unsigned char* sV = smem + 2 * TILE_B;       // [2][TILE_B]
  const float c2 = a.scale_log2;

  // ---- page descriptors (uniform): byte bases of K and V rows of kv head j0
  const int64_t head_off = int64_t(j0) * a.head_stride * int64_t(sizeof(T));
  const char* __restrict__ kcj = static_cast<const char*>(a.k_cache) + head_off;
  const char* __restrict__ vcj = static_cast<const char*>(a.v_cache) + head_off;
  const int64_t page_b = a.page_stride * int64_t(sizeof(T));
  const int64_t slab_b = 16 * a.token_stride * int64_t(sizeof(T));
  const int last_phys = a.num_pages - 1;
  const size_t blk_page_b = size_t(16) * Hkv * D * sizeof(T);

  // ---- loader geometry: thread -> (page row trw + q*RPP, 16-byte chunk tchunk)
  // of both pages, or with the page split of page tpage only
  const int tchunk = threadIdx.x % CPR;
  const int trow = threadIdx.x / CPR;
  const int tpage = PS ? __builtin_amdgcn_readfirstlane(trow >> 4) : 0;  // wave-uniform
  const int trw = PS ? trow & 15 : trow;
  const bool lactive = PS ? trow < 32 : trow < RPP;
  const uint32_t ts_b = uint32_t(a.token_stride * int64_t(sizeof(T)));
  const uint32_t bts_b = uint32_t(Hkv * D * sizeof(T));
  uint32_t coff[RND], wpos[NLD];
#pragma unroll
  for (int qq = 0; qq < RND; ++qq) {
    const uint32_t slot = trw + qq * RPP;
    coff[qq] = slot * ts_b + tchunk * 16;
    if constexpr (PS) {
      wpos[0] = Gm::pos(tpage * 16 + slot, tchunk) * 16;
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) wpos[tt * RND + qq] = Gm::pos(tt * 16 + slot, tchunk) * 16;
    }
  }


  // ---- consumer geometry (compile-time buffer offsets added per stage); the
  // wave's head starts hl*D elements into a stage row
  const int hchunk = hl * (D / EPC);
  uint32_t kpos[DS][8 / EPC];   // row li (page 0), d group lg + 4*ds
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int h = 0; h < 8 / EPC; ++h) kpos[ds][h] = Gm::pos(li, hchunk + (lg + 4 * ds) * 8 / EPC + h) * 16;
  // V rows: token 4*lg + e of page 0 (page 1 is +16 rows), elements
  // dch(li)*DPL .. (dch: vchunk for one 16-byte chunk per lane, else identity)
  constexpr bool kVPerm = DPL * sizeof(T) == 16;
  auto dch = [](int i) { return kVPerm ? vchunk(i) : i; };
  uint32_t vpos[4][DPL * sizeof(T) > 16 ? 2 : 1];
  constexpr int VCH = DPL * sizeof(T) > 16 ? 2 : 1;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int h = 0; h < VCH; ++h) {
      const int row = 4 * lg + e;
      const int e0 = hl * D + dch(li) * DPL + h * EPC;  // first element of this chunk piece
      vpos[e][h] = Gm::pos(row, e0 / EPC) * 16 + (e0 % EPC) * sizeof(T);
    }


  // Block position of each query row this lane scores (rows past G*K repeat
  // the last row, as the query loads do).
  int tq[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) tq[rt] = min((wt + rt) * 16 + li, rows - 1) / G;

  // ---- the range's segments: request b from slab p_lo to p_hi of its keys
  int b = rs.b, S = rs.S, ctx_next = rs.ctx;
  while (S < rs.B1) {   // uniform
    const int ctx = ctx_next;
    const int npages = (ctx + 15) >> 4;          // context slabs
    const int L = npages + a.nbk;                // the request's keys, in slabs
    const int Gb = (L + a.gran - 1) / a.gran;
    const int p_lo = max(rs.B0 - S, 0) * a.gran;
    const int p_hi = min((rs.B1 - S) * a.gran, L);
    // a whole request writes its output; a piece goes to slot 2w + k
    const bool whole = p_lo == 0 && p_hi == L;
    const int pslot = 2 * w + (S > rs.B0 ? 1 : 0);

    if (!q_early) load_q(b);
    const int32_t* __restrict__ pt = a.page_table + size_t(b) * a.max_pages;
    // Page-table window of the hot path: lane l holds the segment's entries
    // pg_lo + 128*w + l and pg_lo + 128*w + 64 + l of the current window w
    // (pg_lo = the segment's first page), and a stage takes its entries with
    // v_readlane.  The window is one vector load per 128 pages (a scalar read
    // waited on at every issue, missing the scalar cache every 8 stages, cost
    // ~4% at 256 stages per item).  Entries past the table row are clamped
    // into it.
    int pwlo = 0, pwhi = 0;
    auto load_window = [&](int wi) __attribute__((always_inline)) {
      const int base = (p_lo >> lsp) + 128 * wi;
      pwlo = pt[min(base + lane, a.max_pages - 1)];
      pwhi = pt[min(base + 64 + lane, a.max_pages - 1)];
    };
    load_window(0);

    // context slabs, then block slabs from block slab bofs on
    const int ncache = max(0, min(npages, p_hi) - p_lo);
    const int bofs = max(p_lo, npages) - npages;
    const int nblk = max(0, p_hi - max(p_lo, npages));
    const int nvp = ncache + nblk;
    const int nstage = (nvp + 1) >> 1;

    Acc<T, D, RT> acc;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      acc.m2[rt] = -INFINITY;
      acc.l[rt] = 0.f;
#pragma unroll
      for (int cc = 0; cc < DPL; ++cc) acc.o[rt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const char* kblk = static_cast<const char*>(a.k_blk) + ((size_t(b) * K) * Hkv + j0) * D * sizeof(T);
    const char* vblk = static_cast<const char*>(a.v_blk) + ((size_t(b) * K) * Hkv + j0) * D * sizeof(T);
    // Stages [0, nhot) are two full context pages each: the hot path.  The rest
    // (a partial last page, the block's own keys) take the general path.
    const int nfull = max(0, min(ctx >> 4, p_hi) - p_lo);
    const int nhot = nfull >> 1;
    struct Page {
      const char* k;
      const char* v;
      int n;     // valid tokens (0 = absent)
      bool blk;  // block page (token stride Hkv*D)
      int cb;    // block-causal block page: 1 + its index among the block pages, else 0
    };
    auto page = [&](int vp) __attribute__((always_inline)) -> Page {
      Page pg{kcj, vcj, 0, false, 0};
      if (vp < ncache) {
        const int lp = p_lo + vp;
        const int phys = pt[lp >> lsp];
        if (phys >= 0 && phys <= last_phys) {
          const int64_t off = int64_t(phys) * page_b + int64_t(lp & smask) * slab_b;
          pg.k = kcj + off;
          pg.v = vcj + off;
          pg.n = min(16, ctx - lp * 16);
        }
      } else if (vp < nvp) {
        const int bp = bofs + vp - ncache;
        pg.k = kblk + bp * blk_page_b;
        pg.v = vblk + bp * blk_page_b;
        pg.n = min(16, K - bp * 16);
        pg.blk = true;
        pg.cb = a.block_causal ? bp + 1 : 0;
      }
      return pg;
    };

    // Two full context pages (stage st < nhot): page numbers from the window,
    // unpredicated loads off scalar page bases (entries clamped into the pool:
    // never a stray read).
    constexpr bool kHot = PS || RPP * CPR == NT;
    auto issue_hot = [&](int st, uint4 (&stk)[NLD], uint4 (&stv)[NLD]) __attribute__((always_inline)) {
      // slabs 2st and 2st+1 of the split: window entries o0, o1 (the same page
      // unless pages are 16 tokens; an even o0 keeps both in one lane half)
      const int q0 = 2 * st, o0 = (q0 >> lsp) & 127, o1 = ((q0 + 1) >> lsp) & 127;
      const int v = (o0 >> 6) ? pwhi : pwlo;
      const int ph0 = min(max(__builtin_amdgcn_readlane(v, o0 & 63), 0), last_phys);
      const int ph1 = min(max(__builtin_amdgcn_readlane(v, o1 & 63), 0), last_phys);
      const int64_t off0 = int64_t(ph0) * page_b + int64_t(q0 & smask) * slab_b;
      const int64_t off1 = int64_t(ph1) * page_b + int64_t((q0 + 1) & smask) * slab_b;
      if constexpr (PS) {
        const int64_t off = tpage ? off1 : off0;
        stk[0] = ld_stream(kcj + off + coff[0]);
        stv[0] = ld_stream(vcj + off + coff[0]);
      } else {
        const char* k0 = kcj + off0;
        const char* v0 = vcj + off0;
        const char* k1 = kcj + off1;
        const char* v1 = vcj + off1;
#pragma unroll
        for (int qq = 0; qq < RND; ++qq) {
          stk[qq] = ld_stream(k0 + coff[qq]);
          stv[qq] = ld_stream(v0 + coff[qq]);
          stk[RND + qq] = ld_stream(k1 + coff[qq]);
          stv[RND + qq] = ld_stream(v1 + coff[qq]);
        }
      }
    };
    auto issue = [&](int st, uint4 (&stk)[NLD], uint4 (&stv)[NLD], int (&nv)[2]) __attribute__((always_inline)) {
      if (kHot && st < nhot) {
        issue_hot(st, stk, stv);
        nv[0] = 16;
        nv[1] = 16;
        return;
      }
      const Page p0 = page(2 * st), p1 = page(2 * st + 1);
      // valid-token count, with the block-causal page index above bit 8: a
      // stage is on the unmasked fast path exactly when both words equal 16
      nv[0] = p0.n | (p0.cb << 8);
      nv[1] = p1.n | (p1.cb << 8);
      if constexpr (PS) {
        // this thread's page, field by field (wave-uniform selects)
        const bool second = tpage != 0;
        const char* pk = second ? p1.k : p0.k;
        const char* pv = second ? p1.v : p0.v;
        const int pn = second ? p1.n : p0.n;
        const bool pblk = second ? p1.blk : p0.blk;
        const uint32_t off = pblk ? uint32_t(trw) * bts_b + tchunk * 16 : coff[0];
        uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);  // absent tokens: V must be 0, not NaN
        if (lactive && trw < pn) {
          kx = *reinterpret_cast<const uint4*>(pk + off);
          vx = *reinterpret_cast<const uint4*>(pv + off);
        }
        stk[0] = kx;
        stv[0] = vx;
      } else {
        // (each page spelled out: selecting between the two by reference would
        // keep the staging registers from being promoted out of memory)
#pragma unroll
        for (int qq = 0; qq < RND; ++qq) {
          const int slot = trow + qq * RPP;
          const uint32_t off = p0.blk ? uint32_t(slot) * bts_b + tchunk * 16 : coff[qq];
          uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);  // absent tokens: V must be 0, not NaN
          if (lactive && slot < p0.n) {
            kx = *reinterpret_cast<const uint4*>(p0.k + off);
            vx = *reinterpret_cast<const uint4*>(p0.v + off);
          }
          stk[qq] = kx;
          stv[qq] = vx;
        }
#pragma unroll
        for (int qq = 0; qq < RND; ++qq) {
          const int slot = trow + qq * RPP;
          const uint32_t off = p1.blk ? uint32_t(slot) * bts_b + tchunk * 16 : coff[qq];
          uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
          if (lactive && slot < p1.n) {
            kx = *reinterpret_cast<const uint4*>(p1.k + off);
            vx = *reinterpret_cast<const uint4*>(p1.v + off);
          }
          stk[RND + qq] = kx;
          stv[RND + qq] = vx;
        }
      }
    };
    auto commit = [&](int buf, const uint4 (&stk)[NLD], const uint4 (&stv)[NLD]) __attribute__((always_inline)) {
      if (lactive) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          *reinterpret_cast<uint4*>(sK + buf * TILE_B + wpos[i]) = stk[i];
          *reinterpret_cast<uint4*>(sV + buf * TILE_B + wpos[i]) = stv[i];
        }
      }
    };

    auto compute = [&](int buf, const int (&nv)[2]) __attribute__((always_inline)) {
      const unsigned char* tk = sK + buf * TILE_B;
      const unsigned char* tv = sV + buf * TILE_B;
      const bool partial = nv[0] != 16 || nv[1] != 16;
      Vec8<T> kop[2][DS];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          if constexpr (sizeof(T) == 2) {
            kop[tt][ds].v = *reinterpret_cast<const uint4*>(tk + tt * 16 * CPR * 16 + kpos[ds][0]);
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint4 x = *reinterpret_cast<const uint4*>(tk + tt * 16 * CPR * 16 + kpos[ds][h]);
              kop[tt][ds].v[4 * h + 0] = __uint_as_float(x.x);
              kop[tt][ds].v[4 * h + 1] = __uint_as_float(x.y);
              kop[tt][ds].v[4 * h + 2] = __uint_as_float(x.z);
              kop[tt][ds].v[4 * h + 3] = __uint_as_float(x.w);
            }
          }
        }
      // Scores of row tile rt.  With two row tiles every tile's scores come
      // first: the K operands die before the softmax, and the second tile's
      // matrix work runs under the first tile's softmax instead of after its
      // max and rescale (the 128-row ragged batch: 298.5 -> 291.7 us).  With
      // one tile they stay next to its softmax (computed first, the head pair
      // at C = 128 took 648.7 against 646.8 us, nine runs each).
      f32x4 sacc[RT][2];
      auto scores = [&](int rt) __attribute__((always_inline)) {
        sacc[rt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sacc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) sacc[rt][tt] = mma8(kop[tt][ds], qv[rt][ds], sacc[rt][tt]);
      };
      constexpr bool kScoresFirst = RT > 1;
      if constexpr (kScoresFirst) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) scores(rt);
      }
      // V operands: lane reads 8 token rows x D/16 values and transposes them
      // in registers.  They do not depend on the softmax, so in the bf16
      // one-head one-tile forms they are read beside the score MFMAs, their
      // LDS latency and permutes then overlapping the matrix work (C = 2 at
      // 8192 tokens: 33.5 -> 32.6 us; one request at 2048 tokens: 19.8 ->
      // 19.2).  The two-tile forms, at their register bound, spill more that
      // way and lose the gain (the 128-row ragged batch: 292 -> 299 us); the
      // head pair measured no better (C = 128: 648.2 against 647.3 us, nine
      // runs each); fp32 operands are twice the registers.  Those read them
      // after the softmax, in the order of the code below.
      constexpr bool kVEarly = sizeof(T) == 2 && RT == 1 && HP == 1;
      auto read_v = [&](VRow<T, DPL> (&vr)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned char* base = tv + (e >> 2) * 16 * CPR * 16;
          if constexpr (sizeof(T) == 2 && DPL == 8) {
            vr[e].v = *reinterpret_cast<const uint4*>(base + vpos[e & 3][0]);
          } else if constexpr (sizeof(T) == 2) {
            vr[e].v = *reinterpret_cast<const uint2*>(base + vpos[e & 3][0]);
          } else {
#pragma unroll
            for (int h = 0; h < DPL / 4; ++h) {
              const uint4 x = *reinterpret_cast<const uint4*>(base + vpos[e & 3][h]);
              vr[e].v[4 * h + 0] = __uint_as_float(x.x);
              vr[e].v[4 * h + 1] = __uint_as_float(x.y);
              vr[e].v[4 * h + 2] = __uint_as_float(x.z);
              vr[e].v[4 * h + 3] = __uint_as_float(x.w);
            }
          }
        }
      };
      Vec8<T> vte[kVEarly ? DPL : 1];
      if constexpr (kVEarly) {
        VRow<T, DPL> vr[8];
        read_v(vr);
#pragma unroll
        for (int cc = 0; cc < DPL; ++cc) vtrans<DPL>(vte[cc], vr, cc);
      }
      float p[RT][8];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if constexpr (!kScoresFirst) scores(rt);
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = sacc[rt][e >> 2][e & 3];
        if (partial) {
          // token 4*lg + (e&3) of page e>>2 is kept when it is one of the page's
          // valid tokens and, on a block-causal block page with index cb-1, its
          // block position 16*(cb-1) + token is at most this row's position
          int lim[2];
#pragma unroll
          for (int pg = 0; pg < 2; ++pg) {
            const int n = nv[pg] & 255, cb = nv[pg] >> 8;
            lim[pg] = cb ? min(n, tq[rt] - 16 * (cb - 1) + 1) : n;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (4 * lg + (e & 3) >= lim[e >> 2]) sv[e] = -INFINITY;
        }
        const float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), sv[2]),
                               fmaxf(fmaxf(sv[3], sv[4]), fmaxf(fmaxf(sv[5], sv[6]), sv[7])));
        const float mx2 = group4_max(mx) * c2;
        const bool need = mx2 > acc.m2[rt] + kRescaleLog2;
        if (__any(need)) {
          if (need) {
            const float alpha = fast_exp2(acc.m2[rt] - mx2);
            acc.l[rt] *= alpha;
#pragma unroll
            for (int cc = 0; cc < DPL; ++cc) acc.o[rt][cc] *= alpha;
            acc.m2[rt] = mx2;
          }
        }
        const float nb = acc.m2[rt] == -INFINITY ? 0.f : -acc.m2[rt];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[rt][e] = fast_exp2(fmaf(sv[e], c2, nb));
        acc.l[rt] += ((p[rt][0] + p[rt][1]) + (p[rt][2] + p[rt][3])) +
                     ((p[rt][4] + p[rt][5]) + (p[rt][6] + p[rt][7]));
      }
      // O^T += V^T . P^T
      VRow<T, DPL> vr[8];
      if constexpr (!kVEarly) read_v(vr);
      Vec8<T> vt[DPL];
#pragma unroll
      for (int cc = 0; cc < DPL; ++cc) {
        if constexpr (kVEarly) {
          vt[cc] = vte[cc];
        } else {
          vtrans<DPL>(vt[cc], vr, cc);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        Vec8<T> pv;
        pack_p(pv, p[rt]);
#pragma unroll
        for (int cc = 0; cc < DPL; ++cc) acc.o[rt][cc] = mma8(vt[cc], pv, acc.o[rt][cc]);
      }
    };

    // Software pipeline: PF stages of loads in flight in registers, two LDS
    // buffers.  Stage st goes to LDS buffer st&1 (last read by stage st-2, which
    // every wave finished before the previous barrier); stage st+PF is then
    // issued into the registers just freed; one barrier; then the math.
    uint4 stk[PF][NLD], stv[PF][NLD];
    int nv[PF][2];
    int st0 = 0;
    if (kHot && nhot >= 2 * PF) {  // uniform over the workgroup
      // Hot loop: every stage it issues is two full context pages, so every
      // slot issues its loads on every path and each wait before a commit
      // counts exactly the newer stage in flight.  The next page-table window
      // is loaded into (pnlo, pnhi) just before the last stage of the current
      // one is issued; at the window's first stage an explicit wait for all
      // but that stage's loads makes it current.  The page numbers read by
      // every issue are thus never a pending load, and the K/V stream never
      // drains for them (a full wait there cost one round trip per 64 stages).
      // vmcnt(2 * NLD): one stage's loads may stay pending (count bits 3:0 and 15:14)
      static_assert(2 * NLD < 64, "vmcnt field");
      constexpr int kWinWait = 0x0F70 | ((2 * NLD) & 15) | (((2 * NLD) >> 4) << 14);
      const int wmask = (64 << lsp) - 1;
      int pnlo = 0, pnhi = 0;
      // The first PF stages go out strictly in slot order.  Interleaved by the
      // scheduler, the loop's wait bookkeeping at its header must assume slot 0
      // may be the newest load, and it then waits for every load in flight
      // before each slot-0 issue, every PF stages of the whole loop.
      static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
        constexpr int pp = decltype(P)::value;
        issue_hot(pp, stk[pp], stv[pp]);
        __builtin_amdgcn_sched_barrier(0);
      });
      __syncthreads();   // LDS free: the previous segment's last stage (or the plan scan) is done
      for (; st0 + 2 * PF <= nhot; st0 += PF) {
        static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
          constexpr int pp = decltype(P)::value;
          const int sn = st0 + pp + PF;   // < nhot
          commit(pp & 1, stk[pp], stv[pp]);
          if ((sn & wmask) == 0) {   // first stage of a 128-page window, loaded one step ago
            __builtin_amdgcn_s_waitcnt(kWinWait);
            pwlo = pnlo;
            pwhi = pnhi;
          } else if (((sn + 1) & wmask) == 0) {   // last stage of this window: fetch the next
            const int base = (p_lo >> lsp) + 128 * ((sn + 1) >> (6 + lsp));
            pnlo = pt[min(base + lane, a.max_pages - 1)];
            pnhi = pt[min(base + 64 + lane, a.max_pages - 1)];
          }
          issue_hot(sn, stk[pp], stv[pp]);
          __syncthreads();
          const int full[2] = {16, 16};
          compute(pp & 1, full);
        });
      }
#pragma unroll
      for (int pp = 0; pp < PF; ++pp) nv[pp][0] = nv[pp][1] = 16;
    } else {
      static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
        constexpr int pp = decltype(P)::value;
        if (pp < nstage) issue(pp, stk[pp], stv[pp], nv[pp]);
      });
      __syncthreads();   // LDS free: the previous segment's last stage (or the plan scan) is done
    }
    // the remaining stages: the hot tail, a partial last page, the block's keys
    for (; st0 < nstage; st0 += PF) {
      static_for<0, PF>([&](auto P) __attribute__((always_inline)) {
        constexpr int pp = decltype(P)::value;
        const int st = st0 + pp;
        if (st < nstage) {  // uniform over the workgroup
          commit(pp & 1, stk[pp], stv[pp]);
          const int n0 = nv[pp][0], n1 = nv[pp][1];
          if (st + PF < nstage) {
            const int sn = st + PF;
            if ((sn & ((64 << lsp) - 1)) == 0 && sn < nhot) load_window(sn >> (6 + lsp));  // next window
            issue(sn, stk[pp], stv[pp], nv[pp]);
          }
          __syncthreads();
          const int nn[2] = {n0, n1};
          compute(pp & 1, nn);
        }
      });
    }

    // store: lane holds row li of each tile and d = dch(4*lg + r)*DPL + cc.
    // A whole request writes its normalised output; a piece writes its own
    // normalised partial O / l in the activation dtype (half the bytes of
    // fp32 for the attention to write and the merge to read) and its fp32
    // (m, l), which weight it in the merge.  A piece whose keys the block-causal
    // mask hides from a row has l = 0 and stores zeros.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float lsum = group4_sum(acc.l[rt]);
      const int row = (wt + rt) * 16 + li;
      if (row >= rows || nstage == 0) continue;
      T* o;
      float inv;
      if (whole) {
        const int t = row / G, gg = row % G;
        o = static_cast<T*>(a.out) + ((size_t(b) * K + t) * a.Hq + j * G + gg) * D;
        inv = 1.f / lsum;
      } else {
        const size_t prow = (size_t(pslot) * Hkv + j) * rows + row;
        o = static_cast<T*>(a.part_o) + prow * D;
        inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(acc.m2[rt], lsum);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        T* dst = o + dch(4 * lg + r) * DPL;
        if constexpr (sizeof(T) == 2) {
          if constexpr (DPL == 8) {
            uint4 pk;
            pk.x = pack_bf16x2(acc.o[rt][0][r] * inv, acc.o[rt][1][r] * inv);
            pk.y = pack_bf16x2(acc.o[rt][2][r] * inv, acc.o[rt][3][r] * inv);
            pk.z = pack_bf16x2(acc.o[rt][4][r] * inv, acc.o[rt][5][r] * inv);
            pk.w = pack_bf16x2(acc.o[rt][6][r] * inv, acc.o[rt][7][r] * inv);
            *reinterpret_cast<uint4*>(dst) = pk;
          } else {
            uint2 pk;
            pk.x = pack_bf16x2(acc.o[rt][0][r] * inv, acc.o[rt][1][r] * inv);
            pk.y = pack_bf16x2(acc.o[rt][2][r] * inv, acc.o[rt][3][r] * inv);
            *reinterpret_cast<uint2*>(dst) = pk;
          }
        } else {
#pragma unroll
          for (int cc = 0; cc < DPL; cc += 4)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + cc) =
                make_float4(acc.o[rt][cc][r] * inv, acc.o[rt][cc + 1][r] * inv,
                            acc.o[rt][cc + 2][r] * inv, acc.o[rt][cc + 3][r] * inv);
        }
      }
    }

    S += Gb + a.seg;   // the next request's keys start after its fixed cost
    ++b;
    if (S < rs.B1) ctx_next = ctx_of(a, b);
  }
}

// ---------------------------------------------------------------------------
// a4: merge of split partials (requests with more than one split only).
// a4: one workgroup per (request, kv head, slab of output columns); the
// body is attn_merge_block (merge.h).
template <typename T, int D, int LPO, int U>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  attn_merge_block<T, D, LPO, U>(a, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
// Stages of K/V loads in flight per workgroup.  With nontemporal loads two
// stages keep pace with four at 64 query rows (C = 128: 707 vs 729 us) and
// leave the 128-row tiles at two waves per SIMD instead of one (workload 4:
// 660 vs 771 us).  (Those figures predate the hot loop below.  With it and
// its loads issued in slot order, depth 4 compiles for the bf16 64-row and
// head-pair forms, 235-237 registers, and is no faster at any C (C = 128:
// 656 vs 650 us); the 128-row forms spill hundreds of registers at depth 4.)
constexpr int kPrefetch = 2;

// (RT row tiles per wave, NW waves) for a query-row count: every wave reads the
// whole stage from LDS, so fewer, wider waves cut LDS traffic per HBM byte.
template <typename T, int D, int RT, int NW, int HP = 1>
static hipError_t launch_attn_cfg(hipStream_t st, const AttnArgs& a) {
  const size_t lds = AttnLds<T, HP * D>::bytes;
  auto kern = k_block_attn<T, D, RT, NW, kPrefetch, HP>;
  // one workgroup per (range, head group), plus the plan writer
  hipLaunchKernelGGL(kern, dim3(a.w_max * (a.Hkv / HP) + 1), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(hipStream_t st, const AttnArgs& a) {
  if (a.rows <= 16) return launch_attn_cfg<T, D, 1, 1>(st, a);
  if (a.rows <= 32) return launch_attn_cfg<T, D, 1, 2>(st, a);
  // Two adjacent kv heads per workgroup (bf16, D = 128, 33..128 rows per
  // head, adjacent heads in the pools): each stage row is then one 512-byte
  // piece of the token's K (V) instead of two 256-byte pieces read by two
  // workgroups, which a read probe of the pattern measures at 7.1-7.2 TB/s
  // against 6.6 TB/s (C = 128: 687 -> 651 us; with two row tiles per wave,
  // 128 rows per head, the 64-head ragged batch went from 315 to 296 us: its
  // odd heads' 256-byte pieces, 256 bytes into each 1 KB of the row, had
  // streamed 15-25% slower).
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    if (a.head_pair && head_pair_fits(a.rows, a.Hkv, a.head_stride, 1, D))
      return a.rows <= 64 ? launch_attn_cfg<T, D, 1, 8, 2>(st, a) : launch_attn_cfg<T, D, 2, 8, 2>(st, a);
  }
  if (a.rows <= 64) return launch_attn_cfg<T, D, 1, 4>(st, a);
  if (a.rows <= 128) return launch_attn_cfg<T, D, 2, 4>(st, a);
  return launch_attn_cfg<T, D, 2, 8>(st, a);
}

size_t attn_lds_bytes(int dtype, int D, int rows, int K) {
  (void)rows;
  (void)K;
  if (dtype == 1) return D == 64 ? AttnLds<bf16_t, 64>::bytes : AttnLds<bf16_t, 128>::bytes;
  return D == 64 ? AttnLds<float, 64>::bytes : AttnLds<float, 128>::bytes;
}

bool head_pair_fits(int rows, int Hkv, int64_t head_stride, int dtype, int D) {
  return dtype == 1 && D == 128 && rows > 32 && rows <= 128 && Hkv % 2 == 0 && head_stride == D;
}

template <typename T, int D, int LPO, int U>
static hipError_t launch_merge_cfg(hipStream_t st, const AttnArgs& a) {
  const dim3 mg(a.C * a.Hkv, (a.rows * (D / 4) + 256 / LPO - 1) / (256 / LPO));
  hipLaunchKernelGGL((k_attn_merge<T, D, LPO, U>), mg, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Four lanes per output (LPO = 4, up to 16 pieces each per round) when the
// plan has many ranges per request, i.e. few long requests cut into many
// pieces (small C); otherwise one lane (up to 8 pieces per round), which
// keeps the grid -- mostly workgroups of whole requests that exit at once --
// four times smaller.
bool merge_wide(const AttnArgs& a) { return a.w_max > 4 * a.C; }

template <typename T, int D>
static hipError_t launch_merge(hipStream_t st, const AttnArgs& a) {
  if (merge_wide(a)) return launch_merge_cfg<T, D, 4, 16>(st, a);
  return launch_merge_cfg<T, D, 1, 8>(st, a);
}

hipError_t launch_block_attn(hipStream_t st, int dtype, const AttnArgs& a, bool merge) {
  hipError_t e;
  if (dtype == 1) {
    e = a.D == 64 ? launch_attn_d<bf16_t, 64>(st, a) : launch_attn_d<bf16_t, 128>(st, a);
  } else {
    e = a.D == 64 ? launch_attn_d<float, 64>(st, a) : launch_attn_d<float, 128>(st, a);
  }
  if (e != hipSuccess) return e;
  if (merge && a.w_max > 1) {  // some request may span several ranges
    if (dtype == 1) {
      e = a.D == 64 ? launch_merge<bf16_t, 64>(st, a) : launch_merge<bf16_t, 128>(st, a);
    } else {
      e = a.D == 64 ? launch_merge<float, 64>(st, a) : launch_merge<float, 128>(st, a);
    }
  }
  return e;
}

}  // namespace hspec
