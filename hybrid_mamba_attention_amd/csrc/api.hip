// C ABI of libhspec.so (declared and documented in include/hspec.h).
//
// Every entry point validates its arguments on the host, before touching the
// HIP runtime, and returns a negative hspec_status on any violation; only
// then does it enqueue kernels on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/hspec.h"
#include "kernels.h"

namespace hspec {
size_t ssd_lds_bytes(int P, int N, int Q);
bool ssd_chunk_fits(int chunk, int N, bool conv);
}

using namespace hspec;

namespace {

constexpr size_t kMaxLds = 160 * 1024;
// GEMM operands up to 2^40 output elements (tile counts stay ints); no
// projection that fits in device memory comes near it
constexpr int64_t kMaxGemmOut = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int esize(int dtype) { return dtype == HSPEC_BF16 ? 2 : 4; }
bool dtype_ok(int dtype) { return dtype == HSPEC_F32 || dtype == HSPEC_BF16; }
int status_of(hipError_t e) { return e == hipSuccess ? HSPEC_OK : HSPEC_ERR_HIP; }

int check_init(int dtype, int C, int d, int S, const void* u, const void* w, const float* h0) {
  if (!dtype_ok(dtype) || C < 1 || d < 1 || S < 1) return HSPEC_ERR_INVALID_ARG;
  if (!u || !w || !h0) return HSPEC_ERR_INVALID_ARG;
  if (!aligned(u, 16) || !aligned(w, 16) || !aligned(h0, 16)) return HSPEC_ERR_INVALID_ARG;
  if (d % 32 || S % 64) return HSPEC_ERR_UNSUPPORTED;
  // a lane's W row offsets within a 32-row k-step are 32-bit byte offsets,
  // and the grid holds (S / 128) * ceil(C / 32) workgroups
  if (S > (1 << 25) || C > (1 << 16)) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

// shape limits of the scan (pointers are checked by the callers); conv: the
// Mamba-2 block's scan with the convolution fused into its loads
int check_ssd_shape(int dtype, int C, int K, int H, int P, int ng, int N, int chunk, bool conv = false) {
  if (!dtype_ok(dtype) || C < 1 || K < 1 || H < 1 || P < 1 || N < 1 || ng < 1 || chunk < 1)
    return HSPEC_ERR_INVALID_ARG;
  if (H % ng) return HSPEC_ERR_INVALID_ARG;
  if (chunk > 64 || (chunk & (chunk - 1))) return HSPEC_ERR_UNSUPPORTED;
  if (!ssd_chunk_fits(chunk, N, conv)) return HSPEC_ERR_UNSUPPORTED;
  if (P > 128 || N > 128) return HSPEC_ERR_UNSUPPORTED;
  if (ssd_lds_bytes(P, N, chunk) > kMaxLds) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(C) * H > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

int check_ssd(int dtype, int C, int K, int H, int P, int ng, int N, int chunk, const void* x,
              const float* delta, const float* A, const void* B, const void* Cm, const float* y) {
  const int st = check_ssd_shape(dtype, C, K, H, P, ng, N, chunk);
  if (st != HSPEC_OK) return st;
  if (!x || !delta || !A || !B || !Cm || !y) return HSPEC_ERR_INVALID_ARG;
  return HSPEC_OK;
}

// Host side of the attention's work plan (the device derives the same plan
// from ctx_lens; include/hspec.h documents it).  The host knows only bounds:
// w_max, the most ranges the plan can use, sizes the grid and the workspace.
struct AttnPlanShape {
  int w_max, gran, range_gran, min_gran, seg, nbk, head_pair;
  size_t plan_bytes, part_o_off, part_ml_off, total;
};

// (range, kv head) units the automatic plan aims at: two per CU, one
// resident round of the one-head forms at their occupancy (measured at
// 8192-token contexts, C = 2..64: 512 units beat both 256, too little in
// flight, and 1024, twice the per-unit prologue and fp32 partials).  The
// head-pair form takes the same ranges in half the workgroups, one round at
// one workgroup per CU.  (Twice the ranges for it -- two rounds -- cut every
// request of a uniform batch in two: C = 32 and 64 at 8192 tokens took 12%
// and 9% longer.)
constexpr int kTargetUnits = 512;
// A request's fixed cost in an automatic range, in slabs of streaming: its
// query rows and page-table window, the first stages' round trip, the partial
// last page and block slabs on the general path, the output store.  A
// timestamp probe of every workgroup (workload 2: C = 32, 512-4096 tokens)
// measured ~6 us per extra request in a range against ~1 us per granule of
// two slabs, and the cost model put the slowest range of that batch at
// 45 us with 12 slabs against 53 us with none.
constexpr int kSegSlabs = 12;
// The same with more than 64 query rows per kv head (two row tiles per wave):
// a segment's query rows, output store and general-path stages are twice the
// work.  Attention on the 64-head ragged batch (128 rows per kv head),
// flushed medians over six runs: 12 slabs 292.9 us, 18 288.5, 24 287.8,
// 32 290.7.
constexpr int kSegSlabsTwoTiles = 24;
int seg_slabs(int rows) { return rows > 64 ? kSegSlabsTwoTiles : kSegSlabs; }
// Ranges (at the batch's bound) of at least this many slabs take two kv heads
// per workgroup when the pools and rows allow it.  Flushed medians of the
// attention call on one box, one head per workgroup -> head pair, 8192-token
// contexts: C = 4 44.4 -> 41.7 us and C = 8 65.4 -> 61.7 (ranges of 32 and 64
// slabs), the C = 32 ragged batch (~126) 74.5 -> 70.4; but C = 1 24.0 -> 27.0
// and C = 2 33.2 -> 33.7 (8 and 16 slabs at the bound; one request at 2048
// tokens: 19.7 -> 23.1), where the halved workgroup count leaves CUs idle or
// each workgroup only a few stages.
constexpr int kPairSlabs = 32;

// log2(page_size / 16) for a supported page size, else -1
int page_shift(int page_size) {
  for (int l = 0; l <= 4; ++l)
    if (page_size == (16 << l)) return l;
  return -1;
}

AttnPlanShape plan_shape(int dtype, int C, int K, int Hq, int Hkv, int D, int64_t head_stride, int max_ctx,
                         int kv_split_pages, int page_size) {
  AttnPlanShape p{};
  const int spp = page_size / 16;
  p.gran = std::max(2, spp);
  p.nbk = (K + 15) / 16;
  p.min_gran = (16 + p.gran - 1) / p.gran;   // ranges of >= 16 slabs when the batch allows
  // granules of a max_ctx request, and of the batch at most
  const int64_t gmax = ((int64_t(max_ctx) + 15) / 16 + p.nbk + p.gran - 1) / p.gran;
  const int64_t tmax = int64_t(C) * gmax;
  // automatic ranges charge each request seg_slabs(rows) slabs' worth of fixed
  // cost
  p.seg = kv_split_pages > 0 ? 0 : (seg_slabs((Hq / Hkv) * K) + p.gran - 1) / p.gran;
  const int64_t tunits = int64_t(C) * (gmax + p.seg);   // the batch's units at its bound
  const bool hp_ok = head_pair_fits((Hq / Hkv) * K, Hkv, head_stride, dtype, D);
  int64_t w_max;
  if (kv_split_pages > 0) {
    p.range_gran = int(std::max<int64_t>(1, (int64_t(kv_split_pages) * spp + p.gran - 1) / p.gran));
    w_max = (tmax + p.range_gran - 1) / p.range_gran;
    p.head_pair = hp_ok && int64_t(p.range_gran) * p.gran >= kPairSlabs;
  } else {
    p.range_gran = 0;
    w_max = std::max<int64_t>(1, kTargetUnits / Hkv);
    // two heads per workgroup when the batch at its bound gives ranges of
    // kPairSlabs slabs or more
    p.head_pair = hp_ok && tmax * p.gran >= kPairSlabs * std::min(w_max, tmax);
    // The device makes W = min(w_max, max(1, floor(T / min_gran))) ranges and
    // T <= tmax (contexts are clamped to max_ctx), so no more can ever be
    // needed: a small batch's grid then holds no workgroups without a range
    // (C = 1 at 8192 tokens: 257 instead of 513, whose idle half still took
    // dispatch slots and ran the range scan).
    w_max = std::min<int64_t>(w_max, std::max<int64_t>(1, tunits / p.min_gran));
  }
  w_max = std::max<int64_t>(1, std::min(w_max, tmax));   // a range holds at least one granule
  p.w_max = int(std::min<int64_t>(w_max, 0x7fffffff));
  const size_t rows = size_t(Hq / Hkv) * K;
  p.plan_bytes = align256((4 + 3 * size_t(C) + size_t(p.w_max) + 1) * 4);
  p.part_o_off = p.plan_bytes;
  size_t po = 0, pml = 0;
  if (p.w_max > 1) {  // only then can a request span several ranges
    po = align256(2 * size_t(p.w_max) * Hkv * rows * D * (dtype == 1 ? 2 : 4));   // activation dtype
    pml = align256(2 * size_t(p.w_max) * Hkv * rows * 2 * 4);
  }
  p.part_ml_off = p.part_o_off + po;
  p.total = p.part_ml_off + pml;
  return p;
}

int check_attn(int dtype, int C, int K, int Hq, int Hkv, int D, const void* q, const void* kb,
               const void* vb, const void* kc, const void* vc, int64_t ps, int64_t ts, int64_t hs,
               int num_pages, int page_size, const int32_t* pt, int max_pages, const int32_t* ctx,
               int max_ctx, int kv_split_pages, float scale, int block_causal, const void* out,
               const size_t* ws_bytes) {
  if (!dtype_ok(dtype) || C < 1 || K < 1 || Hq < 1 || Hkv < 1) return HSPEC_ERR_INVALID_ARG;
  if (Hq % Hkv) return HSPEC_ERR_INVALID_ARG;
  if (!q || !kb || !vb || !kc || !vc || !pt || !ctx || !out || !ws_bytes) return HSPEC_ERR_INVALID_ARG;
  const int e = esize(dtype);
  const int vec = 16 / e;
  if (ps <= 0 || ts <= 0 || hs <= 0 || ps % vec || ts % vec || hs % vec) return HSPEC_ERR_INVALID_ARG;
  // the loader's offsets of a slab's 16 rows are 32-bit byte offsets
  if (ts * e > (int64_t(1) << 27)) return HSPEC_ERR_UNSUPPORTED;
  for (const void* p : {q, kb, vb, kc, vc, out})
    if (!aligned(p, 16)) return HSPEC_ERR_INVALID_ARG;
  if (!aligned(pt, 4) || !aligned(ctx, 4)) return HSPEC_ERR_INVALID_ARG;
  if (num_pages < 1 || max_ctx < 0 || kv_split_pages < 0 || page_size < 1) return HSPEC_ERR_INVALID_ARG;
  if (page_shift(page_size) < 0) return HSPEC_ERR_UNSUPPORTED;
  if (kv_split_pages > 0x7fffffff / (page_size / 16)) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(max_pages) < std::max<int64_t>(1, (int64_t(max_ctx) + page_size - 1) / page_size))
    return HSPEC_ERR_INVALID_ARG;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return HSPEC_ERR_INVALID_ARG;
  if (block_causal != 0 && block_causal != 1) return HSPEC_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return HSPEC_ERR_UNSUPPORTED;
  if (K > 64) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(Hq / Hkv) * K > 256) return HSPEC_ERR_UNSUPPORTED;
  if (attn_lds_bytes(dtype, D, (Hq / Hkv) * K, K) > kMaxLds) return HSPEC_ERR_UNSUPPORTED;
  // the kernels count the batch's keys in 32-bit slabs (granules times
  // slabs per granule) and launch w_max workgroups per kv head group, + 1
  const int spp = page_size / 16, gran = std::max(2, spp);
  const int64_t gmax = ((int64_t(max_ctx) + 15) / 16 + (K + 15) / 16 + gran - 1) / gran;
  const int64_t seg = (seg_slabs((Hq / Hkv) * K) + gran - 1) / gran;
  if (int64_t(C) * (gmax + seg) * gran >= 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  const AttnPlanShape p = plan_shape(dtype, C, K, Hq, Hkv, D, hs, max_ctx, kv_split_pages, page_size);
  if (int64_t(p.w_max) * Hkv >= 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

// The kernel arguments of a3 (arguments validated by check_attn); WORKSPACE
// when `ws` cannot hold the plan and partials.
int attn_args(AttnArgs& a, int dtype, int C, int K, int Hq, int Hkv, int D, const void* q, const void* kb,
              const void* vb, const void* kc, const void* vc, int64_t ps, int64_t ts, int64_t hs,
              int num_pages, int page_size, const int32_t* pt, int max_pages, const int32_t* ctx,
              int max_ctx, int kv_split_pages, float scale, int block_causal, void* out, void* ws,
              size_t ws_bytes) {
  const AttnPlanShape p = plan_shape(dtype, C, K, Hq, Hkv, D, hs, max_ctx, kv_split_pages, page_size);
  if (!ws || !aligned(ws, 256) || ws_bytes < p.total) return HSPEC_ERR_WORKSPACE;
  a = AttnArgs{};
  a.q = q; a.k_blk = kb; a.v_blk = vb; a.k_cache = kc; a.v_cache = vc;
  a.page_stride = ps; a.token_stride = ts; a.head_stride = hs;
  a.num_pages = num_pages; a.page_table = pt; a.max_pages = max_pages;
  a.ctx_lens = ctx; a.max_ctx = max_ctx;
  a.C = C; a.K = K; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D; a.rows = a.G * K;
  const float sc = scale > 0.f ? scale : 1.f / std::sqrt(float(D));
  a.scale_log2 = sc * 1.4426950408889634f;
  a.out = out;
  unsigned char* base = static_cast<unsigned char*>(ws);
  a.plan = reinterpret_cast<int32_t*>(base);
  a.part_o = base + p.part_o_off;
  a.part_ml = reinterpret_cast<float*>(base + p.part_ml_off);
  a.w_max = p.w_max;
  a.gran = p.gran;
  a.range_gran = p.range_gran;
  a.min_gran = p.min_gran;
  a.seg = p.seg;
  a.nbk = p.nbk;
  a.head_pair = p.head_pair;
  a.block_causal = block_causal;
  a.lsp = page_shift(page_size);
  return HSPEC_OK;
}

int run_attn(hipStream_t st, int dtype, int C, int K, int Hq, int Hkv, int D, const void* q,
             const void* kb, const void* vb, const void* kc, const void* vc, int64_t ps, int64_t ts,
             int64_t hs, int num_pages, int page_size, const int32_t* pt, int max_pages,
             const int32_t* ctx, int max_ctx, int kv_split_pages, float scale, int block_causal,
             void* out, void* ws, size_t ws_bytes) {
  AttnArgs a;
  const int st_ = attn_args(a, dtype, C, K, Hq, Hkv, D, q, kb, vb, kc, vc, ps, ts, hs, num_pages, page_size, pt,
                            max_pages, ctx, max_ctx, kv_split_pages, scale, block_causal, out, ws, ws_bytes);
  if (st_ != HSPEC_OK) return st_;
  return status_of(launch_block_attn(st, dtype, a));
}

// Workspace of the Mamba-2 block: the fp32 projection (which the scan reads
// through its fused convolution), the scan output, the normalised
// activations, and split-K partials of either projection.
struct BlockPlan {
  int T, d_inner, conv_dim, d_proj, ngN;
  GemmPlan in_p, out_p;
  size_t zx_off, y_off, n_off, part_off, total;
};

BlockPlan block_plan(const hspec_mamba_args* a) {
  BlockPlan p{};
  p.T = a->C * a->K;
  p.d_inner = a->H * a->P;
  p.ngN = a->ng * a->N;
  p.conv_dim = p.d_inner + 2 * p.ngN;
  p.d_proj = 2 * p.d_inner + 2 * p.ngN + a->H;
  p.in_p = gemm_plan(a->dtype, p.T, p.d_proj, a->d_model);
  p.out_p = gemm_plan(a->dtype, p.T, a->d_model, p.d_inner);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  const size_t T = size_t(p.T);
  p.zx_off = take(T * p.d_proj * 4);
  p.y_off = take(T * p.d_inner * 4);
  p.n_off = take(T * p.d_inner * esize(a->dtype));
  p.part_off = take(std::max(p.in_p.part_floats, p.out_p.part_floats) * 4);
  p.total = std::max<size_t>(off, 256);
  return p;
}

int check_block(const hspec_mamba_args* a) {
  if (!a) return HSPEC_ERR_INVALID_ARG;
  if (!dtype_ok(a->dtype) || a->C < 1 || a->K < 1 || a->d_model < 1) return HSPEC_ERR_INVALID_ARG;
  if (!a->hidden || !a->w_in || !a->conv_w || !a->dt_bias || !a->A || !a->norm_w || !a->w_out || !a->out)
    return HSPEC_ERR_INVALID_ARG;
  const void* al16[] = {a->hidden, a->w_in, a->w_out, a->out, a->conv_w, a->norm_w};
  for (const void* q : al16)
    if (!aligned(q, 16)) return HSPEC_ERR_INVALID_ARG;
  if (!(a->norm_eps >= 0.f) || !std::isfinite(a->norm_eps)) return HSPEC_ERR_INVALID_ARG;
  // the scan's own limits (its inputs are workspace buffers here)
  const int st = check_ssd_shape(HSPEC_F32, a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk, true);
  if (st != HSPEC_OK) return st;
  const int64_t d_inner = int64_t(a->H) * a->P;
  const int64_t d_proj = 2 * d_inner + 2 * int64_t(a->ng) * a->N + a->H;
  const int64_t T = int64_t(a->C) * a->K;
  if (a->d_model % 8 || d_inner % 8) return HSPEC_ERR_UNSUPPORTED;
  // row and column counts stay ints, and so do the projections' tile counts
  if (T > (1 << 30) || d_proj > (1 << 30)) return HSPEC_ERR_UNSUPPORTED;
  if (T * std::max<int64_t>(d_proj, a->d_model) > kMaxGemmOut) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

int run_block(hipStream_t s, const hspec_mamba_args* a, const BlockPlan& p) {
  unsigned char* ws = static_cast<unsigned char*>(a->workspace);
  float* zx = reinterpret_cast<float*>(ws + p.zx_off);
  float* y = reinterpret_cast<float*>(ws + p.y_off);
  void* normed = ws + p.n_off;
  float* part = reinterpret_cast<float*>(ws + p.part_off);
  GemmArgs gi{};
  gi.a = a->hidden; gi.b = a->w_in; gi.c = zx; gi.part = part;
  gi.M = p.T; gi.N = p.d_proj; gi.K = a->d_model;
  gi.lda = a->d_model; gi.ldb = a->d_model; gi.ldc = p.d_proj;
  int st = status_of(launch_gemm_tn(s, a->dtype, 1, gi, p.in_p));
  if (st != HSPEC_OK) return st;
  SsdArgs sa{nullptr, nullptr, a->A, nullptr, nullptr, a->Dskip, a->h0, y, a->h_final,
             a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk,
             zx, a->conv_w, a->conv_b, a->dt_bias, p.d_proj, p.d_inner};
  st = status_of(launch_ssd_scan(s, HSPEC_F32, sa));
  if (st != HSPEC_OK) return st;
  GateNormArgs gn{y, zx, a->norm_w, a->norm_eps, normed, p.T, p.d_inner, p.d_proj};
  st = status_of(launch_gate_norm(s, a->dtype, gn));
  if (st != HSPEC_OK) return st;
  GemmArgs go{};
  go.a = normed; go.b = a->w_out; go.c = a->out; go.part = part;
  go.M = p.T; go.N = a->d_model; go.K = p.d_inner;
  go.lda = p.d_inner; go.ldb = p.d_inner; go.ldc = a->d_model;
  return status_of(launch_gemm_tn(s, a->dtype, 0, go, p.out_p));
}

int check_inject(int dtype, int C, int n_new, int d, int Hkv, int D, const void* hidden,
                 const void* w_kv, const void* kc, const void* vc, int64_t ps, int64_t ts, int64_t hs,
                 int num_pages, int page_size, const int32_t* pt, int max_pages, const int32_t* start,
                 const size_t* ws_bytes) {
  if (!dtype_ok(dtype) || C < 1 || n_new < 1 || d < 1 || Hkv < 1 || D < 1) return HSPEC_ERR_INVALID_ARG;
  if (!hidden || !w_kv || !kc || !vc || !pt || !start || !ws_bytes) return HSPEC_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(w_kv, 16) || !aligned(pt, 4) || !aligned(start, 4))
    return HSPEC_ERR_INVALID_ARG;
  const int vec = 16 / esize(dtype);
  if (ps <= 0 || ts <= 0 || hs <= 0 || ps % vec || ts % vec || hs % vec) return HSPEC_ERR_INVALID_ARG;
  if (num_pages < 1 || max_pages < 1 || page_size < 1) return HSPEC_ERR_INVALID_ARG;
  if (page_shift(page_size) < 0) return HSPEC_ERR_UNSUPPORTED;
  if (d % 8) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(C) * n_new > (1 << 30) || int64_t(Hkv) * D > (1 << 28)) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(C) * n_new * 2 * Hkv * D > kMaxGemmOut) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

// ---------------------------------------------------------------------------
// the drafter stack
// ---------------------------------------------------------------------------

hspec_mamba_args block_args_of(const hspec_stack_args* a, const hspec_stack_layer& L, const void* x,
                               const float* h0, void* out, void* ws, size_t ws_bytes) {
  hspec_mamba_args m{};
  m.dtype = a->dtype; m.C = a->C; m.K = a->K; m.d_model = a->d_model;
  m.H = a->H; m.P = a->P; m.ng = a->ng; m.N = a->N; m.chunk = a->chunk;
  m.hidden = x; m.w_in = L.w_in; m.conv_w = L.conv_w; m.conv_b = L.conv_b; m.dt_bias = L.dt_bias;
  m.A = L.A; m.Dskip = L.Dskip; m.h0 = h0; m.norm_w = L.norm_w; m.norm_eps = a->eps; m.w_out = L.w_out;
  m.out = out; m.h_final = nullptr; m.workspace = ws; m.workspace_bytes = ws_bytes;
  return m;
}

struct StackPlan {
  int T, S;
  BlockPlan bp;
  AttnPlanShape ap;
  GemmPlan gq, gkv, go;
  size_t x_off, ym_off, ya_off, q_off, k_off, v_off, o_off, h0_off, blk_off, attn_off, part_off, total;
};

StackPlan stack_plan(const hspec_stack_args* a) {
  StackPlan p{};
  p.T = a->C * a->K;
  p.S = a->H * a->P * a->N;
  const hspec_stack_layer L{};
  const hspec_mamba_args m = block_args_of(a, L, nullptr, nullptr, nullptr, nullptr, 0);
  p.bp = block_plan(&m);
  p.ap = plan_shape(a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->head_stride, a->max_ctx, a->kv_split_pages,
                    a->page_size);
  p.gq = gemm_plan(a->dtype, p.T, a->Hq * a->D, a->d_model);
  p.gkv = gemm_plan(a->dtype, p.T, a->Hkv * a->D, a->d_model);
  p.go = gemm_plan(a->dtype, p.T, a->d_model, a->Hq * a->D);
  const size_t e = esize(a->dtype), T = size_t(p.T);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  p.x_off = take(T * a->d_model * e);
  p.ym_off = take(T * a->d_model * e);
  p.ya_off = take(T * a->d_model * e);
  p.q_off = take(T * a->Hq * a->D * e);
  p.k_off = take(T * a->Hkv * a->D * e);
  p.v_off = take(T * a->Hkv * a->D * e);
  p.o_off = take(T * a->Hq * a->D * e);
  p.h0_off = take(size_t(a->C) * p.S * 4);
  p.blk_off = take(p.bp.total);
  p.attn_off = take(p.ap.total);
  p.part_off = take(std::max({p.gq.part_floats, p.gkv.part_floats, p.go.part_floats}) * 4);
  p.total = std::max<size_t>(off, 256);
  return p;
}

int check_stack(const hspec_stack_args* a) {
  if (!a || !a->layers || a->n_layers < 1) return HSPEC_ERR_INVALID_ARG;
  if (!dtype_ok(a->dtype) || a->C < 1 || a->K < 1 || a->d_model < 1) return HSPEC_ERR_INVALID_ARG;
  if (!a->hidden_in || !a->u || !a->hidden_out) return HSPEC_ERR_INVALID_ARG;
  const void* al16[] = {a->hidden_in, a->u, a->hidden_out};
  for (const void* q : al16)
    if (!aligned(q, 16)) return HSPEC_ERR_INVALID_ARG;
  if (!(a->eps >= 0.f) || !std::isfinite(a->eps)) return HSPEC_ERR_INVALID_ARG;
  if (a->d_model % 8) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(a->C) * a->K > (1 << 30) || int64_t(a->Hq) * a->D > (1 << 28)) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(a->C) * a->K * std::max<int64_t>(int64_t(a->Hq) * a->D, a->d_model) > kMaxGemmOut)
    return HSPEC_ERR_UNSUPPORTED;
  for (int l = 0; l < a->n_layers; ++l) {
    const hspec_stack_layer& L = a->layers[l];
    if (!L.pre_norm_w || !aligned(L.pre_norm_w, 16)) return HSPEC_ERR_INVALID_ARG;
    if (L.w_in) {
      if (int64_t(a->H) * a->P * a->N > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
      int st = check_init(a->dtype, a->C, a->d_model, a->H * a->P * a->N, a->u, L.w_init, a->hidden_out);
      if (st != HSPEC_OK) return st;
      const hspec_mamba_args m = block_args_of(a, L, a->hidden_in, a->hidden_out, a->hidden_out, nullptr, 0);
      st = check_block(&m);
      if (st != HSPEC_OK) return st;
    }
    if (L.wq) {
      if (!L.wk || !L.wv || !L.wo) return HSPEC_ERR_INVALID_ARG;
      const void* w16[] = {L.wq, L.wk, L.wv, L.wo};
      for (const void* q : w16)
        if (!aligned(q, 16)) return HSPEC_ERR_INVALID_ARG;
      if ((int64_t(a->Hq) * a->D) % 8) return HSPEC_ERR_UNSUPPORTED;
      size_t dummy = 0;
      const int st = check_attn(a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->hidden_in, a->hidden_in,
                                a->hidden_in, L.k_cache, L.v_cache, a->page_stride, a->token_stride,
                                a->head_stride, a->num_pages, a->page_size, a->page_table, a->max_pages,
                                a->ctx_lens, a->max_ctx, a->kv_split_pages, a->scale, 0, a->hidden_in, &dummy);
      if (st != HSPEC_OK) return st;
    }
  }
  return HSPEC_OK;
}

// Enqueue the stack.  s1 == s0 (ev null): everything in order on one stream.
// With ev (2 events per layer): each layer's state projection and Mamba half
// run on s1 once x is ready, concurrently with the attention half on s0,
// which waits for them before the next layer boundary.  (Running all state
// projections up front on a third branch was measured: faster at C = 128,
// 2.23 vs 2.26 ms, slower at C = 1, 0.31 vs 0.28 ms, where the extra W_init
// streams compete with layer 0 for HBM.)
int enqueue_stack(const hspec_stack_args* a, const StackPlan& p, hipStream_t s0, hipStream_t s1,
                  hipEvent_t* ev) {
  unsigned char* ws = static_cast<unsigned char*>(a->workspace);
  void* x = ws + p.x_off;
  void* ym = ws + p.ym_off;
  void* ya = ws + p.ya_off;
  void* q = ws + p.q_off;
  void* kb = ws + p.k_off;
  void* vb = ws + p.v_off;
  void* o = ws + p.o_off;
  float* h0 = reinterpret_cast<float*>(ws + p.h0_off);
  float* part = reinterpret_cast<float*>(ws + p.part_off);
  const int d = a->d_model, HqD = a->Hq * a->D, HkvD = a->Hkv * a->D;
  AddNormArgs an{a->hidden_out, a->hidden_in, nullptr, nullptr, a->layers[0].pre_norm_w, a->eps, x, p.T, d};
  int st = status_of(launch_add_norm(s0, a->dtype, an));
  for (int l = 0; l < a->n_layers && st == HSPEC_OK; ++l) {
    const hspec_stack_layer& L = a->layers[l];
    if (L.w_in) {
      if (ev) {
        if (hipEventRecord(ev[2 * l], s0) != hipSuccess || hipStreamWaitEvent(s1, ev[2 * l], 0) != hipSuccess)
          return HSPEC_ERR_HIP;
      }
      InitArgs ia{a->u, L.w_init, h0, a->C, d, p.S};
      st = status_of(launch_init_state(s1, a->dtype, ia));
      if (st != HSPEC_OK) return st;
      const hspec_mamba_args m = block_args_of(a, L, x, h0, ym, ws + p.blk_off, p.bp.total);
      st = run_block(s1, &m, p.bp);
      if (st != HSPEC_OK) return st;
      if (ev && hipEventRecord(ev[2 * l + 1], s1) != hipSuccess) return HSPEC_ERR_HIP;
    }
    if (L.wq) {
      auto proj = [&](const void* A, const void* W, void* C, int N, int K, const GemmPlan& gp) {
        GemmArgs g{};
        g.a = A; g.b = W; g.c = C; g.part = part;
        g.M = p.T; g.N = N; g.K = K; g.lda = K; g.ldb = K; g.ldc = N;
        return status_of(launch_gemm_tn(s0, a->dtype, 0, g, gp));
      };
      st = proj(x, L.wq, q, HqD, d, p.gq);
      if (st == HSPEC_OK) st = proj(x, L.wk, kb, HkvD, d, p.gkv);
      if (st == HSPEC_OK) st = proj(x, L.wv, vb, HkvD, d, p.gkv);
      if (st == HSPEC_OK)
        st = run_attn(s0, a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, q, kb, vb, L.k_cache, L.v_cache,
                      a->page_stride, a->token_stride, a->head_stride, a->num_pages, a->page_size,
                      a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages, a->scale, 0,
                      o, ws + p.attn_off, p.ap.total);
      if (st == HSPEC_OK) st = proj(o, L.wo, ya, d, HqD, p.go);
      if (st != HSPEC_OK) return st;
    }
    if (L.w_in && ev && hipStreamWaitEvent(s0, ev[2 * l + 1], 0) != hipSuccess) return HSPEC_ERR_HIP;
    const float* nw = l + 1 < a->n_layers ? a->layers[l + 1].pre_norm_w : nullptr;
    AddNormArgs bn{a->hidden_out, nullptr, L.w_in ? ym : nullptr, L.wq ? ya : nullptr, nw, a->eps, x, p.T, d};
    st = status_of(launch_add_norm(s0, a->dtype, bn));
  }
  return st;
}

int check_layer(const hspec_layer_args* a, size_t* need) {
  if (!a) return HSPEC_ERR_INVALID_ARG;
  int st = check_ssd(a->dtype, a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk, a->x, a->delta, a->A,
                     a->B, a->Cm, a->y);
  if (st != HSPEC_OK) return st;
  if (int64_t(a->H) * a->P * a->N > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  // u and w_init both NULL: the direct-reuse-only ablation (no a1, zero state)
  if (a->u || a->w_init) {
    st = check_init(a->dtype, a->C, a->d_model, a->H * a->P * a->N, a->u, a->w_init, a->h0);
    if (st != HSPEC_OK) return st;
  }
  size_t dummy = 0;
  st = check_attn(a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->q, a->k_blk, a->v_blk, a->k_cache,
                  a->v_cache, a->page_stride, a->token_stride, a->head_stride, a->num_pages,
                  a->page_size, a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages,
                  a->scale, a->block_causal, a->out, &dummy);
  if (st != HSPEC_OK) return st;
  *need = plan_shape(a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->head_stride, a->max_ctx, a->kv_split_pages,
                     a->page_size).total;
  return HSPEC_OK;
}

// The layer on one stream: the attention (a0/a3; a4 too unless it joins the
// scan), the state projection (a1), then the scan (a2) and, when some request
// has several splits, the merge of the attention's partials (a4) in one
// launch, so that those two small latency-bound kernels overlap.
int enqueue_layer(const hspec_layer_args* a, hipStream_t s) {
  const bool no_init = !a->u && !a->w_init;
  SsdArgs sa{a->x, a->delta, a->A, a->B, a->Cm, a->Dskip, no_init ? nullptr : a->h0, a->y, a->h_final,
             a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk};
  AttnArgs m;
  int st = attn_args(m, a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->q, a->k_blk, a->v_blk, a->k_cache, a->v_cache,
                     a->page_stride, a->token_stride, a->head_stride, a->num_pages, a->page_size,
                     a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages, a->scale,
                     a->block_causal, a->out, a->workspace, a->workspace_bytes);
  if (st != HSPEC_OK) return st;
  const bool fused = scan_merge_fits(a->dtype, sa, m);
  st = status_of(launch_block_attn(s, a->dtype, m, !fused));
  if (st == HSPEC_OK && !no_init) {
    InitArgs ia{a->u, a->w_init, a->h0, a->C, a->d_model, a->H * a->P * a->N};
    st = status_of(launch_init_state(s, a->dtype, ia));
  }
  if (st != HSPEC_OK) return st;
  return status_of(fused ? launch_scan_merge(s, sa, m) : launch_ssd_scan(s, a->dtype, sa));
}

}  // namespace

// Workspace of hspec_draft_layer_noalloc: one static array per GPU, so that
// entry point allocates nothing.  In host code `scratch` names only a host
// stand-in for the device array: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to kernels.
static __device__ __align__(256) unsigned char scratch[HSPEC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the calling thread's current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HSPEC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HSPEC_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return HSPEC_OK;
}

}  // namespace

struct hspec_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

// Capture `enqueue(s0, s1, events)` on two private streams into an
// executable graph: n_events events for the fork / join points.
template <typename F>
int capture_graph(int n_events, F&& enqueue, hspec_graph* out) {
  hipStream_t s0 = nullptr, s1 = nullptr;
  std::vector<hipEvent_t> ev(n_events, nullptr);
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int st = HSPEC_OK;
  bool ok = hipStreamCreateWithFlags(&s0, hipStreamNonBlocking) == hipSuccess &&
            hipStreamCreateWithFlags(&s1, hipStreamNonBlocking) == hipSuccess;
  for (auto& e : ev) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
  if (ok && hipStreamBeginCapture(s0, hipStreamCaptureModeThreadLocal) == hipSuccess) {
    st = enqueue(s0, s1, ev.data());
    const hipError_t ec = hipStreamEndCapture(s0, &graph);
    ok = st == HSPEC_OK && ec == hipSuccess && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
  } else {
    ok = false;
  }
  for (auto& e : ev)
    if (e) hipEventDestroy(e);
  if (s1) hipStreamDestroy(s1);
  if (s0) hipStreamDestroy(s0);
  if (!ok) {
    if (exec) hipGraphExecDestroy(exec);
    if (graph) hipGraphDestroy(graph);
    return st != HSPEC_OK ? st : HSPEC_ERR_HIP;
  }
  *out = new hspec_graph_s{graph, exec};
  return HSPEC_OK;
}

}  // namespace

extern "C" {

const char* hspec_status_string(int status) {
  switch (status) {
    case HSPEC_OK: return "HSPEC_OK";
    case HSPEC_ERR_INVALID_ARG: return "HSPEC_ERR_INVALID_ARG";
    case HSPEC_ERR_UNSUPPORTED: return "HSPEC_ERR_UNSUPPORTED";
    case HSPEC_ERR_WORKSPACE: return "HSPEC_ERR_WORKSPACE";
    case HSPEC_ERR_HIP: return "HSPEC_ERR_HIP";
    case HSPEC_ERR_SCRATCH: return "HSPEC_ERR_SCRATCH";
    default: return "HSPEC_UNKNOWN_STATUS";
  }
}

int hspec_abi_version(void) { return HSPEC_ABI_VERSION; }

size_t hspec_layer_args_size(void) { return sizeof(hspec_layer_args); }

int hspec_init_state(void* stream, int dtype, int C, int d_model, int S, const void* u,
                     const void* w_init, float* h0) {
  const int st = check_init(dtype, C, d_model, S, u, w_init, h0);
  if (st != HSPEC_OK) return st;
  InitArgs a{u, w_init, h0, C, d_model, S};
  return status_of(launch_init_state(static_cast<hipStream_t>(stream), dtype, a));
}

int hspec_ssd_scan(void* stream, int dtype, int C, int K, int H, int P, int ng, int N, int chunk,
                   const void* x, const float* delta, const float* A, const void* B, const void* Cm,
                   const float* Dskip, const float* h0, float* y, float* h_final) {
  const int st = check_ssd(dtype, C, K, H, P, ng, N, chunk, x, delta, A, B, Cm, y);
  if (st != HSPEC_OK) return st;
  SsdArgs a{x, delta, A, B, Cm, Dskip, h0, y, h_final, C, K, H, P, ng, N, chunk};
  return status_of(launch_ssd_scan(static_cast<hipStream_t>(stream), dtype, a));
}

int hspec_block_attn_inplace(void* stream, int dtype, int C, int K, int Hq, int Hkv, int D,
                             const void* q, const void* k_blk, const void* v_blk,
                             const void* k_cache, const void* v_cache, int64_t page_stride,
                             int64_t token_stride, int64_t head_stride, int num_pages, int page_size,
                             const int32_t* page_table, int max_pages, const int32_t* ctx_lens,
                             int max_ctx, int kv_split_pages, float scale, int block_causal,
                             void* out, void* workspace, size_t* workspace_bytes) {
  const int st = check_attn(dtype, C, K, Hq, Hkv, D, q, k_blk, v_blk, k_cache, v_cache, page_stride,
                            token_stride, head_stride, num_pages, page_size, page_table, max_pages,
                            ctx_lens, max_ctx, kv_split_pages, scale, block_causal, out, workspace_bytes);
  if (st != HSPEC_OK) return st;
  if (!workspace) {
    *workspace_bytes = plan_shape(dtype, C, K, Hq, Hkv, D, head_stride, max_ctx, kv_split_pages, page_size).total;
    return HSPEC_OK;
  }
  return run_attn(static_cast<hipStream_t>(stream), dtype, C, K, Hq, Hkv, D, q, k_blk, v_blk,
                  k_cache, v_cache, page_stride, token_stride, head_stride, num_pages, page_size,
                  page_table, max_pages, ctx_lens, max_ctx, kv_split_pages, scale, block_causal, out, workspace,
                  *workspace_bytes);
}

int hspec_draft_layer(void* stream, const hspec_layer_args* a, size_t* required_bytes) {
  size_t need = 0;
  const int st = check_layer(a, &need);
  if (st != HSPEC_OK) return st;
  if (required_bytes) *required_bytes = need;
  if (!a->workspace) return required_bytes ? HSPEC_OK : HSPEC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return enqueue_layer(a, s);
}

int hspec_draft_layer_noalloc(void* stream, const hspec_layer_args* a) {
  if (!a) return HSPEC_ERR_INVALID_ARG;
  if (a->workspace || a->workspace_bytes) return HSPEC_ERR_INVALID_ARG;
  size_t need = 0;
  int st = check_layer(a, &need);
  if (st != HSPEC_OK) return st;
  if (need > HSPEC_NOALLOC_SCRATCH_BYTES) return HSPEC_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != HSPEC_OK) return st;
  hspec_layer_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = HSPEC_NOALLOC_SCRATCH_BYTES;
  return enqueue_layer(&b, static_cast<hipStream_t>(stream));
}

int hspec_draft_layer_graph(const hspec_layer_args* a, hspec_graph* out) {
  if (!out) return HSPEC_ERR_INVALID_ARG;
  *out = nullptr;
  size_t need = 0;
  const int st = check_layer(a, &need);
  if (st != HSPEC_OK) return st;
  if (!a->workspace || !aligned(a->workspace, 256) || a->workspace_bytes < need) return HSPEC_ERR_WORKSPACE;
  // One branch: the Mamba half forked beside the attention half was measured
  // slower at every C (C = 1: 88 vs 75 us; C = 128: 841 vs 767 us) -- both
  // halves are HBM-bound, so running them together only interferes.
  return capture_graph(0, [&](hipStream_t s0, hipStream_t, hipEvent_t*) {
    return enqueue_layer(a, s0);
  }, out);
}

size_t hspec_mamba_args_size(void) { return sizeof(hspec_mamba_args); }

int hspec_mamba_block(void* stream, const hspec_mamba_args* a, size_t* required_bytes) {
  const int st = check_block(a);
  if (st != HSPEC_OK) return st;
  const BlockPlan p = block_plan(a);
  if (required_bytes) *required_bytes = p.total;
  if (!a->workspace) return required_bytes ? HSPEC_OK : HSPEC_ERR_WORKSPACE;
  if (!aligned(a->workspace, 256) || a->workspace_bytes < p.total) return HSPEC_ERR_WORKSPACE;
  return run_block(static_cast<hipStream_t>(stream), a, p);
}

int hspec_kv_inject(void* stream, int dtype, int C, int n_new, int d_model, int Hkv, int D,
                    const void* hidden, const void* w_kv, void* k_cache, void* v_cache,
                    int64_t page_stride, int64_t token_stride, int64_t head_stride, int num_pages,
                    int page_size, const int32_t* page_table, int max_pages, const int32_t* start_pos,
                    void* workspace, size_t* workspace_bytes) {
  const int st = check_inject(dtype, C, n_new, d_model, Hkv, D, hidden, w_kv, k_cache, v_cache,
                              page_stride, token_stride, head_stride, num_pages, page_size, page_table,
                              max_pages, start_pos, workspace_bytes);
  if (st != HSPEC_OK) return st;
  const int M = C * n_new, N = 2 * Hkv * D;
  const GemmPlan p = gemm_plan(dtype, M, N, d_model);
  const size_t need = std::max<size_t>(256, align256(p.part_floats * 4));
  if (!workspace) {
    *workspace_bytes = need;
    return HSPEC_OK;
  }
  if (!aligned(workspace, 256) || *workspace_bytes < need) return HSPEC_ERR_WORKSPACE;
  GemmArgs g{};
  g.a = hidden; g.b = w_kv; g.c = nullptr; g.part = static_cast<float*>(workspace);
  g.M = M; g.N = N; g.K = d_model; g.lda = d_model; g.ldb = d_model; g.ldc = N;
  g.scatter = 1;
  g.sc = KvScatter{page_table, start_pos, k_cache, v_cache, page_stride, token_stride, head_stride,
                   n_new, max_pages, num_pages, Hkv * D, D, 4 + page_shift(page_size)};
  return status_of(launch_gemm_tn(static_cast<hipStream_t>(stream), dtype, 0, g, p));
}

size_t hspec_stack_args_size(void) { return sizeof(hspec_stack_args); }

int hspec_draft_stack(void* stream, const hspec_stack_args* a, size_t* required_bytes) {
  const int st = check_stack(a);
  if (st != HSPEC_OK) return st;
  const StackPlan p = stack_plan(a);
  if (required_bytes) *required_bytes = p.total;
  if (!a->workspace) return required_bytes ? HSPEC_OK : HSPEC_ERR_WORKSPACE;
  if (!aligned(a->workspace, 256) || a->workspace_bytes < p.total) return HSPEC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return enqueue_stack(a, p, s, s, nullptr);
}

int hspec_draft_stack_graph(const hspec_stack_args* a, hspec_graph* out) {
  if (!out) return HSPEC_ERR_INVALID_ARG;
  *out = nullptr;
  const int st = check_stack(a);
  if (st != HSPEC_OK) return st;
  const StackPlan p = stack_plan(a);
  if (!a->workspace || !aligned(a->workspace, 256) || a->workspace_bytes < p.total) return HSPEC_ERR_WORKSPACE;
  return capture_graph(2 * a->n_layers, [&](hipStream_t s0, hipStream_t s1, hipEvent_t* ev) {
    return enqueue_stack(a, p, s0, s1, ev);
  }, out);
}

int hspec_graph_launch(hspec_graph g, void* stream) {
  if (!g) return HSPEC_ERR_INVALID_ARG;
  return status_of(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

int hspec_graph_destroy(hspec_graph g) {
  if (!g) return HSPEC_ERR_INVALID_ARG;
  const hipError_t e1 = hipGraphExecDestroy(g->exec);
  const hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  return (e1 == hipSuccess && e2 == hipSuccess) ? HSPEC_OK : HSPEC_ERR_HIP;
}

}  // extern "C"
