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

#include "../../include/hspec.h"
#include "kernels.h"

namespace hspec {
size_t ssd_lds_bytes(int P, int N, int Q);
}

using namespace hspec;

namespace {

constexpr size_t kMaxLds = 160 * 1024;

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
  if (int64_t(S) / 64 > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

// shape limits of the scan (pointers are checked by the callers)
int check_ssd_shape(int dtype, int C, int K, int H, int P, int ng, int N, int chunk) {
  if (!dtype_ok(dtype) || C < 1 || K < 1 || H < 1 || P < 1 || N < 1 || ng < 1 || chunk < 1)
    return HSPEC_ERR_INVALID_ARG;
  if (H % ng) return HSPEC_ERR_INVALID_ARG;
  if (chunk > 16 || (chunk & (chunk - 1))) return HSPEC_ERR_UNSUPPORTED;
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

struct AttnPlanShape {
  int pps, M, MS;  // 16-token slabs per split, C * MS work items, splits of a max_ctx request
  size_t plan_bytes, part_o_off, part_ml_off, total;
};

// log2(page_size / 16) for a supported page size, else -1
int page_shift(int page_size) {
  for (int l = 0; l <= 4; ++l)
    if (page_size == (16 << l)) return l;
  return -1;
}

// Slabs (16 tokens) per split; splits start on page boundaries, so the result
// is a multiple of the page's slab count spp.
int auto_pages_per_split(int C, int Hkv, int max_ctx, int spp) {
  const int max_pages = (max_ctx + 15) / 16;
  if (max_pages <= 0) return 16;
  const int64_t base = int64_t(C) * Hkv;
  // Aim at about 512 work items -- two per CU, one resident round at the
  // attention kernel's occupancy: measured at 8192-token contexts, C = 2..64,
  // 512 items beat both 256 (too little in flight) and 1024 (twice the
  // per-item prologue and fp32 partials: G*K rows x (D+2) written and read
  // back by the merge).  Past 512 (request, kv head) pairs nothing is split.
  const int64_t target = 512;
  if (base >= target) return (max_pages + spp - 1) / spp * spp;
  const int64_t splits = (target + base - 1) / base;
  int64_t pps = (max_pages + splits - 1) / splits;
  if (pps < 16) pps = 16;    // >= 256 tokens per item: partials stay small next to the KV they summarise
  const int64_t m = std::max(8, spp);
  return int((pps + m - 1) / m * m);
}

AttnPlanShape plan_shape(int C, int K, int Hq, int Hkv, int D, int max_ctx, int kv_split_pages,
                         int page_size) {
  AttnPlanShape p{};
  const int spp = page_size / 16;
  p.pps = kv_split_pages > 0 ? kv_split_pages * spp : auto_pages_per_split(C, Hkv, max_ctx, spp);
  const int64_t max_pages = (int64_t(max_ctx) + 15) / 16;
  const int64_t max_splits = std::max<int64_t>(1, (max_pages + p.pps - 1) / p.pps);
  p.MS = int(std::min<int64_t>(max_splits, 0x7fffffff));
  p.M = int(std::min<int64_t>(int64_t(C) * max_splits, 0x7fffffff));
  const size_t rows = size_t(Hq / Hkv) * K;
  p.plan_bytes = align256(size_t(4 + 2 * size_t(C) + 2 * size_t(p.M)) * 4);
  p.part_o_off = p.plan_bytes;
  size_t po = 0, pml = 0;
  if (p.M > C) {  // only then can a request have more than one split
    po = align256(size_t(p.M) * Hkv * rows * D * 4);
    pml = align256(size_t(p.M) * Hkv * rows * 2 * 4);
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
  const AttnPlanShape p = plan_shape(C, K, Hq, Hkv, D, max_ctx, kv_split_pages, page_size);
  if (int64_t(C) * p.MS * Hkv > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

int run_attn(hipStream_t st, int dtype, int C, int K, int Hq, int Hkv, int D, const void* q,
             const void* kb, const void* vb, const void* kc, const void* vc, int64_t ps, int64_t ts,
             int64_t hs, int num_pages, int page_size, const int32_t* pt, int max_pages,
             const int32_t* ctx, int max_ctx, int kv_split_pages, float scale, int block_causal,
             void* out, void* ws, size_t ws_bytes) {
  const AttnPlanShape p = plan_shape(C, K, Hq, Hkv, D, max_ctx, kv_split_pages, page_size);
  if (!ws || !aligned(ws, 256) || ws_bytes < p.total) return HSPEC_ERR_WORKSPACE;
  AttnArgs a{};
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
  a.part_o = reinterpret_cast<float*>(base + p.part_o_off);
  a.part_ml = reinterpret_cast<float*>(base + p.part_ml_off);
  a.max_items = p.M;
  a.pps = p.pps;
  a.max_splits = p.MS;
  a.block_causal = block_causal;
  a.lsp = page_shift(page_size);
  return status_of(launch_block_attn(st, dtype, a));
}

// Workspace of the Mamba-2 block: fp32 projection, scan inputs and output,
// the normalised activations, and split-K partials of either projection.
struct BlockPlan {
  int T, d_inner, conv_dim, d_proj, ngN;
  GemmPlan in_p, out_p;
  size_t zx_off, x_off, b_off, c_off, dt_off, y_off, n_off, part_off, total;
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
  p.x_off = take(T * p.d_inner * 4);
  p.b_off = take(T * p.ngN * 4);
  p.c_off = take(T * p.ngN * 4);
  p.dt_off = take(T * a->H * 4);
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
  const int st = check_ssd_shape(HSPEC_F32, a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk);
  if (st != HSPEC_OK) return st;
  const int64_t d_inner = int64_t(a->H) * a->P;
  const int64_t d_proj = 2 * d_inner + 2 * int64_t(a->ng) * a->N + a->H;
  const int64_t T = int64_t(a->C) * a->K;
  if (a->d_model % 8 || d_inner % 8) return HSPEC_ERR_UNSUPPORTED;
  // row and column counts stay ints; requests index grid.y of the conv kernel
  if (T > (1 << 30) || d_proj > (1 << 30) || a->C > 65535) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

int run_block(hipStream_t s, const hspec_mamba_args* a, const BlockPlan& p) {
  unsigned char* ws = static_cast<unsigned char*>(a->workspace);
  float* zx = reinterpret_cast<float*>(ws + p.zx_off);
  float* xs = reinterpret_cast<float*>(ws + p.x_off);
  float* bs = reinterpret_cast<float*>(ws + p.b_off);
  float* cs = reinterpret_cast<float*>(ws + p.c_off);
  float* dt = reinterpret_cast<float*>(ws + p.dt_off);
  float* y = reinterpret_cast<float*>(ws + p.y_off);
  void* normed = ws + p.n_off;
  float* part = reinterpret_cast<float*>(ws + p.part_off);
  GemmArgs gi{};
  gi.a = a->hidden; gi.b = a->w_in; gi.c = zx; gi.part = part;
  gi.M = p.T; gi.N = p.d_proj; gi.K = a->d_model;
  gi.lda = a->d_model; gi.ldb = a->d_model; gi.ldc = p.d_proj;
  int st = status_of(launch_gemm_tn(s, a->dtype, 1, gi, p.in_p));
  if (st != HSPEC_OK) return st;
  ConvActArgs ca{zx, a->conv_w, a->conv_b, a->dt_bias, xs, bs, cs, dt,
                 a->C, a->K, p.d_inner, p.ngN, a->H, p.d_proj};
  st = status_of(launch_conv_act(s, ca));
  if (st != HSPEC_OK) return st;
  SsdArgs sa{xs, dt, a->A, bs, cs, a->Dskip, a->h0, y, a->h_final,
             a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk};
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
    *workspace_bytes = plan_shape(C, K, Hq, Hkv, D, max_ctx, kv_split_pages, page_size).total;
    return HSPEC_OK;
  }
  return run_attn(static_cast<hipStream_t>(stream), dtype, C, K, Hq, Hkv, D, q, k_blk, v_blk,
                  k_cache, v_cache, page_stride, token_stride, head_stride, num_pages, page_size,
                  page_table, max_pages, ctx_lens, max_ctx, kv_split_pages, scale, block_causal, out, workspace,
                  *workspace_bytes);
}

int hspec_draft_layer(void* stream, const hspec_layer_args* a, size_t* required_bytes) {
  if (!a) return HSPEC_ERR_INVALID_ARG;
  int st = check_ssd(a->dtype, a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk, a->x, a->delta, a->A,
                     a->B, a->Cm, a->y);
  if (st != HSPEC_OK) return st;
  if (int64_t(a->H) * a->P * a->N > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  const int S = a->H * a->P * a->N;
  // u and w_init both NULL: the direct-reuse-only ablation (no a1, zero state)
  const bool no_init = !a->u && !a->w_init;
  if (!no_init) {
    st = check_init(a->dtype, a->C, a->d_model, S, a->u, a->w_init, a->h0);
    if (st != HSPEC_OK) return st;
  }
  size_t dummy = 0;
  st = check_attn(a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->q, a->k_blk, a->v_blk, a->k_cache,
                  a->v_cache, a->page_stride, a->token_stride, a->head_stride, a->num_pages,
                  a->page_size, a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages,
                  a->scale,
                  a->block_causal, a->out, &dummy);
  if (st != HSPEC_OK) return st;
  const size_t need = plan_shape(a->C, a->K, a->Hq, a->Hkv, a->D, a->max_ctx, a->kv_split_pages,
                                 a->page_size).total;
  if (required_bytes) *required_bytes = need;
  if (!a->workspace) return required_bytes ? HSPEC_OK : HSPEC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_attn(s, a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->q, a->k_blk, a->v_blk, a->k_cache,
                a->v_cache, a->page_stride, a->token_stride, a->head_stride, a->num_pages,
                a->page_size, a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages,
                a->scale,
                a->block_causal, a->out, a->workspace, a->workspace_bytes);
  if (st != HSPEC_OK) return st;
  if (!no_init) {
    InitArgs ia{a->u, a->w_init, a->h0, a->C, a->d_model, S};
    st = status_of(launch_init_state(s, a->dtype, ia));
    if (st != HSPEC_OK) return st;
  }
  SsdArgs sa{a->x, a->delta, a->A, a->B, a->Cm, a->Dskip, no_init ? nullptr : a->h0, a->y, a->h_final,
             a->C, a->K, a->H, a->P, a->ng, a->N, a->chunk};
  return status_of(launch_ssd_scan(s, a->dtype, sa));
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

}  // extern "C"
