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

int check_ssd(int dtype, int C, int K, int H, int P, int ng, int N, int chunk, const void* x,
              const float* delta, const float* A, const void* B, const void* Cm, const float* y) {
  if (!dtype_ok(dtype) || C < 1 || K < 1 || H < 1 || P < 1 || N < 1 || ng < 1 || chunk < 1)
    return HSPEC_ERR_INVALID_ARG;
  if (H % ng) return HSPEC_ERR_INVALID_ARG;
  if (!x || !delta || !A || !B || !Cm || !y) return HSPEC_ERR_INVALID_ARG;
  if (chunk > 16 || (chunk & (chunk - 1))) return HSPEC_ERR_UNSUPPORTED;
  if (P > 128 || N > 128) return HSPEC_ERR_UNSUPPORTED;
  if (ssd_lds_bytes(P, N, chunk) > kMaxLds) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(C) * H > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

struct AttnPlanShape {
  int pps, M, MS;  // pages per split, C * MS work items, splits of a max_ctx request
  size_t plan_bytes, part_o_off, part_ml_off, total;
};

int auto_pages_per_split(int C, int Hkv, int max_ctx) {
  const int max_pages = (max_ctx + 15) / 16;
  if (max_pages <= 0) return 16;
  const int64_t base = int64_t(C) * Hkv;
  // Aim at about 512 work items -- two per CU, one resident round at the
  // attention kernel's occupancy: measured at 8192-token contexts, C = 2..64,
  // 512 items beat both 256 (too little in flight) and 1024 (twice the
  // per-item prologue and fp32 partials: G*K rows x (D+2) written and read
  // back by the merge).  Past 512 (request, kv head) pairs nothing is split.
  const int64_t target = 512;
  if (base >= target) return max_pages;
  const int64_t splits = (target + base - 1) / base;
  int64_t pps = (max_pages + splits - 1) / splits;
  if (pps < 16) pps = 16;    // >= 256 tokens per item: partials stay small next to the KV they summarise
  return int((pps + 7) / 8 * 8);
}

AttnPlanShape plan_shape(int C, int K, int Hq, int Hkv, int D, int max_ctx, int kv_split_pages) {
  AttnPlanShape p{};
  p.pps = kv_split_pages > 0 ? kv_split_pages : auto_pages_per_split(C, Hkv, max_ctx);
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
               int num_pages, const int32_t* pt, int max_pages, const int32_t* ctx, int max_ctx,
               int kv_split_pages, float scale, int block_causal, const void* out,
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
  if (num_pages < 1 || max_ctx < 0 || kv_split_pages < 0) return HSPEC_ERR_INVALID_ARG;
  if (int64_t(max_pages) < std::max<int64_t>(1, (int64_t(max_ctx) + 15) / 16)) return HSPEC_ERR_INVALID_ARG;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return HSPEC_ERR_INVALID_ARG;
  if (block_causal != 0 && block_causal != 1) return HSPEC_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return HSPEC_ERR_UNSUPPORTED;
  if (K > 64) return HSPEC_ERR_UNSUPPORTED;
  if (int64_t(Hq / Hkv) * K > 256) return HSPEC_ERR_UNSUPPORTED;
  if (attn_lds_bytes(dtype, D, (Hq / Hkv) * K, K) > kMaxLds) return HSPEC_ERR_UNSUPPORTED;
  const AttnPlanShape p = plan_shape(C, K, Hq, Hkv, D, max_ctx, kv_split_pages);
  if (int64_t(C) * p.MS * Hkv > 0x7fffffff) return HSPEC_ERR_UNSUPPORTED;
  return HSPEC_OK;
}

int run_attn(hipStream_t st, int dtype, int C, int K, int Hq, int Hkv, int D, const void* q,
             const void* kb, const void* vb, const void* kc, const void* vc, int64_t ps, int64_t ts,
             int64_t hs, int num_pages, const int32_t* pt, int max_pages, const int32_t* ctx,
             int max_ctx, int kv_split_pages, float scale, int block_causal, void* out, void* ws,
             size_t ws_bytes) {
  const AttnPlanShape p = plan_shape(C, K, Hq, Hkv, D, max_ctx, kv_split_pages);
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
  return status_of(launch_block_attn(st, dtype, a));
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
                             int64_t token_stride, int64_t head_stride, int num_pages,
                             const int32_t* page_table, int max_pages, const int32_t* ctx_lens,
                             int max_ctx, int kv_split_pages, float scale, int block_causal,
                             void* out, void* workspace, size_t* workspace_bytes) {
  const int st = check_attn(dtype, C, K, Hq, Hkv, D, q, k_blk, v_blk, k_cache, v_cache, page_stride,
                            token_stride, head_stride, num_pages, page_table, max_pages, ctx_lens,
                            max_ctx, kv_split_pages, scale, block_causal, out, workspace_bytes);
  if (st != HSPEC_OK) return st;
  if (!workspace) {
    *workspace_bytes = plan_shape(C, K, Hq, Hkv, D, max_ctx, kv_split_pages).total;
    return HSPEC_OK;
  }
  return run_attn(static_cast<hipStream_t>(stream), dtype, C, K, Hq, Hkv, D, q, k_blk, v_blk,
                  k_cache, v_cache, page_stride, token_stride, head_stride, num_pages, page_table,
                  max_pages, ctx_lens, max_ctx, kv_split_pages, scale, block_causal, out, workspace,
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
                  a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages, a->scale,
                  a->block_causal, a->out, &dummy);
  if (st != HSPEC_OK) return st;
  const size_t need = plan_shape(a->C, a->K, a->Hq, a->Hkv, a->D, a->max_ctx, a->kv_split_pages).total;
  if (required_bytes) *required_bytes = need;
  if (!a->workspace) return required_bytes ? HSPEC_OK : HSPEC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_attn(s, a->dtype, a->C, a->K, a->Hq, a->Hkv, a->D, a->q, a->k_blk, a->v_blk, a->k_cache,
                a->v_cache, a->page_stride, a->token_stride, a->head_stride, a->num_pages,
                a->page_table, a->max_pages, a->ctx_lens, a->max_ctx, a->kv_split_pages, a->scale,
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

}  // extern "C"
