// Launch interfaces between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hspec {

struct AttnArgs {
  const void* q;
  const void* k_blk;
  const void* v_blk;
  const void* k_cache;
  const void* v_cache;
  int64_t page_stride, token_stride, head_stride;
  int num_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* ctx_lens;
  int max_ctx;
  int C, K, Hq, Hkv, G, D, rows;  // rows = G * K query rows per kv head
  float scale_log2;               // softmax scale * log2(e)
  void* out;
  int32_t* plan;                  // workspace head: the work plan (written by the last block)
  void* part_o;                   // [2 * w_max, Hkv, rows, D], activation dtype: piece of range
                                  // w's segment k at slot 2w + k, normalised by its own l
  float* part_ml;                 // [2 * w_max, Hkv, rows, 2]
  // Work plan: each request's keys are its context slabs (16 tokens) then
  // nbk block slabs, counted in granules of `gran` slabs; the batch's
  // granules are cut into W <= w_max equal ranges, one workgroup per (range,
  // kv head group).  W = ceil(T / range_gran) for fixed ranges, else
  // min(w_max, max(1, floor(T / min_gran))) (T = the batch's granules).
  int w_max;
  int gran;
  int range_gran;                 // 0 = automatic
  int min_gran;
  int seg;                        // a request's fixed cost in units (automatic ranges; else 0)
  int nbk;
  int head_pair;                  // 1: two kv heads per workgroup when the shape allows (long ranges)
  int block_causal;               // 1: block query t sees block keys s <= t only
  int lsp;                        // log2(page size / 16)
};

// a0 + a3 + a4 on `st` (merge = false: a4 is left to launch_scan_merge).
hipError_t launch_block_attn(hipStream_t st, int dtype, const AttnArgs& a, bool merge = true);
// dynamic LDS bytes of the attention kernel for a shape (host planning only)
size_t attn_lds_bytes(int dtype, int D, int rows, int K);
// the merge's lanes per output: 4 when ranges outnumber requests four to one
bool merge_wide(const AttnArgs& a);
// whether the two-heads-per-workgroup form exists for a shape
bool head_pair_fits(int rows, int Hkv, int64_t head_stride, int dtype, int D);

struct SsdArgs {
  const void* x;
  const float* delta;
  const float* A;
  const void* B;
  const void* Cm;
  const float* Dskip;
  const float* h0;
  float* y;
  float* h_final;
  int C, K, H, P, ng, N, chunk;
  // Fused front of the Mamba-2 block (zx set; x, delta, B, Cm unused): the
  // scan reads the raw projection rows zx [C*K, d_proj] (z | x | B | C | dt)
  // and applies the width-4 causal convolution + SiLU and the softplus step
  // itself; fp32 only.
  const float* zx;
  const float* conv_w;   // [d_inner + 2*ng*N, 4]
  const float* conv_b;   // same channels, or null
  const float* dt_bias;  // [H]
  int d_proj, d_inner;
};
hipError_t launch_ssd_scan(hipStream_t st, int dtype, const SsdArgs& a);
// The drafter layer's last launch: a2's scan and a4's merge of the
// attention's partials in one grid (scan workgroups first).  Only for bf16
// activations, N % 4 == 0, chunks of at most 16, D = 128 and no fused
// convolution (scan_merge_fits); otherwise the two kernels run one after the
// other.
bool scan_merge_fits(int dtype, const SsdArgs& s, const AttnArgs& m);
hipError_t launch_scan_merge(hipStream_t st, const SsdArgs& s, const AttnArgs& m);

struct InitArgs {
  const void* u;
  const void* w;
  float* h0;
  int C, d, S;
};
hipError_t launch_init_state(hipStream_t st, int dtype, const InitArgs& a);

// Paged destination of a KV-injection GEMM: output row m = b * n_new + i is
// token position start[b] + i of request b; columns [0, HD) are its K row,
// [HD, 2*HD) its V row (head h at h*D .. h*D + D - 1).  A launch over the
// columns [col0, col0 + n) of the projection (a ragged tail launched on its
// own) numbers its columns from 0, so `col0` is added back before the
// column's pool and offset are looked up.
struct KvScatter {
  const int32_t* page_table;  // [C, max_pages]
  const int32_t* start;       // [C]
  void* k_cache;
  void* v_cache;
  int64_t ps, ts, hs;         // page, token, head strides in elements
  int n_new, max_pages, num_pages, HD, D;
  int lpt;                    // log2(tokens per page)
  int col0;                   // first projection column of this launch
};

// C[M, N] = A[M, K] . B[N, K]^T (row strides in elements); K % 8 == 0.
struct GemmArgs {
  const void* a;
  const void* b;
  void* c;          // OutT [M, ldc] (unused when scattering)
  float* part;      // fp32 [splits, M, N] split-K partials (splits > 1)
  int M, N, K, lda, ldb, ldc;
  int tiles_m, splits, kchunk;  // filled in by the launcher from the plan
  int scatter;                  // 1: write through `sc` instead of `c`
  KvScatter sc;
};
// One launch over output columns [n0, n0 + n).
struct GemmPart {
  int cfg, bm, bn, tiles_m, tiles, splits, kchunk, n0, n;
};
struct GemmPlan {
  GemmPart part[2];     // the columns, or the whole tiles and a ragged tail
  int nparts;
  size_t part_floats;   // workspace floats the split-K partials need
};
GemmPlan gemm_plan(int dtype, int M, int N, int K);
// out_f32: store fp32 (else the activation type of dtype)
hipError_t launch_gemm_tn(hipStream_t st, int dtype, int out_f32, const GemmArgs& g, const GemmPlan& p);

struct GateNormArgs {
  const float* y;       // fp32 [T, d_inner]
  const float* zx;      // fp32 [T, d_proj], z in columns [0, d_inner)
  const float* norm_w;  // fp32 [d_inner]
  float eps;
  void* out;            // act [T, d_inner]
  int T, d_inner, d_proj;
};
hipError_t launch_gate_norm(hipStream_t st, int dtype, const GateNormArgs& a);

// Residual stream between stack layers: h = src ? src : h + add0 + add1, then
// x = RMSNorm(h) * norm_w when norm_w is set.
struct AddNormArgs {
  float* h;             // fp32 [T, d], in place
  const void* src;      // act [T, d] or null
  const void* add0;     // act [T, d] or null
  const void* add1;     // act [T, d] or null
  const float* norm_w;  // fp32 [d] or null (no x)
  float eps;
  void* x;              // act [T, d]
  int T, d;
};
hipError_t launch_add_norm(hipStream_t st, int dtype, const AddNormArgs& a);

}  // namespace hspec
