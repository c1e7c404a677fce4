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
  int32_t* plan;                  // workspace head: the split plan (written by block 0)
  float* part_o;                  // [max_items, Hkv, rows, D], item = request * max_splits + split
  float* part_ml;                 // [max_items, Hkv, rows, 2]
  int max_items;                  // C * max_splits
  int pps, max_splits;            // context pages per split; splits of a max_ctx request
  int block_causal;               // 1: block query t sees block keys s <= t only
};

// a0 + a3 + a4 on `st`.
hipError_t launch_block_attn(hipStream_t st, int dtype, const AttnArgs& a);
// dynamic LDS bytes of the attention kernel for a shape (host planning only)
size_t attn_lds_bytes(int dtype, int D, int rows, int K);

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
};
hipError_t launch_ssd_scan(hipStream_t st, int dtype, const SsdArgs& a);

struct InitArgs {
  const void* u;
  const void* w;
  float* h0;
  int C, d, S;
};
hipError_t launch_init_state(hipStream_t st, int dtype, const InitArgs& a);

}  // namespace hspec
