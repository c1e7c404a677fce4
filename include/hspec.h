/*
 * hspec.h -- C ABI of libhspec.so, the MI355X (gfx950) drafter-layer library.
 *
 * The layer is the block-parallel drafter layer of "H-Spec: Parallel
 * Speculative Decoding Without a Drafter-Side KV Cache" (Abstract; review
 * page, Summary): a Mamba-2 module whose state starts from a projection of the
 * target's last-token hidden state and scans the K-token draft block in
 * parallel, and an attention module whose K block queries read the target's
 * paged KV cache in place -- the layer has no argument through which it
 * could write a drafter-side KV cache.
 *
 * Entry points
 *   hspec_init_state, hspec_ssd_scan,       the layer's steps (a1, a2, a0+a3+a4)
 *   hspec_block_attn_inplace
 *   hspec_draft_layer (+ _graph, _noalloc)  the layer (a5)
 *   hspec_mamba_block                       the Mamba-2 block around the scan
 *   hspec_draft_stack (+ _graph)            a stack of hybrid layers
 *   hspec_kv_inject                         contrast workload: the drafter-side
 *                                           KV injection H-Spec avoids
 *   hspec_graph_launch, hspec_graph_destroy the graph objects of the _graph forms
 *
 * Conventions shared by every entry point
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises.  Host-side
 *     argument errors are returned before anything is enqueued; launch errors
 *     come back as HSPEC_ERR_HIP; faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - All pointers except the integer metadata noted below are device
 *     pointers.  The caller owns every buffer; the library allocates no
 *     device memory and keeps no state between calls (the _graph forms create
 *     host-side HIP graph objects, freed by hspec_graph_destroy; the static
 *     scratch of hspec_draft_layer_noalloc and its per-device address live
 *     until the process ends), so calls on different streams may run
 *     concurrently as long as their output and workspace buffers differ.
 *   - `dtype` selects the element type of the "act" tensors: HSPEC_F32
 *     (float) or HSPEC_BF16 (bfloat16 bits).  Accumulation is always fp32.
 *   - Shapes are row-major, last index fastest; "act" tensors are contiguous
 *     unless strides are given; every device pointer must be 16-byte aligned.
 */
#ifndef HSPEC_H
#define HSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HSPEC_F32 = 0, HSPEC_BF16 = 1 } hspec_dtype;

typedef enum {
  HSPEC_OK = 0,
  HSPEC_ERR_INVALID_ARG = -1,   /* a size, pointer or stride breaks the contract      */
  HSPEC_ERR_UNSUPPORTED = -2,   /* legal but outside the shapes these kernels handle  */
  HSPEC_ERR_WORKSPACE = -3,     /* workspace pointer missing or smaller than required */
  HSPEC_ERR_HIP = -4,           /* the HIP runtime refused a launch                   */
  HSPEC_ERR_SCRATCH = -5        /* hspec_draft_layer_noalloc: the call needs more
                                   than HSPEC_NOALLOC_SCRATCH_BYTES of scratch       */
} hspec_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* hspec_status_string(int status);

/* ABI version of this header; bumped on any incompatible change. */
#define HSPEC_ABI_VERSION 8
int hspec_abi_version(void);

/*
 * a1 -- initial Mamba-2 state from the target's last-token hidden state.
 * H-Spec, Abstract and review Summary: the Mamba module is initialised from
 * a projection of the last-token target hidden state.  Linear, no bias:
 *
 *   h0[b, s] = sum_i u[b, i] * w_init[i, s],   s = (h*P + p)*N + n
 *
 *   u       act  [C, d_model]      last-token hidden state per request
 *   w_init  act  [d_model, S]      projection weight, S = H*P*N
 *   h0      fp32 [C, S]            output (overwritten)
 * Limits: 1 <= C <= 65536, d_model % 32 == 0, S % 64 == 0, S <= 2^25 (else
 * UNSUPPORTED).
 * Runs on bf16 (or fp32) matrix cores with fp32 accumulation.
 */
int hspec_init_state(void* stream, int dtype, int C, int d_model, int S,
                     const void* u, const void* w_init, float* h0);

/*
 * a2 -- Mamba-2 (SSD) chunked parallel scan over the draft block.
 * H-Spec, Abstract: the Mamba module keeps drafting block-parallel through
 * its parallel scan.  Per request b and head h (group g = h / (H/ng)):
 *
 *   H_t = exp(delta[b,t,h] * A[h]) * H_{t-1} + delta[b,t,h] * x[b,t,h,:] (outer) B[b,t,g,:]
 *   y[b,t,h,:] = H_t @ Cm[b,t,g,:] + Dskip[h] * x[b,t,h,:],     H_{-1} = h0[b,h]
 *
 * evaluated chunk by chunk (intra-chunk decay matrix + inter-chunk state
 * passing, Mamba-2's SSD form), which equals the recurrence exactly in real
 * arithmetic.
 *   x       act  [C, K, H, P]
 *   delta   fp32 [C, K, H]        step sizes, already positive
 *   A       fp32 [H]              per-head decay rate (negative)
 *   B, Cm   act  [C, K, ng, N]
 *   Dskip   fp32 [H] or NULL      NULL = no skip term
 *   h0      fp32 [C, H, P, N] or NULL (NULL = zero state); the layout of a1's h0
 *   y       fp32 [C, K, H, P]     output
 *   h_final fp32 [C, H, P, N] or NULL: the state after the last block position
 * Limits: chunk in {1, 2, 4, 8, 16, 32, 64} (the whole chunk is staged at
 * once: its decay matrix spans all its positions); chunks of 32 and 64 take
 * N <= 64 with N % 4 == 0; P <= 128; N <= 128; ng divides H (else
 * INVALID_ARG / UNSUPPORTED).
 */
int hspec_ssd_scan(void* stream, int dtype, int C, int K, int H, int P, int ng, int N, int chunk,
                   const void* x, const float* delta, const float* A,
                   const void* B, const void* Cm, const float* Dskip,
                   const float* h0, float* y, float* h_final);

/*
 * a0 + a3 + a4 -- block-query attention over the target's paged KV, in place.
 * H-Spec, Abstract and review Summary: attention reuses the target's KV
 * where it lies; no drafter-side KV cache exists.  Per request b and query
 * head i (kv head j = i / (Hq/Hkv)), the K block queries attend, with no mask
 * inside the block, to the ctx_lens[b] context tokens read through the page
 * table plus the K block keys:
 *
 *   keys   = Kc[page_table[b][n/P], n%P, j] (n < ctx_lens[b])  ++  k_blk[b, :, j]
 *   out[b, :, i] = softmax(scale * q[b, :, i] @ keys^T) @ values
 *
 * block_causal = 1 selects the block-causal variant instead (the pages fix
 * no mask; this is the masked alternative, with the mask applied only among
 * the block keys): block query t then sees every context key and the block
 * keys s <= t.  0 is the mask-free form above; any other value is INVALID.
 *
 *   q            act [C, K, Hq, D]
 *   k_blk, v_blk act [C, K, Hkv, D]   the block's own keys / values (transient)
 *   k_cache,     act pools, read only; element (page, slot, j, d) sits at
 *   v_cache          page*page_stride + slot*token_stride + j*head_stride + d
 *                    (strides in elements, multiples of 8; d contiguous;
 *                    P = page_size slots per page).  NHD [pages,P,Hkv,D] and
 *                    HND [pages,Hkv,P,D] pools are both just strides.
 *   num_pages    pages in each pool (entries must lie in [0, num_pages))
 *   page_size    tokens per page P: 16, 32, 64, 128 or 256 (else UNSUPPORTED)
 *   page_table   int32 [C, max_pages] device; row b lists request b's pages
 *                in context order; entries past ceil(ctx_lens[b]/P) are unused
 *   ctx_lens     int32 [C] device; 0 <= ctx_lens[b] <= max_ctx
 *   max_ctx      host upper bound of ctx_lens (sizes the grid and workspace);
 *                max_pages >= ceil(max_ctx/P)
 *   kv_split_pages  0 = automatic work ranges (below); otherwise ranges of
 *                this many pages of P tokens each (the last one shorter).
 *                Results do not depend on it beyond rounding (fp32
 *                accumulation, and each piece's output rounded to the
 *                activation dtype before the merge), and are bitwise
 *                repeatable for a fixed value
 *   scale        softmax scale; 0.f means 1/sqrt(D)
 *   out          act [C, K, Hq, D]
 *   workspace / workspace_bytes:
 *       workspace == NULL: size query -- *workspace_bytes receives the bytes
 *       this call needs; nothing is launched.  Otherwise *workspace_bytes is
 *       the capacity of `workspace` (device, 256-byte aligned), which must be
 *       at least the queried size.
 * Work plan.  Request b's keys are its ceil(ctx_b/16) context slabs of 16
 * tokens followed by its ceil(K/16) block slabs, counted in granules of
 * g = max(2, P/16) slabs from the request's start (G_b granules).
 * Automatic ranges charge each request a fixed cost of s = ceil(12/g)
 * units, ceil(24/g) with more than 64 query rows per kv head ((Hq/Hkv)*K),
 * placed before its keys (s = 0 with kv_split_pages), so request b
 * spans s + G_b units, request after request, and its keys start at unit
 * S_b; the batch's T = sum (s + G_b) units are cut into W ranges
 * [B_w, B_{w+1}): automatically W = min(w_max, max(1, floor(T /
 * ceil(16/g)))) ranges of nearly equal cost, B_w = floor(w*T/W);
 * with kv_split_pages, ranges of R = ceil(kv_split_pages*(P/16)/g)
 * granules, B_w = min(w*R, T).  One workgroup per (range, kv head group)
 * takes its range's slabs request by request; a request inside one range is
 * finished there, a request spanning several ranges (its pieces) is merged
 * by log-sum-exp.  w_max, a bound the host derives from C, max_ctx, K, Hkv
 * and the page size, sizes the grid and the workspace: automatically
 * min(512/Hkv, max(1, floor(C*(s + Gmax) / ceil(16/g)))), Gmax the granules
 * of a max_ctx request; with kv_split_pages, ceil(C*Gmax / R).  The workspace
 * starts with the int32 plan the kernels derive from ctx_lens:
 *         [0] W  [1] g  [2] C  [3] w_max
 *         [4, 4+C) S_b    [4+C, 4+2C) range of request b's first key granule
 *         [4+2C, 4+3C) ranges request b spans (its pieces)
 *         [4+3C, 4+3C+w_max+1) B_0 .. B_W (B_W = T), then -1
 *       followed, when w_max > 1, by the partials of two slots per range:
 *       each piece's output divided by its own softmax sum, in the activation
 *       dtype, and its fp32 (max, sum).
 * Limits: D in {64, 128}; 1 <= K <= 64; Hq % Hkv == 0; (Hq/Hkv)*K <= 256;
 * token_stride times the element size <= 2^27 bytes; the batch's keys at
 * their bound, C * g * ceil((ceil(max_ctx/16) + ceil(K/16)) / g) slabs,
 * below 2^31 (else UNSUPPORTED).
 */
int hspec_block_attn_inplace(void* stream, int dtype, int C, int K, int Hq, int Hkv, int D,
                             const void* q, const void* k_blk, const void* v_blk,
                             const void* k_cache, const void* v_cache,
                             int64_t page_stride, int64_t token_stride, int64_t head_stride,
                             int num_pages, int page_size, const int32_t* page_table, int max_pages,
                             const int32_t* ctx_lens, int max_ctx,
                             int kv_split_pages, float scale, int block_causal, void* out,
                             void* workspace, size_t* workspace_bytes);

/*
 * a5 -- the whole drafter layer: a1 -> a2 (Mamba half) and a0 -> a3 -> a4
 * (attention half) on one stream, with the arguments of the calls above.
 * H-Spec, Abstract: the two kinds of target context (last-token hidden
 * state, in-place target KV) enter through the two complementary modules.
 * `h0` is written by a1 and read by a2; `h_final` and `Dskip` may be NULL.
 * `u` and `w_init` both NULL select the direct-reuse-only ablation (H-Spec,
 * Section 3.1 / Figure 4 and the source ablation of Figure 7a: target KV
 * reused in place with no hidden-state initialisation): a1 is skipped,
 * a2 starts from the zero state and `h0` is neither read nor written (it may
 * be NULL).  Exactly one of them NULL is INVALID_ARG.
 * `workspace` == NULL is a size query exactly as for a3.
 */
typedef struct hspec_layer_args {
  int dtype;
  int C, K;
  /* Mamba half */
  int d_model, H, P, ng, N, chunk;
  const void* u; const void* w_init; float* h0;
  const void* x; const float* delta; const float* A; const void* B; const void* Cm;
  const float* Dskip; float* y; float* h_final;
  /* attention half */
  int Hq, Hkv, D;
  const void* q; const void* k_blk; const void* v_blk;
  const void* k_cache; const void* v_cache;
  int64_t page_stride, token_stride, head_stride;
  int num_pages; int page_size; const int32_t* page_table; int max_pages;
  const int32_t* ctx_lens; int max_ctx;
  int kv_split_pages; float scale; int block_causal; void* out;
  void* workspace; size_t workspace_bytes;
} hspec_layer_args;

/* sizeof(hspec_layer_args) as compiled into the library (binding check). */
size_t hspec_layer_args_size(void);

/* `required_bytes` receives the workspace size a5 needs (may be NULL when
 * a->workspace is set). */
int hspec_draft_layer(void* stream, const hspec_layer_args* a, size_t* required_bytes);

/*
 * a5 for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels as hspec_draft_layer, but its workspace (the split plan and the
 * attention's split partials) is a static device array of the library,
 * HSPEC_NOALLOC_SCRATCH_BYTES long, instead of a caller's buffer.
 *   a->workspace must be NULL and a->workspace_bytes 0 (else INVALID_ARG).
 *   A call whose workspace (the size hspec_draft_layer would report) exceeds
 *   HSPEC_NOALLOC_SCRATCH_BYTES returns HSPEC_ERR_SCRATCH and launches
 *   nothing.
 * The array exists once per GPU (on the calling thread's current device,
 * which must be the stream's device) and is held until the process ends; its
 * address is looked up on the first call on each device.  Nothing is
 * allocated and nothing needs clearing: every byte a call reads from it was
 * written earlier in the same call.  All calls on one GPU share the array,
 * so calls that overlap in time on one GPU (concurrent streams, or two
 * threads) race: serialise them.
 */
#define HSPEC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int hspec_draft_layer_noalloc(void* stream, const hspec_layer_args* a);

/* Executable HIP graph of a layer or a stack (see hspec_draft_stack_graph). */
typedef struct hspec_graph_s* hspec_graph;

/* a5 captured once into a HIP graph (its kernels in the order of
 * hspec_draft_layer), for callers that replay graphs; bound to the buffers
 * and workspace in `a` (contents may change between launches).  Creating it
 * launches nothing and allocates no device memory. */
int hspec_draft_layer_graph(const hspec_layer_args* a, hspec_graph* out);

/*
 * The Mamba-2 block around a2: input projection, short causal convolution,
 * the scan, gated RMS normalisation and output projection.  H-Spec, Abstract:
 * the drafter's Mamba modules are Mamba-2 modules; the block is Mamba-2's
 * (Dao & Gu 2024, "Transformers are SSMs"), which the pages do not print.
 * Per request b and block position t (token row r = b*K + t):
 *
 *   zxbcdt[r] = w_in . hidden[r]                 rows z | x | B | C | dt
 *   xBC[r, c] = SiLU(conv_b[c] + sum_j conv_w[c, j] * xBC_raw[r - 3 + j, c])
 *               (positions before the block start are zero)
 *   delta[r, h] = softplus(dt_raw[r, h] + dt_bias[h])
 *   y = a2 scan of (x, delta, A, B, C) from h0, with the skip term Dskip
 *   normed[r] = g / sqrt(mean(g^2) + eps) * norm_w,   g = y[r] * SiLU(z[r])
 *   out[r] = w_out . normed[r]
 *
 * Shapes (d_inner = H*P, conv_dim = d_inner + 2*ng*N,
 * d_proj = 2*d_inner + 2*ng*N + H):
 *   hidden  act  [C, K, d_model]
 *   w_in    act  [d_proj, d_model]    ([out, in], rows z | x | B | C | dt)
 *   conv_w  fp32 [conv_dim, 4]        tap 3 multiplies the current token
 *   conv_b  fp32 [conv_dim] or NULL
 *   dt_bias fp32 [H];  A fp32 [H] (negative);  Dskip fp32 [H] or NULL
 *   h0      fp32 [C, H, P, N] or NULL (zero state)
 *   norm_w  fp32 [d_inner];  norm_eps >= 0
 *   w_out   act  [d_model, d_inner]
 *   out     act  [C, K, d_model]
 *   h_final fp32 [C, H, P, N] or NULL
 * x channel h*P + p is head h, element p; B and C channel g*N + n is group g.
 * Projections run on bf16 matrix cores with fp32 accumulation (fp32 FMA for
 * fp32 activations); the convolution, scan and norm run in fp32 and the
 * normalised activations are rounded to the activation type before the
 * output projection.  `workspace` == NULL is a size query as for a3
 * (256-byte aligned device memory otherwise).
 * Limits: d_model % 8 == 0, d_inner % 8 == 0, the scan limits of a2 with
 * chunk <= 16 (the convolution runs inside the scan's 16-position staging),
 * C*K <= 2^30 and C*K * max(d_in_proj, d_model) <= 2^40 (else UNSUPPORTED);
 * hidden, w_in, w_out, out, conv_w and norm_w 16-byte aligned (else
 * INVALID_ARG).
 */
typedef struct hspec_mamba_args {
  int dtype;
  int C, K, d_model, H, P, ng, N, chunk;
  const void* hidden; const void* w_in;
  const float* conv_w; const float* conv_b; const float* dt_bias;
  const float* A; const float* Dskip; const float* h0;
  const float* norm_w; float norm_eps;
  const void* w_out;
  void* out; float* h_final;
  void* workspace; size_t workspace_bytes;
} hspec_mamba_args;

/* sizeof(hspec_mamba_args) as compiled into the library (binding check). */
size_t hspec_mamba_args_size(void);

/* `required_bytes` receives the workspace size (may be NULL when
 * a->workspace is set). */
int hspec_mamba_block(void* stream, const hspec_mamba_args* a, size_t* required_bytes);

/*
 * Contrast workload, not part of H-Spec's path: the drafter-side KV
 * injection of the parallel drafters H-Spec is compared with (H-Spec,
 * Abstract, Table 1 and Figure 3: a projection of the target hidden state at
 * every new position into a drafter KV cache; H-Spec never runs this step).
 * Per request b and new position i < n_new, token position
 * p = start_pos[b] + i:
 *
 *   kv = w_kv . hidden[b, i]                    (w_kv: K rows, then V rows)
 *   k_cache[page_table[b][p/P], p%P, h, :] = kv[h*D .. h*D + D)
 *   v_cache[page_table[b][p/P], p%P, h, :] = kv[Hkv*D + h*D .. Hkv*D + h*D + D)
 *
 * written in the activation type; nothing else in the pools changes.
 *   hidden      act [C, n_new, d_model]
 *   w_kv        act [2*Hkv*D, d_model]       ([out, in])
 *   k_cache,    act pools written in place, strides in elements and the page
 *   v_cache         size P as for hspec_block_attn_inplace
 *   page_table  int32 [C, max_pages] device;  start_pos int32 [C] device
 * A position whose page-table slot lies past max_pages, or whose entry lies
 * outside [0, num_pages), is skipped (never a stray write).  Requests must
 * own distinct pages: writes to one slot from two requests race.
 * Runs on bf16 matrix cores (fp32 FMA for fp32), fp32 accumulation.
 * `workspace` == NULL is a size query as for a3 (split-K partials).
 * Limits: d_model % 8 == 0, C*n_new <= 2^30, Hkv*D <= 2^28 and
 * C*n_new * 2*Hkv*D <= 2^40 (else UNSUPPORTED); hidden, w_kv 16-byte aligned.
 */
int hspec_kv_inject(void* stream, int dtype, int C, int n_new, int d_model, int Hkv, int D,
                    const void* hidden, const void* w_kv, void* k_cache, void* v_cache,
                    int64_t page_stride, int64_t token_stride, int64_t head_stride, int num_pages,
                    int page_size, const int32_t* page_table, int max_pages, const int32_t* start_pos,
                    void* workspace, size_t* workspace_bytes);

/*
 * A drafter stack of hybrid layers over the draft block, eager on one stream
 * or captured once into a HIP graph.  H-Spec, Abstract (a backbone of Mamba-2
 * and attention modules) and the runtime analysis of Figure 8 (the deeper
 * stack is slower at low concurrency); the pages print no stack, and the
 * wiring is this reading, with fp32 residual stream h:
 *
 *   h = hidden_in
 *   for each layer l:
 *     x  = RMSNorm(h) * pre_norm_w[l]                       (eps)
 *     ym = Mamba-2 block of x (as hspec_mamba_block) from h0 = u . w_init[l]
 *                                                 (a1; layers with w_in set)
 *     ya = (block attention of x.wq^T, x.wk^T, x.wv^T over the layer's
 *           target KV pools, read in place, as hspec_block_attn_inplace) . wo^T
 *                                                 (layers with wq set)
 *     h  = h + ym + ya
 *   hidden_out = h
 *
 * A layer may hold either half or both; all layers share the page table,
 * context lengths and shapes.  Weights are [out, in] in the activation type
 * except w_init [d_model, S] (as a1).  Intermediate activations are rounded
 * to the activation type.  No RoPE, biases or MLP.
 *   hidden_in  act [C, K, d_model];  u act [C, d_model] (last-token target hidden)
 *   hidden_out fp32 [C, K, d_model]
 *   layers     host array [n_layers]; the pointers inside are device memory
 *   workspace  as for a3: NULL = size query into *required_bytes
 * Limits: those of a1 (d_model % 32, S % 64), of the Mamba-2 block and of
 * a3; d_model % 8 == 0; C*K * max(Hq*D, d_model) <= 2^40; pre_norm_w 16-byte
 * aligned.
 */
typedef struct hspec_stack_layer {
  const float* pre_norm_w;      /* [d_model] */
  /* Mamba half (w_in NULL: none) */
  const void* w_init; const void* w_in;
  const float* conv_w; const float* conv_b; const float* dt_bias;
  const float* A; const float* Dskip; const float* norm_w; const void* w_out;
  /* attention half (wq NULL: none) */
  const void* wq; const void* wk; const void* wv; const void* wo;
  const void* k_cache; const void* v_cache;
} hspec_stack_layer;

typedef struct hspec_stack_args {
  int dtype;
  int C, K, d_model, n_layers;
  int H, P, ng, N, chunk;
  float eps;
  int Hq, Hkv, D;
  int64_t page_stride, token_stride, head_stride;
  int num_pages; int page_size; const int32_t* page_table; int max_pages;
  const int32_t* ctx_lens; int max_ctx; int kv_split_pages; float scale;
  const void* hidden_in; const void* u; float* hidden_out;
  const hspec_stack_layer* layers;
  void* workspace; size_t workspace_bytes;
} hspec_stack_args;

size_t hspec_stack_args_size(void);

/* Eager: every kernel of the stack on `stream`, in layer order. */
int hspec_draft_stack(void* stream, const hspec_stack_args* a, size_t* required_bytes);

/* Graph form: captures the stack once (the state projections and Mamba
 * halves on a forked branch, concurrent with the attention halves) into an
 * executable HIP graph bound to the buffers and the workspace in `a`
 * (which must stay allocated; their contents may change between launches).
 * Creating it launches nothing and allocates no device memory. */
int hspec_draft_stack_graph(const hspec_stack_args* a, hspec_graph* out);
int hspec_graph_launch(hspec_graph g, void* stream);
int hspec_graph_destroy(hspec_graph g);

#ifdef __cplusplus
}
#endif
#endif /* HSPEC_H */
