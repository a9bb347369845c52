/*
 * ea.h - C ABI of the MI355X (gfx950) head-routed hybrid attention prefill.
 *
 * The method is Elastic Attention's inference path ("Elastic Attention:
 * Test-time Adaptive Sparsity Ratios for Efficient Transformers"; summarised
 * in "Technical Summary: Elastic Attention"):
 *
 *   1. an attention router pools the Key states of each KV head over the first
 *      and last 100 tokens, runs a task MLP and a router MLP to logits
 *      z in R^{H x 2}, and takes the argmax as a hard per-head decision,
 *      0 = full attention (FA), 1 = sparse attention (SA)
 *      (paper body: router paragraphs on Fig. 3(b) and Fig. 3(c), boundary
 *      pooling in the implementation details; summary Sec. 2.1);
 *   2. one fused GQA attention forward then serves every head in a single
 *      pass, FA heads attending causally to all keys and SA heads to a
 *      retained subset of K/V, with the head outputs concatenated along the
 *      feature axis (paper body: FA and SA equations of the preliminaries,
 *      hybrid-head output equation and its GQA footnote; summary Sec. 2.3).
 *
 * The sparse subset is static: n_sink attention-sink blocks plus a causal
 * local window of w key blocks, in blocks of 64 tokens, with
 * w = max(n_sink + 1, floor(rho * N + 1/2)) - n_sink for N = ceil(L / 64)
 * key blocks (rho = keep_fraction) unless window_blocks > 0 gives w directly.
 * Query i (sequence-local) sees key j iff j <= i and (mode == FA or
 * j / 64 < n_sink or i / 64 - j / 64 < w).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no device memory and keeps no state between calls.
 *  - Tensors are dense and row-major with the last axis innermost; sequences
 *    are packed back to back ("varlen"), delimited by cu_seqlens (int32,
 *    [B + 1], cu_seqlens[0] = 0, non-decreasing).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise the host.
 *  - Host-checkable errors return a negative status before anything is
 *    launched; ea_last_error() then returns a message (thread-local).  A
 *    failed launch returns EA_ERR_HIP.
 *  - Device contents are checked on the device by the planner that every
 *    prefill, dual, XA and backward call runs first: cu_seqlens[0] == 0,
 *    cu_seqlens non-decreasing, cu_seqlens[B] == total_tokens, every length
 *    <= max_seqlen, and every mode 0 or 1 (the router paragraph on Fig. 3(b)
 *    of the paper body: the hard decision per KV head is 0 or 1).  On a
 *    failed check the planner marks its workspace invalid and no later kernel
 *    of the call reads Q, K, V or writes an output (the outputs keep their
 *    previous contents).  By default nothing waits for the verdict:
 *    ea_workspace_status() reads it.  With the environment variable
 *    EA_VALIDATE set (to anything but "" or "0"), every such call waits for
 *    the checks itself and returns EA_ERR_INVALID_ARG with a message naming
 *    the failed check; ea_route and ea_kvcache_prefill then also copy
 *    cu_seqlens to the host and check it there.
 *  - n_sink_blocks and window_blocks are at most 2^24 (EA_ERR_INVALID_ARG).
 */
#ifndef EA_H
#define EA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EA_ABI_VERSION 2

typedef enum {
  EA_OK = 0,
  EA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad value */
  EA_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, dtype, block size */
  EA_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  EA_ERR_HIP = -4          /* a HIP launch failed; message has the HIP error */
} ea_status;

typedef enum {
  EA_F32 = 0,  /* float32 */
  EA_BF16 = 1  /* bfloat16 (arithmetic: bf16 MFMA operands, fp32 accumulate) */
} ea_dtype;

/* Router parameters: float32 device arrays in nn.Linear layout [out, in].
 *   task MLP:   t = W2 GELU(W1 x' + b1) + b2      W1 [task_hidden, head_dim],
 *                                                  W2 [head_dim, task_hidden]
 *   router MLP: z = W4 GELU(W3 t + b3) + b4       W3 [router_hidden, head_dim],
 *                                                  W4 [2, router_hidden]
 * GELU is the exact erf form.  One router is shared by all KV heads.
 * Limits: 1 <= head_dim <= 256, 1 <= task_hidden <= 4096,
 * 1 <= router_hidden <= 1024, pool_len >= 1 (the pages use 100). */
typedef struct {
  int32_t head_dim;
  int32_t task_hidden;
  int32_t router_hidden;
  int32_t pool_len;
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  const float* w3;
  const float* b3;
  const float* w4;
  const float* b4;
} ea_router_desc;

/* Sparse-attention geometry and softmax scale.
 *   block          must be 64
 *   n_sink_blocks  >= 0 attention-sink blocks kept by SA heads
 *   window_blocks  > 0: local window of that many blocks; 0: derive it from
 *                  keep_fraction per sequence (formula above, evaluated in
 *                  double on the float32 value)
 *   keep_fraction  in (0, 1]; read only when window_blocks == 0
 *   softmax_scale  > 0, or 0 for 1/sqrt(head_dim) */
typedef struct {
  int32_t block;
  int32_t n_sink_blocks;
  int32_t window_blocks;
  float keep_fraction;
  float softmax_scale;
} ea_sparsity_params;

/* ABI version of the loaded library (EA_ABI_VERSION it was built with). */
int32_t ea_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ea_last_error(void);

/* ea_workspace_status - verdict of the planner's device-content checks.
 *
 *   workspace        a workspace that a prefill, plan, dual, XA or backward
 *                    call has planned (its header is read; the rest is not)
 *   workspace_bytes  its size, at least 256
 *   stream           the stream the planning call ran on
 *
 * Waits for `stream`, then returns EA_OK if the last plan written into the
 * workspace passed every check listed in the conventions above, or
 * EA_ERR_INVALID_ARG with a message naming the failed checks.  A workspace
 * no call has planned holds no verdict (its result is meaningless). */
ea_status ea_workspace_status(const void* workspace, size_t workspace_bytes, void* stream);

/* ea_route - hard FA/SA decision per (sequence, KV head).
 *
 *   K           [T, Hkv, head_dim] of `dtype` (16-byte aligned); only the
 *               boundary rows of each sequence are read
 *   cu_seqlens  int32 [B + 1]
 *   router      parameters (struct on the host, arrays on the device)
 *   modes       out int8 [B, Hkv]: 0 = FA, 1 = SA; argmax of z with ties to FA
 *   logits      out float32 [B, Hkv, 2], or NULL
 *
 * Pooling is the mean over the union of a sequence's first and last pool_len
 * rows (a row in both counts once), accumulated in float32.  An empty
 * sequence gets mode 0 and logits (0, 0). */
ea_status ea_route(const void* K, ea_dtype dtype, const int32_t* cu_seqlens, int32_t B,
                   int32_t Hkv, const ea_router_desc* router, int8_t* modes, float* logits,
                   void* stream);

/* Bytes of device workspace ea_hybrid_prefill needs for these sizes (0 if the
 * sizes are invalid).  The workspace holds the per-launch work list and its
 * sort buffers (a few bytes per query tile); its contents need not be
 * initialised. */
size_t ea_hybrid_prefill_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                        int32_t Hq, int32_t Hkv, int32_t head_dim,
                                        ea_dtype dtype);

/* ea_hybrid_prefill_noalloc - ea_hybrid_prefill for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and results without
 * the workspace, which is instead a static array of
 * ea_hybrid_prefill_noalloc_max_workspace() bytes (4 MiB) inside the library,
 * one per GPU, held until the process ends.  The call allocates nothing.
 *
 * Sizes whose workspace (ea_hybrid_prefill_workspace_size) exceeds that
 * array return EA_ERR_WORKSPACE before anything is launched; 4 MiB covers,
 * with 8 KV heads and 4 query heads per KV head, about 1.2 million tokens.
 * Every call on a GPU uses that GPU's one array, so calls that overlap on
 * one GPU (concurrent streams, threads) race and must be ordered by the
 * caller.  Nothing in the array needs to start at any value: each call
 * writes what it reads.  EA_VALIDATE does not make this call wait (it never
 * synchronises); ea_workspace_status cannot see its workspace. */
size_t ea_hybrid_prefill_noalloc_max_workspace(void);
ea_status ea_hybrid_prefill_noalloc(const void* Q, const void* K, const void* V, ea_dtype dtype,
                                    const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                                    int64_t total_tokens, int32_t max_seqlen, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, const ea_sparsity_params* p,
                                    void* O, float* lse, void* stream);

/* ea_hybrid_prefill_plan_layout - where ea_hybrid_prefill_plan (and the
 * one-shot call) put the work list inside a workspace of these sizes, for
 * inspection.  Byte offsets of: the item records (n_slots records of five
 * int32: sequence, KV head, query tile, cost in visible 64-key blocks,
 * computation mode), their uint32 sort keys (0 = costliest band of 32 key
 * blocks), and the int32 list order (record indices, ascending key, equal
 * keys in record order).  The first tiles * Hkv slots are real items, tiles =
 * int32 word 0 of the workspace; the rest are empty and sort last.  The
 * layout is a pure function of the sizes (EA_OK, or EA_ERR_INVALID_ARG /
 * EA_ERR_UNSUPPORTED for sizes the workspace query rejects). */
ea_status ea_hybrid_prefill_plan_layout(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                        int32_t Hq, int32_t Hkv, int32_t head_dim, ea_dtype dtype,
                                        int64_t* items_offset, int64_t* keys_offset,
                                        int64_t* order_offset, int64_t* n_slots);

/* ea_hybrid_prefill - fused hybrid GQA attention forward over all heads.
 *
 *   Q           [T, Hq, head_dim]  of `dtype` (16-byte aligned)
 *   K, V        [T, Hkv, head_dim] of `dtype` (16-byte aligned)
 *   modes       int8 [B, Hkv], values 0 (FA) or 1 (SA); query head hq uses
 *               KV head hq / (Hq / Hkv) and its mode
 *   cu_seqlens  int32 [B + 1]; total_tokens = cu_seqlens[B] = T < 2^31
 *   max_seqlen  >= every sequence length (>= 1 when T > 0)
 *   params      sparse geometry and scale (host struct)
 *   O           out [T, Hq, head_dim] of `dtype`, written in place: no
 *               per-mode gather or scatter
 *   lse         out float32 [Hq, T] natural-log sum of exp of the scaled
 *               visible scores, or NULL
 *   workspace   device buffer of >= ea_hybrid_prefill_workspace_size() bytes
 *               (256-byte aligned); not shared between concurrent calls
 *
 * head_dim must be 64 or 128; Hq must be a multiple of Hkv with
 * Hq / Hkv <= 256; max_seqlen * Hq * head_dim must be < 2^31 (one
 * sequence's rows are addressed with 32-bit byte offsets: 512K tokens at
 * Hq = 32, d = 128).  Each output row is written by exactly one workgroup with
 * no atomics on O, so results are bitwise reproducible. */
ea_status ea_hybrid_prefill(const void* Q, const void* K, const void* V, ea_dtype dtype,
                            const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                            int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                            int32_t head_dim, const ea_sparsity_params* params, void* O,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ea_hybrid_prefill_plan / ea_hybrid_prefill_run - the two halves of
 * ea_hybrid_prefill, for callers that time or reuse them separately.
 *
 * plan builds the cost-ordered work list of (sequence, KV-head group, query
 * tile) items into `workspace`: each item's cost is its number of visible
 * 64-key blocks (all causal blocks for an FA head, sink blocks plus the local
 * window for an SA head), and the list runs most expensive first, so FA and SA
 * tiles load-balance in the single fused launch (summary Sec. 2.3: one pass
 * over all routed heads, no splitting or recombining of tensors).  It reads
 * only modes and cu_seqlens.
 *
 * run launches the fused attention forward over a workspace that plan filled
 * with the same modes, cu_seqlens, sizes and params, on the same stream or
 * after it; the list is not modified, so one plan serves any number of runs
 * over different Q, K, V with that routing.  Arguments, errors and outputs are
 * those of ea_hybrid_prefill; a workspace that was not planned for these
 * arguments is a precondition violation (not detected). */
ea_status ea_hybrid_prefill_plan(const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                                 int64_t total_tokens, int32_t max_seqlen, int32_t Hq,
                                 int32_t Hkv, int32_t head_dim, ea_dtype dtype,
                                 const ea_sparsity_params* params, void* workspace,
                                 size_t workspace_bytes, void* stream);

ea_status ea_hybrid_prefill_run(const void* Q, const void* K, const void* V, ea_dtype dtype,
                                const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                                int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                                int32_t head_dim, const ea_sparsity_params* params, void* O,
                                float* lse, const void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- Training forward ------------------------------------------------------
 *
 * During router training the pages feed the logits z through a Gumbel-Softmax
 * with an annealed temperature and make hard decisions with a straight-through
 * estimator: the forward pass uses r_hard = argmax r_soft while gradients flow
 * through r_soft (paper body: Gumbel-Softmax and STE paragraphs of the method
 * section; summary Sec. 2.2).  A head's output is r[0] O_FA + r[1] O_SA with
 * r = r_hard - sg(r_soft) + r_soft, so the training forward computes every
 * head in both modes. */

/* ea_gumbel_route - r_soft and hard modes from routing logits.
 *
 *   logits  float32 [n, 2] device array (z of ea_route, rows (b, g) flattened)
 *   gumbel  float32 [n, 2] standard Gumbel noise, or NULL for none
 *   tau     temperature, finite and > 0
 *   r_soft  out float32 [n, 2]: softmax((z + g) / tau) over the two modes, or NULL
 *   modes   out int8 [n]: 1 (SA) iff (z1 + g1) / tau > (z0 + g0) / tau, taken in
 *           float32 (a tie goes to FA)
 * n >= 0.  Asynchronous on `stream`. */
ea_status ea_gumbel_route(const float* logits, const float* gumbel, float tau, int32_t n,
                          float* r_soft, int8_t* modes, void* stream);

/* Bytes of device workspace ea_dual_prefill needs (0 if the sizes are invalid):
 * the work list of ea_hybrid_prefill with two entries per query tile. */
size_t ea_dual_prefill_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                      int32_t Hq, int32_t Hkv, int32_t head_dim,
                                      ea_dtype dtype);

/* ea_dual_prefill - dual-mode attention forward: every query head in both
 * modes in one launch, then the straight-through mix.
 *
 *   Q, K, V, cu_seqlens, sizes, params: as for ea_hybrid_prefill
 *   O_fa, O_sa  out [T, Hq, head_dim] of `dtype`: each head's FA and SA output
 *   lse_fa, lse_sa  out float32 [Hq, T]: their natural-log sums of exponentials
 *   O       out [T, Hq, head_dim] of `dtype`, the forward value of the mix:
 *           O_sa where modes[b, hq / (Hq / Hkv)] == 1, else O_fa; or NULL
 *   modes   int8 [B, Hkv] hard decisions (e.g. from ea_gumbel_route); read
 *           only when O is not NULL
 *
 * Every causal key block of a head is visited once: the SA set (sinks and
 * window) gives O_SA and LSE_SA, the remaining blocks a partial that a merge
 * pass combines with them into O_FA and LSE_FA (attention over disjoint key
 * sets combines by their LSE weights), so the matrix work equals that of an
 * FA-only forward.  The outputs must not alias; limits and errors are those of
 * ea_hybrid_prefill. */
ea_status ea_dual_prefill(const void* Q, const void* K, const void* V, ea_dtype dtype,
                          const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                          int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                          int32_t head_dim, const ea_sparsity_params* params, void* O,
                          void* O_fa, void* O_sa, float* lse_fa, float* lse_sa, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ea_router_logit_grad - gradient of the loss with respect to the routing
 * logits through the straight-through estimator and the Gumbel-Softmax
 * (paper body: STE paragraph; summary Sec. 2.2).  With O = r[0] O_fa +
 * r[1] O_sa per (sequence b, KV head g) and r = r_hard - sg(r_soft) + r_soft:
 *   dr[b, g, m] = sum over b's tokens and g's query heads of <dO, O_m>,
 *   dz = r_soft * (dr - <dr, r_soft>) / tau.
 *
 *   dO, O_fa, O_sa  [T, Hq, head_dim] of `dtype` (O_fa, O_sa from ea_dual_prefill)
 *   r_soft          float32 [B, Hkv, 2] (from ea_gumbel_route), tau as there
 *   dz              out float32 [B, Hkv, 2]; dr out float32 [B, Hkv, 2] or NULL
 *   workspace       >= ea_router_logit_grad_workspace_size() bytes
 * Sums run in a fixed order (no atomics): bitwise reproducible. */
size_t ea_router_logit_grad_workspace_size(int32_t B, int32_t max_seqlen, int32_t Hkv);
ea_status ea_router_logit_grad(const void* dO, const void* O_fa, const void* O_sa, ea_dtype dtype,
                               const int32_t* cu_seqlens, int32_t B, int64_t total_tokens,
                               int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t head_dim,
                               const float* r_soft, float tau, float* dz, float* dr,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace ea_hybrid_backward needs (0 if the sizes are
 * invalid): the forward's work list plus two float32 [Hq, T] arrays. */
size_t ea_hybrid_backward_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                         int32_t Hq, int32_t Hkv, int32_t head_dim,
                                         ea_dtype dtype);

/* ea_hybrid_backward - gradients of the hybrid layer for an upstream dO.
 *
 * The router is trained behind a frozen backbone in every layer (paper body:
 * training paragraphs), so a layer's backward must carry gradients through
 * its routed attention: with P = softmax(scale Q K^T) over each head's
 * visible keys and O = P V,
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV of a KV head summed over its query heads.
 *
 *   Q, K, V, modes, cu_seqlens, sizes, params: as for ea_hybrid_prefill
 *   O, lse     the forward's outputs for these inputs (lse required)
 *   dO         [T, Hq, head_dim] upstream gradient
 *   dQ         out [T, Hq, head_dim]; dK, dV out [T, Hkv, head_dim]
 * bf16 only (float32 accumulation); every output row is written once, by one
 * workgroup, with no atomics (bitwise reproducible).  Other limits and errors
 * are those of ea_hybrid_prefill. */
ea_status ea_hybrid_backward(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* lse, ea_dtype dtype,
                             const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                             int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                             int32_t head_dim, const ea_sparsity_params* params, void* dQ,
                             void* dK, void* dV, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ---- Decode with a mode-aware KV cache -------------------------------------
 *
 * One new token per sequence attends to its cached keys with the prefill's
 * visibility rule for a query at the last position of a sequence one token
 * longer (paper body: FA and SA equations, hybrid-head output equation).  An
 * FA head's cache slot holds every block; an SA head's holds its sink blocks
 * and a ring of R blocks, R = the window at max_len (the window never moves
 * back, so a block that leaves it is never needed again): at keep_fraction
 * 0.2 an SA slot is about a fifth of an FA slot.  Blocks are 64 tokens; the
 * cache is bfloat16; one sequence's slots follow its routing modes, fixed
 * when the cache is initialised. */
typedef struct {
  int32_t B;              /* sequences */
  int32_t Hkv;            /* KV heads */
  int32_t head_dim;       /* 64 or 128 */
  int32_t max_len;        /* tokens a sequence may reach, 1 .. 2^21 */
  int32_t n_sink_blocks;  /* as in ea_sparsity_params */
  int32_t window_blocks;  /* > 0: fixed window; 0: from keep_fraction per length */
  float keep_fraction;    /* in (0, 1], read when window_blocks == 0 */
} ea_kvcache_desc;

/* Bytes of a cache for `desc` with the routing `modes_host` (int8 [B, Hkv] in
 * HOST memory, 0 = FA, 1 = SA); 0 if desc is invalid. */
size_t ea_kvcache_bytes(const ea_kvcache_desc* desc, const int8_t* modes_host);

/* ea_kvcache_init - lay out an empty cache in `cache` (device buffer of
 * `bytes`, 256-byte aligned) for the routing `modes` (int8 [B, Hkv] DEVICE
 * memory, the same values ea_kvcache_bytes was given): slot table, zeroed
 * blocks, lengths 0.  A buffer smaller than the layout needs leaves the cache
 * marked unusable (later calls then write nothing and decode outputs zeros). */
ea_status ea_kvcache_init(const ea_kvcache_desc* desc, const int8_t* modes, void* cache,
                          size_t bytes, void* stream);

/* ea_kvcache_prefill - store a packed prompt batch (K, V [T, Hkv, head_dim]
 * bf16, cu_seqlens int32 [B + 1], T = total_tokens) into the cache: every row
 * an FA head or a later SA query can see; lengths[b] = L_b.  L_b <= max_len
 * is a precondition (a longer sequence's slots are left untouched). */
ea_status ea_kvcache_prefill(const ea_kvcache_desc* desc, void* cache, size_t bytes,
                             const void* K, const void* V, const int32_t* cu_seqlens,
                             int64_t total_tokens, void* stream);

/* Bytes of device workspace ea_decode_step needs (chunk partials of the split
 * over the cache); 0 if the sizes are invalid. */
size_t ea_decode_workspace_size(const ea_kvcache_desc* desc, int32_t Hq);

/* ea_decode_step - append one token per sequence and attend with it.
 *
 *   q             [B, Hq, head_dim] bf16: the new token's queries
 *   k_new, v_new  [B, Hkv, head_dim] bf16: its keys and values, stored at
 *                 position lengths[b] before the attention
 *   softmax_scale > 0, or 0 for 1/sqrt(head_dim)
 *   O             out [B, Hq, head_dim] bf16
 *   lse           out float32 [B, Hq] natural-log sums of exponentials, or NULL
 * Then lengths[b] += 1.  Hq must be a multiple of Hkv with Hq / Hkv <= 16;
 * lengths[b] < max_len is a precondition (a full sequence gets O = 0 and
 * keeps its length). */
ea_status ea_decode_step(const ea_kvcache_desc* desc, void* cache, size_t bytes, const void* q,
                         const void* k_new, const void* v_new, int32_t Hq, float softmax_scale,
                         void* O, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- XAttention head mode -------------------------------------------------
 *
 * The pages also run heads in XAttention (XA) mode: a head configuration
 * "{retrieval-head mode}-{sparse-head mode}" maps the router's decision 0
 * (retrieval head) and 1 (sparse head) to computation modes, FA-SSA being the
 * routed prefill above, FA-XA and XA-SSA the two with XA heads, with
 * XAttention's threshold tau = 0.9 and its other settings at their defaults
 * (paper body: experimental setup, baselines paragraph; its efficiency
 * summary quotes the largest prefill speedup for XA-SSA).  XAttention itself
 * ("XAttention: Block Sparse Attention with Antidiagonal Scoring", method
 * section) picks, per query head and per query block of `block` tokens, the
 * key blocks an XA head attends to:
 *
 *   1. score every pair of stride-S position groups by the sum over the
 *      antidiagonal of their S x S tile of Q K^T,
 *      sum_t <q[aS + S-1-t], k[cS + t]>, positions past the sequence end
 *      reading as zero;
 *   2. scale by softmax_scale / S, mask groups after the query group, softmax
 *      over each group row;
 *   3. sum those probabilities inside each block x block tile (block mass);
 *   4. keep block 0 and the diagonal block, then further key blocks in
 *      decreasing mass (ties to the lower index) until the kept mass reaches
 *      tau times the row's total.
 *
 * An XA head then attends causally to the keys of its kept blocks. */
typedef enum {
  EA_HEADS_FA_SSA = 0, /* decision 0 -> FA, 1 -> SA (sink + window) */
  EA_HEADS_FA_XA = 1,  /* decision 0 -> FA, 1 -> XA */
  EA_HEADS_XA_SSA = 2  /* decision 0 -> XA, 1 -> SA */
} ea_head_config;

/* XAttention settings.
 *   block        XA block edge in tokens; must be 128 (XAttention's default)
 *   stride       antidiagonal stride S; must be 8 (XAttention's default)
 *   threshold    tau in [0, 1]
 *   head_config  an ea_head_config value */
typedef struct {
  int32_t block;
  int32_t stride;
  float threshold;
  int32_t head_config;
} ea_xa_params;

/* Bytes of device workspace ea_xa_prefill needs (0 if the sizes are invalid):
 * the routed prefill's work list plus, per (sequence, KV head, query block),
 * a count and the list of kept key blocks (a triangular array of int32), and
 * the selection's scratch: per (sequence, query head, query block i, key block
 * j <= i) 16 float32 (about 64 * Hq * B * nqb^2 / 2 bytes: 1.07 GB at
 * 128K tokens, Hq = 32). */
size_t ea_xa_prefill_workspace_size(int32_t B, int64_t total_tokens, int32_t max_seqlen,
                                    int32_t Hq, int32_t Hkv, int32_t head_dim, ea_dtype dtype);

/* ea_xa_prefill - hybrid prefill with FA, SA and XA heads in one fused
 * attention launch.
 *
 * Arguments as for ea_hybrid_prefill, plus:
 *   xa        XAttention settings (host struct)
 *   xa_mass   out float32 [B, Hq, nqb, nqb] block masses of step 3 for the
 *             XA heads (nqb = ceil(max_seqlen / block); row i holds key
 *             blocks 0..i of query block i, the rest untouched), or NULL
 *   xa_keep   out uint8 [B, Hq, nqb, nqb]: 1 where step 4 keeps key block j
 *             for query block i, 0 for the other j <= i; or NULL
 *
 * Rows of heads that are not XA, and rows past a sequence's last block, are
 * left untouched in xa_mass and xa_keep.  The selection is made per query
 * head; the attention kernel walks the union of a KV group's kept blocks and
 * masks each head to its own.  Each key block is scored once: the
 * log2-sum-exp2 of every group row over the block is kept in the workspace and
 * turned into masses once the row's total is known.  The masses are
 * accumulated in float32 and the threshold decision is taken in float32.  dtype must be EA_BF16; head_dim 64
 * or 128; Hq / Hkv <= 16 and a power of two >= 2 (a query tile then lies
 * inside one XA block); nqb <= 4096.  Work per XA query block grows with its
 * index (every earlier key block is scored). */
ea_status ea_xa_prefill(const void* Q, const void* K, const void* V, ea_dtype dtype,
                        const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                        int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                        int32_t head_dim, const ea_sparsity_params* params,
                        const ea_xa_params* xa, void* O, float* lse, float* xa_mass,
                        uint8_t* xa_keep, void* workspace, size_t workspace_bytes, void* stream);

/* ea_xa_prefill_plan / ea_xa_prefill_run - the two halves of ea_xa_prefill.
 *
 * plan runs the XA selection of every XA head (reading Q, K, modes and
 * cu_seqlens; writing xa_mass / xa_keep when given) and builds the
 * cost-ordered work list, XA items costed by their kept blocks, into
 * `workspace`; run launches the fused attention over a workspace that plan
 * filled with the same arguments.  Arguments, limits and errors are those of
 * ea_xa_prefill; running over a workspace that was not planned for these
 * arguments is a precondition violation (not detected). */
ea_status ea_xa_prefill_plan(const void* Q, const void* K, ea_dtype dtype, const int8_t* modes,
                             const int32_t* cu_seqlens, int32_t B, int64_t total_tokens,
                             int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t head_dim,
                             const ea_sparsity_params* params, const ea_xa_params* xa,
                             float* xa_mass, uint8_t* xa_keep, void* workspace,
                             size_t workspace_bytes, void* stream);

ea_status ea_xa_prefill_run(const void* Q, const void* K, const void* V, ea_dtype dtype,
                            const int8_t* modes, const int32_t* cu_seqlens, int32_t B,
                            int64_t total_tokens, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                            int32_t head_dim, const ea_sparsity_params* params,
                            const ea_xa_params* xa, void* O, float* lse, const void* workspace,
                            size_t workspace_bytes, void* stream);

/* ea_mfma_probe - measurement helper, not part of the attention path: the
 * practical bf16 matrix-core ceiling that the attention kernel's throughput is
 * set against beside the data-sheet peak (256 CUs x 2.4 GHz x 4096 FLOP/clk).
 *
 * Launches n_workgroups workgroups of 8 waves (one per CU: each reserves
 * 96 KiB of LDS), each wave issuing `iters` rounds of 16 back-to-back
 * v_mfma_f32_32x32x16_bf16 over 4 independent accumulators, operands random
 * bf16 drawn from `seed` and held in registers: no memory traffic in the loop,
 * so the board's clock settles where a pure matrix load puts it.
 *
 *   out     out float32 [n_workgroups * 512] device buffer (16-byte aligned),
 *           one checksum per thread (keeps the loop live; values not meaningful)
 *   flops   out, host: FLOPs the launch performs
 *           (n_workgroups * 8 * iters * 16 * 32768), or NULL
 *
 * 1 <= n_workgroups <= 2^20, 1 <= iters <= 2^26.  Asynchronous on `stream`. */
ea_status ea_mfma_probe(float* out, int32_t n_workgroups, int32_t iters, uint32_t seed,
                        int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EA_H */
