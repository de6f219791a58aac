/*
 * libgqa -- grouped-query attention (GQA) and grouped query experts (GQE)
 * for AMD Instinct MI355X (gfx950). C ABI.
 *
 * Problem statement the entry points follow:
 *  - GQA (ml-canon "56 GQA / MQA", section "Idea and mechanism" and the
 *    PyTorch GQA function; IBM Think "What is grouped query attention
 *    (GQA)?"): h query heads are split into g groups and every group shares
 *    one key/value head; g = 1 is multi-query attention (MQA), g = h is
 *    multi-head attention (MHA). q is [B, h, T, d], k and v are [B, g, T, d],
 *    g divides h, query head i reads KV head i / (h/g) (contiguous groups:
 *    freenetmedia "Grouped-Query Attention", section on how it works, example
 *    of 8 heads in 2 groups).
 *  - Attention per head (IBM Think page, scaled dot-product attention):
 *    out = softmax(q k^T * scale) v over keys, scale usually 1/sqrt(d).
 *  - Causal mask: query at position t sees keys 0..t (IBM Think page, on
 *    autoregressive decoders attending to previous tokens).
 *  - Decode over a KV cache (aiunderstanding.org "Attention aux requetes
 *    groupees", section "Plongee profonde"): the keys and values of all
 *    previous tokens are cached, and one new query per sequence attends to
 *    them.
 *  - GQE (gist.science explainer of "Grouped Query Experts: Mixture-of-Experts
 *    on GQA Self-Attention", section "Architecture et Routage"): a router keeps
 *    k query-head experts per token inside every KV group; K/V stay dense; the
 *    kept outputs are weighted by router probabilities renormalised over the
 *    k kept.
 *
 * Conventions for every entry point:
 *  - Memory: all tensor pointers are device pointers to caller-owned memory,
 *    contiguous row-major in the stated layouts, 16-byte aligned. The library
 *    allocates nothing and frees nothing. Between calls it keeps only a
 *    thread-local error message and a host-side cache of the dispatch order
 *    planned for each causal prefill shape (built once per shape under a
 *    mutex, then read).
 *  - dtypes: GQA_F32 = IEEE fp32, GQA_BF16 = bfloat16 (raw 16-bit storage).
 *    Accumulation is always fp32; fp32 inputs are never rounded to bf16.
 *  - Execution: work is enqueued on `stream` (a hipStream_t, NULL = the
 *    default stream) and the call returns without synchronising. A fault in
 *    a kernel surfaces at the caller's next synchronisation.
 *  - Errors: arguments are checked before any HIP call; a rejected call
 *    returns GQA_ERR_INVALID_ARG or GQA_ERR_UNSUPPORTED and enqueues nothing.
 *    GQA_ERR_NO_DEVICE means no HIP device is visible. GQA_ERR_HIP means a
 *    HIP launch failed. gqa_last_error() returns the calling thread's
 *    message for its last failed call.
 *  - Empty problems (B = 0 or T = 0) return GQA_OK and enqueue nothing.
 *  - scale must be finite and > 0. causal must be 0 or 1.
 *  - Element counts must fit the int32 index arithmetic of the kernels:
 *    h*T and g*T below 2^31 per batch element (byte offsets are 64-bit).
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Status codes and element types. Both are int-sized in every language; C++
 * sees them with the fixed underlying type int, so any int a C caller passes
 * (an unknown dtype, say) is a value of the type and is rejected by the
 * argument checks rather than being undefined behaviour.
 */
#ifdef __cplusplus
enum gqa_status : int {
#else
typedef enum {
#endif
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,
  GQA_ERR_UNSUPPORTED = 2,
  GQA_ERR_WORKSPACE = 3,
  GQA_ERR_NO_DEVICE = 4,
  GQA_ERR_HIP = 5
#ifdef __cplusplus
};
enum gqa_dtype : int { GQA_F32 = 0, GQA_BF16 = 1 };
#else
} gqa_status;
typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;
#endif

/* Version of this ABI; bumped on any incompatible change. */
int gqa_abi_version(void);

/*
 * GQA prefill (self-attention over one sequence block).
 *   q   [B, h, T, d] in_dtype      k, v [B, g, T, d] in_dtype
 *   out [B, h, T, d] out_dtype (written in full)
 * out[b, i, t] = sum_j softmax_j(scale * q[b,i,t] . k[b, i/(h/g), j]) v[b, i/(h/g), j]
 * over j <= t when causal, over all j < T otherwise.
 * Supported: d in {16, 32, 64, 128} for both input dtypes; out_dtype F32 or
 * BF16 (round to nearest even). bf16 inputs at d 64 and 128 run on the matrix
 * cores (P rounded to bf16 for the P.V product, fp32 accumulation); fp32
 * inputs, and bf16 inputs at d 16 and 32, run in fp32 arithmetic throughout.
 */
gqa_status gqa_prefill(const void* q, const void* k, const void* v, void* out,
                       int B, int h, int g, int T, int d,
                       gqa_dtype in_dtype, gqa_dtype out_dtype,
                       float scale, int causal, void* stream);

/*
 * Bytes of device workspace gqa_decode needs: two partial results (h/g heads
 * of d fp32 values plus a max and a sum each) per wave of the decode grid,
 * which holds one wave per resident wave slot of the current device. It does
 * not depend on B or T_max (they are accepted for the shape check only, and
 * B = 0 or T_max = 0 give the same size as any other valid shape); 0 for an
 * invalid shape. The GQA_DECODE_UNITS environment variable overrides the wave
 * count.
 */
size_t gqa_decode_workspace_bytes(int B, int h, int g, int T_max, int d);

/*
 * GQA decode: one new query token per sequence over a KV cache.
 *   q       [B, h, d] in_dtype
 *   k_cache [B, g, T_max, d] in_dtype, v_cache the same
 *   lens    [B] int32, device memory: valid cached positions per sequence,
 *           read on the device and clamped to [0, T_max]. The cache already
 *           holds the new token's key/value at position lens[b]-1. Positions
 *           >= lens[b] are never read (they may hold anything, NaN included).
 *   out     [B, h, d] out_dtype; lens[b] = 0 gives a zero row.
 *   workspace: device memory of at least gqa_decode_workspace_bytes(...)
 *           bytes, 16-byte aligned; contents are scratch (no zeroing needed).
 *           Calls that overlap on one workspace race.
 * Supported: in_dtype BF16 or F32, d in {16, 32, 64, 128}, h/g <= 64. F32
 * caches run with fp32 operands throughout (fp32 matrix instructions) and
 * read the cache once per 16 heads of a group.
 * Returns GQA_ERR_WORKSPACE when workspace_bytes is too small.
 */
gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* lens, void* out,
                      int B, int h, int g, int T_max, int d,
                      gqa_dtype in_dtype, gqa_dtype out_dtype, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and kernels as gqa_decode, with the split partials kept in
 * a static device array of the library (16 MiB on every device the library
 * runs on, held until the process ends) instead of a caller's workspace. The
 * call itself allocates nothing. Arguments as for gqa_decode, without the
 * workspace. All calls on one device share that array, so calls that overlap
 * on one device race; consecutive calls on one stream are safe (every partial
 * a call reads was written by that call, so the array needs no clearing).
 * Returns GQA_ERR_WORKSPACE when the shape needs more partials than the array
 * holds (gqa_decode_workspace_bytes(...) above 16 MiB), and GQA_ERR_HIP when
 * the array's device address cannot be looked up.
 */
gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* lens, void* out,
                              int B, int h, int g, int T_max, int d,
                              gqa_dtype in_dtype, gqa_dtype out_dtype, float scale, void* stream);

/*
 * GQE layer output as the pages build it (gist.science explainer of "Grouped
 * Query Experts", section "Architecture et Routage", output construction):
 * the outputs of the k experts kept in every group, concatenated; a weighted
 * sum of them with the router probabilities renormalised over the k kept; and
 * one more head, shared and always active, computed for every token. At 16
 * query heads in 8 groups with k = 1 that is 9 query-attention computations
 * of 16. Readings where the pages are silent: the shared head reads KV head
 * shared_kv and has a query of its own; the outputs are token-major.
 *   q [B, h, T, d], k/v [B, g, T, d], router_logits [B, T, h]: as for
 *           gqe_routed_prefill; in_dtype BF16 only.
 *   q_shared [B, T, d] in_dtype: the shared head's queries.
 *   top_k   experts kept per group, 1 <= top_k <= h/g <= 64.
 *   shared_kv  KV head read by the shared head, 0 <= shared_kv < g.
 *   out_concat [B, T, g, top_k, d] out_dtype, written: the attention rows of
 *           the kept heads (not gated), groups in order, experts in rank order.
 *   out_wsum [B, T, g, d] out_dtype, written: sum over j of gate_j * row_j,
 *           formed from out_concat as stored (rounded to out_dtype).
 *   out_shared [B, T, d] out_dtype, written: the shared head's attention.
 *   topk_idx / topk_gate [B, T, g, top_k]: as for gqe_routed_prefill.
 * Supported: d in {64, 128}. Errors as for gqe_routed_prefill, plus
 * GQA_ERR_INVALID_ARG for shared_kv outside [0, g) and GQA_ERR_UNSUPPORTED
 * for fp32 inputs.
 */
gqa_status gqe_prefill_build(const void* q, const void* q_shared, const void* k, const void* v,
                             const float* router_logits, int top_k, int shared_kv,
                             void* out_concat, void* out_wsum, void* out_shared,
                             int32_t* topk_idx, float* topk_gate,
                             int B, int h, int g, int T, int d,
                             gqa_dtype in_dtype, gqa_dtype out_dtype,
                             float scale, int causal, void* stream);

/*
 * GQE router with its projection: logits = x w_r^T for every token, then the
 * top-k experts of every KV group and their gates, in one kernel.
 * The pages have the router examine each token and keep k query-head experts
 * per group (gist.science explainer of "Grouped Query Experts", section
 * "Architecture et Routage") without fixing the router's form; this is the
 * linear reading (one weight row per head, like the attention projections).
 *   x       [n_tokens, d_model] bf16, device: the tokens' input vectors
 *           (n_tokens = B*T for a [B, T, d_model] batch).
 *   w_r     [h, d_model] bf16, device: one row of router weights per head.
 *   top_k   experts kept per group, 1 <= top_k <= h/g.
 *   logits  [n_tokens, h] fp32, device, written when not NULL: the scores the
 *           selection used (accumulated in fp32); they can be passed to
 *           gqe_routed_prefill as its router_logits.
 *   topk_idx  [n_tokens, g, top_k] int32, written: kept heads in rank order
 *           (higher logit first, equal logits by lower head id).
 *   topk_gate [n_tokens, g, top_k] fp32, written: softmax of the kept logits.
 * Supported: in_dtype BF16, h <= 64, d_model a multiple of 128.
 * Errors: GQA_ERR_INVALID_ARG (shape, top_k, null or misaligned pointer),
 * GQA_ERR_UNSUPPORTED, GQA_ERR_NO_DEVICE, GQA_ERR_HIP.
 */
gqa_status gqe_router(const void* x, const void* w_r, int top_k, float* logits,
                      int32_t* topk_idx, float* topk_gate,
                      int n_tokens, int d_model, int h, int g,
                      gqa_dtype in_dtype, void* stream);

/*
 * GQE routed decode: one new token per sequence over a KV cache, with the
 * router of gqe_routed_prefill applied to that token (gist.science explainer
 * of "Grouped Query Experts", section "Architecture et Routage": top-k query
 * head experts per KV group, the key/value path stays dense).
 *   q, k_cache, v_cache, lens, out, workspace: as for gqa_decode (the same
 *           gqa_decode_workspace_bytes(...) bytes suffice).
 *   router_logits [B, h] fp32, device: the router's score of every head for
 *           the new token.
 *   top_k   experts kept per group, 1 <= top_k <= h/g <= 64.
 *   topk_idx  [B, g, top_k] int32, written: kept heads in rank order (higher
 *           logit first, equal logits by lower head id).
 *   topk_gate [B, g, top_k] fp32, written: softmax of the kept logits.
 *   out [B, h, d] out_dtype, written in full: a kept head's row is gate times
 *           the plain decode row of that head (every cached key of its group
 *           below lens[b]); every other row is 0, as is every row of a
 *           sequence with lens[b] = 0.
 * Supported and errors: as for gqa_decode, plus GQA_ERR_INVALID_ARG for
 * top_k outside [1, h/g] or a null router pointer.
 */
gqa_status gqe_routed_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* lens, const float* router_logits, int top_k,
                             void* out, int32_t* topk_idx, float* topk_gate,
                             int B, int h, int g, int T_max, int d,
                             gqa_dtype in_dtype, gqa_dtype out_dtype, float scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * GQE routed prefill.
 *   q [B, h, T, d], k/v [B, g, T, d] in_dtype, as for gqa_prefill.
 *   router_logits [B, T, h] fp32, device: the router's score of every query
 *           head (expert) for every token.
 *   top_k   experts kept per (token, group), 1 <= top_k <= h/g <= 64.
 *   topk_idx  [B, T, g, top_k] int32, written: global head ids of the kept
 *           experts in rank order (higher logit first, equal logits by lower
 *           head id).
 *   topk_gate [B, T, g, top_k] fp32, written: softmax of the kept logits
 *           (router probabilities renormalised over the kept experts).
 *   out [B, h, T, d] out_dtype, written in full: out[b, i, t] is
 *           gate * (GQA attention row of head i at token t, dense K/V) when
 *           the router kept head i for token t, and 0 otherwise.
 *   workspace: null, or device memory (16-byte aligned) of at least
 *           gqe_workspace_bytes(...) bytes; its contents need no
 *           initialisation and are not kept between calls. Calls that
 *           overlap on one workspace race.
 * Supported: as gqa_prefill. Returns GQA_ERR_WORKSPACE when a non-null
 * workspace is smaller than gqe_workspace_bytes(...).
 */
gqa_status gqe_routed_prefill(const void* q, const void* k, const void* v,
                              const float* router_logits, int top_k,
                              void* out, int32_t* topk_idx, float* topk_gate,
                              int B, int h, int g, int T, int d,
                              gqa_dtype in_dtype, gqa_dtype out_dtype,
                              float scale, int causal,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace gqe_routed_prefill can use at this shape (causal
 * bf16 on the current device; 0 when it would use none). With the workspace,
 * a launch whose grid is less than two blocks per CU may split the key range
 * of its heaviest causal row tiles over two jobs: the first stores its
 * partial result (the row max and row sum in fp32, the output rows divided by
 * their sum in bf16)
 * with a ready flag, and the second merges it into its own and writes the
 * rows. The same result up to rounding (each part rounds its probabilities
 * to bf16 against its own reference maximum, and the first part's rows are
 * rounded to bf16 once), with the work spread over the
 * chip. The second part's wait is bounded; if it runs out (it should not: the
 * first part waits for nothing), that tile's rows are written as NaN. The
 * GQA_SPLIT_WAIT_POLLS environment variable (0 .. 2^20, default 2^20) sets
 * the bound, for tests of that path.
 */
size_t gqe_workspace_bytes(int B, int h, int g, int T, int d, int top_k);

/*
 * KV-cache size in bytes for one layer: 2 (keys and values) * n_kv * d * T
 * * sizeof(dtype) * B (ml-canon page, section on where the KV-cache saving
 * comes from). Returns 0 for negative sizes.
 */
uint64_t gqa_kv_cache_bytes(int B, int n_kv, int T, int d, gqa_dtype dtype);

/* Static description of a status code. */
const char* gqa_status_string(gqa_status status);

/* Detail message of the calling thread's last failed call ("" if none). */
const char* gqa_last_error(void);

/*
 * Peak microbenchmarks: measurement support, not part of the attention path.
 * They give the rates the path's kernels are compared with besides the
 * datasheet peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s). The caller times
 * them (events on `stream`).
 *
 * gqa_peak_hbm_read: reads every 16-byte word of buf once, with the whole
 * chip, and XORs all 32-bit words of it into *xor_out (device memory; the
 * caller sets its start value, 0 for the plain XOR of the buffer).
 *   buf      device memory, 16-byte aligned; bytes a multiple of 16 (0: no-op).
 * Errors: GQA_ERR_INVALID_ARG (size, null or misaligned pointer),
 * GQA_ERR_NO_DEVICE, GQA_ERR_HIP.
 */
gqa_status gqa_peak_hbm_read(const void* buf, size_t bytes, uint32_t* xor_out, void* stream);

/*
 * gqa_peak_mfma_bf16: iters rounds of four independent
 * v_mfma_f32_32x32x16_bf16 per wave, two waves on every SIMD of the device,
 * on register operands only (no memory traffic in the loop).
 *   operands  device memory, 16-byte aligned, 2 KiB: 64 bf16x8 A fragments
 *             (lane l: row l%32, k = 8*(l/32) .. +7 of a 32x16 A) and then 64
 *             B fragments (lane l: column l%32, the same k). Random values
 *             give the power-limited rate of real data.
 *   sum_out   device float: the sum of all accumulators is added to it,
 *             i.e. (waves * 4 * iters) * sum(A B).
 *   flops     host double, written: the flops the launch performs.
 * Errors: GQA_ERR_INVALID_ARG (iters < 1, null or misaligned pointer),
 * GQA_ERR_NO_DEVICE, GQA_ERR_HIP.
 */
gqa_status gqa_peak_mfma_bf16(const void* operands, int iters, float* sum_out, double* flops, void* stream);

/*
 * gqa_peak_attn_tile: the attention tile loop of the bf16 prefill on one tile
 * staged in LDS: per iteration, for one 32-key tile of 32 query rows (head dim
 * 128), the K and V fragment reads from LDS, S^T = K Q^T (8
 * v_mfma_f32_32x32x16_bf16), the online softmax with its bf16 rounding of P,
 * and O^T += V^T P^T (8 more MFMAs), the same tile every iteration, twelve
 * waves on every CU (three per SIMD), no global memory traffic and no barrier. The rate bounds any kernel that does this per-tile work on
 * the device (IBM Think page, scaled dot-product attention; the ml-canon GQA
 * function).
 *   qkv   device memory, 16-byte aligned: q, k and v of one tile, each
 *         [32][128] bf16 row-major.
 *   scale the softmax scale (finite, > 0).
 *   out   device [32][128] fp32, written: the normalised output of one wave,
 *         i.e. softmax(scale q k^T) v over the 32 keys (the tile repeats).
 *   flops host double, written: the flops the launch performs (counted as
 *         16 MFMAs of 2*32*32*16 per wave and iteration).
 * Errors: GQA_ERR_INVALID_ARG (iters < 1, bad scale, null or misaligned
 * pointer), GQA_ERR_NO_DEVICE, GQA_ERR_HIP.
 */
gqa_status gqa_peak_attn_tile(const void* qkv, int iters, float scale, float* out, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
