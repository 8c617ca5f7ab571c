/*
 * orthros.h - C ABI of the Orthros attention hot path for AMD MI355X (gfx950).
 *
 * Orthros attention keeps two token streams in one layer (pages: "Orthros:
 * Phase-Aware Heterogeneous Attention for Efficient Transformers", paper
 * text §3.1; the paper-notes page of the same title, key designs 1-3):
 *
 *   base stream    q_t  = alpha  (.) (x_t W_Q) + beta    for every position
 *                  o_t  = softmax over keys [t-W+1, t] (window W) of
 *                         q_t . k_j / sqrt(D), applied to V
 *   output stream  q'_t = alpha' (.) (x'_t W_Q) + beta'  for the last T_out
 *                         positions only
 *                  o'_t = softmax over keys [0, t] of q'_t . k_j / sqrt(D),
 *                         applied to V
 *
 * K/V come from the base stream only and form the full per-layer cache that
 * both streams read; the output stream never writes K/V (reproduction note
 * "Orthros：阶段异构注意力", background section). The attention entry
 * points take the projected, pre-affine queries and the projected K/V;
 * orthros_layer_forward also runs the projections and W_O.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  * Indices are 0-based: position t of the pages' 1-based formulas is t-1
 *    here, so the base range is [max(0, t-W+1), t] (exactly min(t+1, W) keys)
 *    and the output range is [0, t].
 *  * Device pointers (marked [dev]) point to device memory owned by the
 *    caller; the library keeps no pointer after a call returns. The
 *    attention entry points never allocate or free device memory: scratch
 *    comes from the caller (ws arguments). Two pieces of device memory are
 *    the library's own: a sticky error flag per device (a static device
 *    variable, see orthros_check_device_errors), and the hipBLASLt handle
 *    that orthros_layer_forward creates on its first call on a device (the
 *    library's allocation, kept until the process ends). Tensors are dense, row-major, no strides.
 *    Host pointers are marked [host] and are read before the call returns.
 *  * Element type `dtype`: ORTHROS_F32 or ORTHROS_BF16 for Q, K, V and the
 *    outputs. alpha/beta vectors are always fp32 with Hq*D entries (one per
 *    channel of the query projection, head-major). Accumulation is fp32.
 *  * D is the per-head dimension and the one in sqrt(D).
 *  * head_map [host] int32[Hq]: KV head read by each query head, values in
 *    [0, Hkv); NULL means the contiguous grouping h / (Hq/Hkv), which then
 *    requires Hq % Hkv == 0.
 *  * K/V cache layout: [B, Hkv, cap, D] (rows 0..cap-1 per batch entry and
 *    KV head); projection layout of new K/V: [B, n, Hkv, D].
 *  * All arguments are validated on the host before any HIP call. On error
 *    the call returns a negative ORTHROS_E* code, launches nothing and
 *    records a message readable with orthros_last_error() (thread-local).
 *  * Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream). Nothing is synchronised; results are ready when the
 *    stream is. Calls that share buffers must be ordered by the caller.
 *  * Zero-sized work (B == 0, T == 0, n_new == 0) returns ORTHROS_OK and
 *    launches nothing.
 *  * Split-KV workspaces (the ws of orthros_global_xattn and the decode
 *    pairs) begin with arrival counters: the first
 *    orthros_workspace_counter_bytes(...) bytes must be zero when a call
 *    starts, and every call leaves them zero. Zero a workspace once after
 *    allocating it (hipMemset); it can then serve any number of calls with
 *    the same B and head grouping. Zero it again before a call with more
 *    (batch entry, head group) pairs, whose counters would overlap bytes an
 *    earlier call used for partial results. The rest of the workspace is
 *    scratch: its contents on entry are ignored and left undefined.
 *  * Device-side capacity faults (a cache length that would exceed cap)
 *    never write out of bounds: the affected batch entry is skipped and a
 *    sticky device flag is raised, reported by orthros_check_device_errors.
 */
#ifndef ORTHROS_H
#define ORTHROS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORTHROS_ABI_VERSION 7

/* dtype codes */
#define ORTHROS_F32 0
#define ORTHROS_BF16 1

/* status codes */
#define ORTHROS_OK 0
#define ORTHROS_EINVAL (-1)       /* bad pointer, size, range or head map */
#define ORTHROS_EUNSUPPORTED (-2) /* dtype or head dimension not supported */
#define ORTHROS_ECAPACITY (-3)    /* cache capacity would be exceeded */
#define ORTHROS_EWORKSPACE (-4)   /* workspace missing or too small */
#define ORTHROS_EHIP (-5)         /* a HIP runtime call failed */

/* workspace query operation codes */
#define ORTHROS_OP_GLOBAL_XATTN 1
#define ORTHROS_OP_DECODE_PAIR 2

/* Largest supported head dimension, query-head count and cache capacity. */
#define ORTHROS_MAX_D 256
#define ORTHROS_MAX_HEADS 128

/*
 * orthros_kv_append - materialise base-stream K/V in the per-layer cache.
 *
 * Pages: paper text §3.1 (k_i = x_i W_K and v_i = x_i W_V for every base
 * position, forming the layer-wise cache); reproduction note, background
 * section (only the base stream writes K/V; the full cache is kept and grows
 * by one row per decode step).
 *
 * For every batch entry b, rows cache_len[b] .. cache_len[b]+n_new-1 of
 * k_cache/v_cache receive k_new[b, 0..n_new-1] / v_new[b, ...]; then
 * cache_len[b] += n_new. A prefill calls it once with n_new = T on an empty
 * cache (cache_len = 0).
 *
 *   k_cache, v_cache [dev] [B, Hkv, cap, D] dtype, written
 *   cache_len        [dev] int32[B], read then advanced
 *   k_new, v_new     [dev] [B, n_new, Hkv, D] dtype, read
 * Errors: EINVAL (null pointer, negative size), EUNSUPPORTED (dtype, D),
 * EHIP. A batch entry whose new length would exceed cap is skipped and the
 * device flag is raised (ECAPACITY from orthros_check_device_errors).
 */
int orthros_kv_append(void *k_cache, void *v_cache, int32_t *cache_len,
                      const void *k_new, const void *v_new, int B, int n_new,
                      int Hkv, int D, int64_t cap, int dtype, void *stream);

/*
 * orthros_swa_prefill - base-stream sliding-window attention, every position.
 *
 * Pages: paper text §3.1, the o_t equation (window w) and the base-query
 * scale-offset; paper-notes page, key designs 1 and 2 (same formulas; the
 * base branch is a local-window attention); reproduction note, mapping
 * section (a local T x window view, never a dense T x T mask).
 *
 * For b < B, t < T, query head h with KV head g = map(h):
 *   q   = alpha[h*D..] (.) q_pre[b,t,h,:] + beta[h*D..]
 *   o[b,t,h,:] = sum_{j=max(0,t-W+1)}^{t} softmax_j(q . k_j / sqrt(D)) v_j
 * with k_j = k_cache[b,g,j,:], v_j = v_cache[b,g,j,:]; rows 0..T-1 of the
 * cache must be valid (orthros_kv_append). W >= T gives full causal
 * attention over the prefix (with identity alpha/beta: standard causal
 * attention).
 *
 *   q_pre        [dev] [B, T, Hq, D] dtype (pre-affine projected queries)
 *   alpha, beta  [dev] fp32 [Hq*D]
 *   k_cache, v_cache [dev] [B, Hkv, cap, D] dtype, cap >= T
 *   o            [dev] [B, T, Hq, D] dtype, written
 *   W            window, >= 1
 * Errors: EINVAL, EUNSUPPORTED, EHIP.
 */
int orthros_swa_prefill(const void *q_pre, const float *alpha,
                        const float *beta, const void *k_cache,
                        const void *v_cache, void *o, int B, int T, int Hq,
                        int Hkv, int D, int64_t cap, int W,
                        const int32_t *head_map, int dtype, void *stream);

/*
 * orthros_global_xattn - output-stream full cross-attention.
 *
 * Pages: paper text §3.1, the o'_t equation and the output-query
 * scale-offset (computed only for the last T_out positions); §3.2 for the
 * (T_in, T_out) settings: prefilling T_in = T-1, T_out = 1; SFT
 * T_out = response length; pre-training T_in = 0, T_out = T; paper-notes
 * page, key design 3 (the cross branch is an attention with unbounded
 * window over the shared cache).
 *
 * Output row r (0 <= r < T_out) sits at position t = T_in + r:
 *   q'  = alpha_x (.) qx_pre[b,r,h,:] + beta_x
 *   o_x[b,r,h,:] = sum_{j=0}^{t} softmax_j(q' . k_j / sqrt(D)) v_j
 * Cache rows 0..T_in+T_out-1 must be valid.
 *
 *   qx_pre       [dev] [B, T_out, Hq, D] dtype
 *   alpha_x, beta_x [dev] fp32 [Hq*D]
 *   k_cache, v_cache [dev] [B, Hkv, cap, D], cap >= T_in + T_out
 *   o_x          [dev] [B, T_out, Hq, D] dtype, written
 *   ws, ws_bytes [dev] scratch of at least orthros_workspace_bytes(
 *                ORTHROS_OP_GLOBAL_XATTN, B, Hq, Hkv, D, T_out, T_in+T_out,
 *                head_map) bytes (may be NULL when that size is 0); its
 *                leading counters zero (see the conventions above).
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP.
 */
int orthros_global_xattn(const void *qx_pre, const float *alpha_x,
                         const float *beta_x, const void *k_cache,
                         const void *v_cache, void *o_x, int B, int T_in,
                         int T_out, int Hq, int Hkv, int D, int64_t cap,
                         const int32_t *head_map, int dtype, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * orthros_decode_pair - one decoding step of the decoupled token pair.
 *
 * Pages: paper text §3.1 (each decoding step processes a decoupled pair: one
 * token runs the window attention and updates the cache, the other runs full
 * cross-attention to predict the next output) and §3.2 Decoding (T = 1,
 * T_out = 1); paper-notes page, key design 4.
 *
 * For each batch entry b with old length n = cache_len[b]:
 *   1. append: k_cache[b,g,n,:] = k_new[b,g,:], v_cache likewise;
 *   2. base query   q  = alpha (.) q_pre[b,h,:] + beta, keys [max(0,n-W+1), n]
 *      -> o[b,h,:]
 *   3. output query q' = alpha_x (.) qx_pre[b,h,:] + beta_x, keys [0, n]
 *      -> o_x[b,h,:]
 *   4. cache_len[b] = n + 1 (after both attentions have read the cache).
 * Reading: the base token's own K/V is appended before it attends, so its
 * window contains itself, as in the prefill formula.
 *
 *   q_pre, qx_pre      [dev] [B, Hq, D] dtype
 *   alpha, beta, alpha_x, beta_x [dev] fp32 [Hq*D]
 *   k_new, v_new       [dev] [B, Hkv, D] dtype
 *   k_cache, v_cache   [dev] [B, Hkv, cap, D], appended in place
 *   cache_len          [dev] int32[B], read then advanced by one
 *   o, o_x             [dev] [B, Hq, D] dtype, written
 *   max_len_after      host upper bound of cache_len[b] + 1 over all b,
 *                      1 <= max_len_after <= cap (sizes the launch). A batch
 *                      entry exceeding it is skipped and the device flag is
 *                      raised.
 *   W                  base window, >= 1
 *   ws, ws_bytes       scratch of orthros_workspace_bytes(
 *                      ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, D, 1, max_len_after,
 *                      head_map), its leading counters zero
 * Errors: EINVAL, EUNSUPPORTED, ECAPACITY (max_len_after > cap), EWORKSPACE,
 * EHIP.
 */
int orthros_decode_pair(const void *q_pre, const void *qx_pre,
                        const float *alpha, const float *beta,
                        const float *alpha_x, const float *beta_x,
                        const void *k_new, const void *v_new, void *k_cache,
                        void *v_cache, int32_t *cache_len, void *o, void *o_x,
                        int B, int Hq, int Hkv, int D, int64_t cap,
                        int64_t max_len_after, int W, const int32_t *head_map,
                        int dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * orthros_decode_pair_noalloc - orthros_decode_pair without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory around the call: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc. The split-KV partials go to
 * a static device array of ORTHROS_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends (its address is
 * looked up on the first call on a device). The call allocates nothing and
 * calls no allocating routine.
 *
 * Sizes whose scratch (orthros_workspace_bytes(ORTHROS_OP_DECODE_PAIR, ...,
 * head_map)) exceeds ORTHROS_NOALLOC_SCRATCH_BYTES are rejected with
 * ORTHROS_EWORKSPACE before anything is launched; 64 MiB covers, e.g.,
 * B = 64 sequences of 32/8 heads up to about 60K cached keys. The array's
 * first ORTHROS_NOALLOC_COUNTER_BYTES hold the arrival counters at a fixed
 * place (zero when the library is loaded, left zero by every call), so
 * sizes whose counters (orthros_workspace_counter_bytes) exceed that are
 * rejected too; the partials follow them. Every call on a device shares
 * that device's array: calls that overlap in time on one device (different
 * streams, no ordering) race and give wrong results.
 * Arguments, results and errors otherwise as orthros_decode_pair.
 */
#define ORTHROS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
#define ORTHROS_NOALLOC_COUNTER_BYTES ((size_t)64 << 10)
int orthros_decode_pair_noalloc(const void *q_pre, const void *qx_pre,
                                const float *alpha, const float *beta,
                                const float *alpha_x, const float *beta_x,
                                const void *k_new, const void *v_new,
                                void *k_cache, void *v_cache,
                                int32_t *cache_len, void *o, void *o_x, int B,
                                int Hq, int Hkv, int D, int64_t cap,
                                int64_t max_len_after, int W,
                                const int32_t *head_map, int dtype,
                                void *stream);

/*
 * Paged K/V cache (variable-length batched decoding).
 *
 * Pages: paper text §3.3 (decoding is bound by memory I/O; batched decoding
 * raises the useful work per byte) and §5, Limitation and Future Work
 * (fitting the decoding mechanism into modern inference frameworks, for
 * single-sample and batched decoding, is left open; the full cache is
 * kept). Layout choice, not from the pages: a pool of fixed-size pages
 * shared by all sequences, so lengths can differ and grow without moving
 * rows.
 *
 *   k_pool, v_pool [dev] [n_pages, Hkv, page_size, D] dtype
 *   block_table    [dev] int32 [B, max_pages]: key i of batch entry b lives
 *                  in page block_table[b * max_pages + i / page_size], row
 *                  i % page_size. Entries must lie in [0, n_pages); pages may
 *                  be shared only by rows that are never written twice.
 *   page_size      power of two, 32 <= page_size <= 65536
 *   cache_len      [dev] int32 [B], per-sequence lengths (ragged)
 * A block-table entry outside [0, n_pages) never causes an out-of-range
 * access: the rows it would address are skipped (append) or its page is
 * replaced by page 0 (decode), the sticky device flag is raised and the
 * outputs of that batch entry are undefined.
 */

/*
 * orthros_kv_append_paged - orthros_kv_append for a paged cache: for every
 * b, rows cache_len[b] .. cache_len[b]+n_new-1 receive k_new[b, 0..n_new-1]
 * / v_new[b, ...] ([B, n_new, Hkv, D]); then cache_len[b] += n_new. A batch
 * entry whose new length exceeds max_pages * page_size is skipped and
 * raises the device flag (ECAPACITY from orthros_check_device_errors).
 * Errors: EINVAL, EUNSUPPORTED (dtype, D), EHIP.
 */
int orthros_kv_append_paged(void *k_pool, void *v_pool, int64_t n_pages,
                            int page_size, const int32_t *block_table,
                            int max_pages, int32_t *cache_len,
                            const void *k_new, const void *v_new, int B,
                            int n_new, int Hkv, int D, int dtype,
                            void *stream);

/*
 * orthros_decode_pair_paged - orthros_decode_pair on a paged cache, with
 * per-sequence (ragged) lengths: for each b with old length n = cache_len[b]
 * the new row is stored at key n, the base query attends keys
 * [max(0, n-W+1), n], the output query keys [0, n], then cache_len[b] =
 * n + 1. bf16 with D = 128 only.
 *
 *   max_len_after  host upper bound of cache_len[b] + 1 over all b,
 *                  1 <= max_len_after <= max_pages * page_size
 *   ws, ws_bytes   scratch of orthros_workspace_bytes(
 *                  ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, D, 1, max_len_after,
 *                  head_map), its leading counters zero
 * Other arguments as orthros_decode_pair.
 * Errors: EINVAL, EUNSUPPORTED (dtype or D), ECAPACITY, EWORKSPACE, EHIP.
 */
int orthros_decode_pair_paged(const void *q_pre, const void *qx_pre,
                              const float *alpha, const float *beta,
                              const float *alpha_x, const float *beta_x,
                              const void *k_new, const void *v_new,
                              void *k_pool, void *v_pool, int64_t n_pages,
                              int page_size, const int32_t *block_table,
                              int max_pages, int32_t *cache_len, void *o,
                              void *o_x, int B, int Hq, int Hkv, int D,
                              int64_t max_len_after, int W,
                              const int32_t *head_map, int dtype, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * orthros_attn_backward - gradients of both attention streams (training).
 *
 * Pages: paper text §3.1 (the o_t and o'_t equations, the query
 * scale-offset) and §3.2 (pre-training makes every position an output row,
 * T_out = T; SFT the response positions), where both streams are trained.
 * Given the forward inputs, the forward outputs o, o' and the upstream
 * gradients dO, dO', it returns, by the chain rule through each softmax row
 * (p = softmax(s), dp_j = dO . v_j, ds_j = p_j (dp_j - dO . o)):
 *   dq_pre  = alpha  (.) sum_j ds_j k_j / sqrt(D)          (base rows)
 *   dqx_pre = alpha' (.) ...                                (output rows)
 *   dk_j = sum over the rows of both streams that see key j of
 *          ds q / sqrt(D), dv_j = sum of p dO  (q = alpha (.) q_pre + beta)
 *   d_alpha = sum over rows of dq (.) q_pre, d_beta = sum of dq (per
 *          channel, over batch and rows), likewise d_alpha_x, d_beta_x.
 * Output row r sits at position T - T_out + r and sees keys [0, that
 * position]; base row t sees [max(0, t-W+1), t], as in the forward calls.
 *
 *   q_pre, o, d_o       [dev] [B, T, Hq, D] bf16
 *   qx_pre, o_x, d_ox   [dev] [B, T_out, Hq, D] bf16 (NULL when T_out = 0)
 *   alpha, beta, alpha_x, beta_x [dev] fp32 [Hq*D]
 *   k_cache, v_cache    [dev] [B, Hkv, cap, D] bf16, rows 0..T-1 used
 *   dq_pre, dqx_pre     [dev] shapes of q_pre, qx_pre, written
 *   dk, dv              [dev] [B, T, Hkv, D] bf16 (projection layout), written
 *   d_alpha, d_beta, d_alpha_x, d_beta_x [dev] fp32 [Hq*D], written
 *                       (the _x pair is written with zeros when T_out = 0
 *                       and the pointers are given)
 *   ws, ws_bytes        [dev] scratch of orthros_backward_workspace_bytes()
 * bf16, D = 128, 16-byte aligned tensors, T <= 2^24, and every KV head
 * with 1..8 query heads; otherwise EUNSUPPORTED. Summation order is fixed,
 * so results are bit-reproducible. Errors: EINVAL, EUNSUPPORTED,
 * EWORKSPACE, EHIP.
 */
int orthros_attn_backward(
    const void *q_pre, const void *qx_pre, const float *alpha,
    const float *beta, const float *alpha_x, const float *beta_x,
    const void *k_cache, const void *v_cache, const void *o, const void *o_x,
    const void *d_o, const void *d_ox, void *dq_pre, void *dqx_pre, void *dk,
    void *dv, float *d_alpha, float *d_beta, float *d_alpha_x,
    float *d_beta_x, int B, int T, int T_out, int Hq, int Hkv, int D,
    int64_t cap, int W, const int32_t *head_map, int dtype, void *ws,
    size_t ws_bytes, void *stream);

/* Scratch bytes orthros_attn_backward needs (0 for invalid sizes). */
size_t orthros_backward_workspace_bytes(int B, int T, int T_out, int Hq,
                                        int Hkv, int D);

/*
 * orthros_layer_forward - one Orthros attention layer, projections included.
 *
 * Pages: paper text §3.1 (k_i = x_i W_K, v_i = x_i W_V for the T base
 * tokens; q_i = alpha (.) (x_i W_Q) + beta for every base token and
 * q'_i = alpha' (.) (x'_i W_Q) + beta' for the T_out output-specific tokens,
 * one shared W_Q) and its description of Algorithm 1 and Figure 1(b): the
 * input is the T base rows followed by the T_out output rows, and the
 * outputs of the two streams, in that same row order, go through W_O.
 *
 * For every batch entry b (T_in = T - T_out, output row r at position
 * T_in + r):
 *   Q    = x[b] W_Q                      all T + T_out rows
 *   K, V = x[b, 0..T-1] W_K, W_V         written to cache rows 0..T-1,
 *                                        then cache_len[b] = T
 *   o    = sliding window (W) of the base queries      rows 0..T-1
 *   o'   = global cross-attention of the output queries rows T..T+T_out-1
 *   y[b] = [o; o'] W_O
 * Projections are hipBLASLt GEMMs (bf16 operands, fp32 accumulation, bf16
 * results); every intermediate (Q, K, V, o) is rounded to bf16, as in the
 * other entry points. Query heads map to KV heads contiguously (h / (Hq/Hkv)).
 *
 *   x           [dev] [B, T + T_out, d_model] bf16
 *   w_q         [dev] [Hq*D, d_model] bf16: W_Q stored out x in (row j holds
 *               column j of W_Q), the layout of a linear layer's weight
 *   w_k, w_v    [dev] [Hkv*D, d_model] bf16, the same way
 *   w_o         [dev] [d_model, Hq*D] bf16, the same way
 *   alpha, beta, alpha_x, beta_x [dev] fp32 [Hq*D] (the _x pair may be NULL
 *               when T_out = 0)
 *   k_cache, v_cache [dev] [B, Hkv, cap, D] bf16, rows 0..T-1 written
 *   cache_len   [dev] int32[B], set to T (whatever it held before)
 *   y           [dev] [B, T + T_out, d_model] bf16, written
 *   ws, ws_bytes [dev] scratch of orthros_layer_workspace_bytes(...) bytes
 *               (intermediates of one batch entry plus GEMM workspace);
 *               contents on entry are ignored (the call zeroes the counters
 *               its cross-attention needs)
 * 1 <= T, 0 <= T_out <= T, cap >= T, W >= 1, Hq a multiple of Hkv.
 * Errors: EINVAL, EUNSUPPORTED (D), EWORKSPACE, EHIP (also a failing
 * hipBLASLt call). The first call on a device creates that device's
 * hipBLASLt handle, kept until the process ends.
 */
int orthros_layer_forward(const void *x, const void *w_q, const void *w_k,
                          const void *w_v, const void *w_o, const float *alpha,
                          const float *beta, const float *alpha_x,
                          const float *beta_x, void *k_cache, void *v_cache,
                          int32_t *cache_len, void *y, int B, int T, int T_out,
                          int d_model, int Hq, int Hkv, int D, int64_t cap,
                          int W, void *ws, size_t ws_bytes, void *stream);

/* Scratch bytes orthros_layer_forward needs (0 for invalid sizes). */
size_t orthros_layer_workspace_bytes(int B, int T, int T_out, int d_model,
                                     int Hq, int Hkv, int D);

/*
 * Scratch bytes needed by orthros_global_xattn (op ORTHROS_OP_GLOBAL_XATTN,
 * max_len = T_in + T_out) or orthros_decode_pair (op ORTHROS_OP_DECODE_PAIR,
 * T_out = 1, max_len = max_len_after; also orthros_decode_pair_paged).
 * head_map [host] is the map the call will be given (NULL for the
 * contiguous grouping): the query heads of each KV head are packed into
 * groups, and the number and width of the groups size the scratch. The size
 * depends on these arguments only, not on the device. Returns 0 for an
 * unknown op, invalid sizes or an invalid map, and when the call needs no
 * scratch for these sizes (ws may then be NULL). Pure host function; it
 * leaves orthros_last_error() unchanged.
 */
size_t orthros_workspace_bytes(int op, int B, int Hq, int Hkv, int D,
                               int T_out, int64_t max_len,
                               const int32_t *head_map);

/*
 * Leading bytes of that workspace holding the arrival counters, which must
 * be zero when a call starts (every call leaves them zero). A split-KV call
 * whose grid the chip holds at once runs as one launch: each workgroup
 * writes its partial result, then counts itself in, and the last to arrive
 * for a (batch entry, head group) combines the partials (in a decode step
 * the last to leave a batch entry also advances its length); larger grids
 * merge in a second launch. Depends on B and the head grouping only.
 * Arguments and zero returns as orthros_workspace_bytes; pure host function.
 */
size_t orthros_workspace_counter_bytes(int op, int B, int Hq, int Hkv, int D,
                                       int T_out, int64_t max_len,
                                       const int32_t *head_map);

/* Static description of a status code. */
const char *orthros_strerror(int code);

/* Message of the last failing call on this host thread ("" if none). */
const char *orthros_last_error(void);

/*
 * Synchronises `stream`, then reads and clears the sticky device flag raised
 * by a capacity fault in orthros_kv_append / orthros_decode_pair on the
 * current device. Returns ORTHROS_OK, ORTHROS_ECAPACITY or ORTHROS_EHIP.
 */
int orthros_check_device_errors(void *stream);

/* ORTHROS_ABI_VERSION of the built library. */
int orthros_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ORTHROS_H */
