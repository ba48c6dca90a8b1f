/*
 * mimo_attn.h -- C ABI of the MiMo-V2.6-Flash attention layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (sources, cited by page title and section):
 *   - miles docs "MiMo-V2.6-Flash", section 1 "Model Introduction": hybrid attention with 39 sliding-window
 *     layers (window 128, learnable attention sink) and 9 global layers, 8 vs 4 KV heads, RoPE bases 1e4 vs
 *     1e7; 192-dim Q/K and 128-dim V, V scaled by 0.707, partial RoPE on 64 of 192 dims.
 *   - miles docs "MiMo-V2.6-Flash", section 5.4 "Notable quirks": a sliding-window query sees itself plus
 *     the 128 previous keys (129 in total), window_size = (128, 0); section 5.1 "Parallelism": THD packing of
 *     variable-length samples.
 *   - miles pull request "feat(models): add MiMo-V2.6-Flash-RL support", PR body and commit messages: the
 *     core attention receives (k_channels, v_channels) = (192, 128) and the sink setting, and scales V.
 *
 * What every call computes, for query token i of sequence b (position p = i - cu_seqlens[b]) and query
 * head h, with G = n_q_heads / n_kv_heads and kv = h / G:
 *   q' = RoPE(q[i,h], p), k'_j = RoPE(k[j,kv], p_j): dims 0..63 rotated in rotate-half pairs (d, d+32) by
 *   angle p * rope_base^(-d/32), d = 0..31; dims 64..191 pass through.
 *   s_j = q'.k'_j / sqrt(192) for keys j of the same sequence with j <= i and, when window >= 0,
 *   j >= i - window (window = 128 gives 129 keys); window = -1 is plain causal attention.
 *   LSE = ln(exp(sink[h]) + sum_j exp(s_j))   (the sink term is absent when sink == NULL)
 *   out[i,h] = sum_j exp(s_j - LSE) * 0.707 * v[j,kv]
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous, row-major, in the shapes given.
 *     bf16 means IEEE bfloat16 bit patterns (uint16 storage).  Outputs are fully overwritten.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the null stream).  There is
 *     no host synchronisation and no device-data validation: cu_seqlens must be non-decreasing with
 *     cu_seqlens[0] = 0 and cu_seqlens[batch] = total_tokens, and no sequence may be longer than max_seqlen.
 *   - Argument checks happen on the host before anything is launched; a failing check returns
 *     MIMO_ERR_INVALID_ARG or MIMO_ERR_UNSUPPORTED and launches nothing.  A launch failure returns
 *     MIMO_ERR_HIP.  mimo_attn_last_error() gives a human-readable reason (thread-local).
 *   - The library keeps one RoPE cos/sin table per (device, rope_base) that grows to the largest
 *     max_seqlen seen; it is allocated on first use and freed by mimo_attn_release().
 *   - Head dims are fixed at 192 (Q/K) and 128 (V); n_q_heads % n_kv_heads must be 0.
 */
#ifndef MIMO_ATTN_H
#define MIMO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MIMO_OK = 0,
    MIMO_ERR_INVALID_ARG = 1,   /* a null pointer, a negative size, heads not divisible, window < -1 ... */
    MIMO_ERR_UNSUPPORTED = 2,   /* valid but not built: e.g. a GQA group size this build has no kernel for */
    MIMO_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed */
    MIMO_ERR_WORKSPACE = 4      /* workspace NULL or smaller than the matching *_workspace_size() */
} mimo_status_t;

/* Forward attention of one layer over a THD-packed batch (the training / prefill forward).
 *   q     bf16 [total_tokens, n_q_heads, 192]   un-rotated (RoPE is applied inside)
 *   k     bf16 [total_tokens, n_kv_heads, 192]  un-rotated
 *   v     bf16 [total_tokens, n_kv_heads, 128]  unscaled (the 0.707 factor is applied inside)
 *   sink  fp32 [n_q_heads] learnable sink logits (unscaled; may be -inf), or NULL for no sink
 *   cu_seqlens int32 [batch + 1] device; batch >= 0; max_seqlen >= every sequence length
 *   window   -1 (causal) or >= 0 (the query plus `window` previous keys)
 *   out   bf16 [total_tokens, n_q_heads, 128]
 *   lse   fp32 [n_q_heads, total_tokens] natural-log softmax denominator incl. the sink, or NULL
 *   q_rot bf16 [total_tokens, n_q_heads, 192] or NULL: when given, receives q with RoPE applied, exactly
 *         the values the scores use; a training caller passes it on to mimo_attn_bwd, which then skips
 *         rotating q again
 *   k_rot bf16 [total_tokens, n_kv_heads, 192] or NULL: when given, receives k with RoPE applied (the keys
 *         the scores use), for mimo_attn_bwd in the same way
 *   workspace: device memory of at least mimo_attn_fwd_workspace_size() bytes, owned by the caller; needs
 *   no initialisation and must not be shared with a concurrent call.
 * Source: miles docs "MiMo-V2.6-Flash" sections 1, 5.1, 5.4; miles PR "feat(models): add MiMo-V2.6-Flash-RL
 * support" (core attention with asymmetric channels, sink, V scale). */
mimo_status_t mimo_attn_fwd(const void *q, const void *k, const void *v, const float *sink,
                            const int32_t *cu_seqlens, int32_t batch, int32_t total_tokens,
                            int32_t max_seqlen, int32_t window, double rope_base, int32_t n_q_heads,
                            int32_t n_kv_heads, void *out, float *lse, void *q_rot, void *k_rot,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace mimo_attn_fwd needs: RoPE-rotated K and per-head transposed V (about
 * 640 * n_kv_heads bytes per token), which the kernels then stream from HBM straight into LDS. */
size_t mimo_attn_fwd_workspace_size(int32_t total_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t window);

/* Least bytes of device workspace mimo_attn_bwd needs for these sizes (0 is never returned for valid
 * sizes).  With this much the dq kernel recomputes the scores and dP of every (query, key) pair. */
size_t mimo_attn_bwd_workspace_size(int32_t total_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t window);

/* Bytes of device workspace for the faster backward: the dk/dv kernel keeps every 32 x 32 block of dS it
 * computes (bf16, in the workspace) and the dq kernel reads them back instead of recomputing them.  The
 * size is an upper bound from total_tokens, batch and max_seqlen (causal layers: about
 * n_q_heads * total_tokens * max_seqlen bytes; sliding-window layers: n_q_heads * total_tokens * 384 bytes
 * for window 128).  Equals mimo_attn_bwd_workspace_size() where this path does not apply (n_q_heads /
 * n_kv_heads not a multiple of 4).  mimo_attn_bwd takes this path whenever workspace_bytes reaches this
 * size; both paths give the same gradients up to fp32 summation order. */
size_t mimo_attn_bwd_workspace_size_fast(int32_t total_tokens, int32_t batch, int32_t max_seqlen,
                                         int32_t n_q_heads, int32_t n_kv_heads, int32_t window);

/* Backward of mimo_attn_fwd (the training backward, "given the forward outputs").
 *   q, k, v, sink, cu_seqlens, batch, total_tokens, max_seqlen, window, rope_base, heads: as the forward
 *   out   bf16 [total_tokens, n_q_heads, 128]  forward output (used for D = rowsum(dO * O))
 *   lse   fp32 [n_q_heads, total_tokens]       forward LSE
 *   dout  bf16 [total_tokens, n_q_heads, 128]  upstream gradient dO
 *   q_rot bf16 [total_tokens, n_q_heads, 192]  the forward's q_rot output for these q and positions, or
 *         NULL (the backward then rotates q itself into the workspace); read only
 *   k_rot bf16 [total_tokens, n_kv_heads, 192]  the forward's k_rot output for these k and positions, or
 *         NULL; read only.  The stored-dS path then reads it instead of rotating k into the workspace (the
 *         least-workspace path needs a transposed copy and still prepares its own)
 *   dq    bf16 [total_tokens, n_q_heads, 192]  gradient w.r.t. the un-rotated q
 *   dk    bf16 [total_tokens, n_kv_heads, 192] gradient w.r.t. the un-rotated k (summed over the group)
 *   dv    bf16 [total_tokens, n_kv_heads, 128] gradient w.r.t. the unscaled v (summed over the group)
 *   dsink fp32 [n_q_heads] gradient of the sink logits; must be non-NULL exactly when sink is non-NULL
 *   workspace: device memory of at least mimo_attn_bwd_workspace_size() bytes (at least
 *   mimo_attn_bwd_workspace_size_fast() bytes selects the stored-dS path), owned by the caller, needs no
 *   initialisation, and must not be shared with a concurrent call.  max_seqlen must not be below the longest
 *   sequence (the stored-dS path sizes its blocks by it; a smaller value gives wrong gradients, never an
 *   access outside the workspace).
 * dsink is summed in a fixed order (no float atomics), so it is bitwise repeatable.
 * Source: the exact gradient of the forward above; miles docs "MiMo-V2.6-Flash" section 5.4 (the trainer's
 * fused attention carries the sink in training). */
mimo_status_t mimo_attn_bwd(const void *q, const void *k, const void *v, const float *sink,
                            const void *out, const float *lse, const void *dout, const void *q_rot,
                            const void *k_rot, const int32_t *cu_seqlens, int32_t batch, int32_t total_tokens,
                            int32_t max_seqlen, int32_t window, double rope_base, int32_t n_q_heads,
                            int32_t n_kv_heads, void *dq, void *dk, void *dv, float *dsink,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace mimo_attn_decode needs. */
size_t mimo_attn_decode_workspace_size(int32_t batch, int32_t max_cache_len, int32_t n_q_heads,
                                       int32_t window);

/* One decode step: each of `batch` sequences has one new token at position positions[b].
 *   q      bf16 [batch, n_q_heads, 192]   un-rotated query of the new token
 *   k_new  bf16 [batch, n_kv_heads, 192]  un-rotated key of the new token
 *   v_new  bf16 [batch, n_kv_heads, 128]  value of the new token (unscaled)
 *   k_cache bf16 [rows, n_kv_heads, 192]  cached keys, ALREADY rotated at their own positions
 *   v_cache bf16 [rows, n_kv_heads, 128]  cached values, unscaled
 *   cu_cache int32 [batch + 1] device: sequence b owns cache rows cu_cache[b] .. cu_cache[b+1]-1, oldest
 *            first; max_cache_len >= every cu_cache[b+1] - cu_cache[b]
 *   positions int32 [batch] device: position of the new token (used to rotate q and k_new)
 *   sink   fp32 [n_q_heads] or NULL; window -1 (all cached rows) or >= 0 (the last min(n_b, window) rows)
 *   out    bf16 [batch, n_q_heads, 128]
 *   workspace: at least mimo_attn_decode_workspace_size() bytes of device memory (split-KV partials).
 * The cache is read, never written.  A 128-entry ring cache with window 128 is attended whole, so the ring
 * order does not matter (softmax does not depend on the order of its keys).
 * Source: miles PR "feat(models): add MiMo-V2.6-Flash-RL support", commit message on the rollout engine's
 * window (query + 128 previous keys); miles docs section 3.2 (separate sliding-window KV pools). */
mimo_status_t mimo_attn_decode(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                               const void *v_cache, const int32_t *cu_cache, const int32_t *positions,
                               const float *sink, int32_t batch, int32_t max_cache_len, int32_t window,
                               double rope_base, int32_t n_q_heads, int32_t n_kv_heads, void *out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace mimo_attn_prefill_cached needs (0 for invalid sizes). */
size_t mimo_attn_prefill_cached_workspace_size(int32_t total_tokens, int32_t total_cache, int32_t n_kv_heads);

/* Prefill of a chunk of new tokens over a cached prefix: the serving engine prefills long prompts in chunks
 * (up to 49152 tokens) against its KV cache.  Source: SGLang cookbook page "MiMo-V2.6", section 2
 * "Configuration tips", "Context length and memory" (chunked prefill size, page size 1).
 *   q, k, v   the new tokens, THD-packed as in mimo_attn_fwd: bf16 [total_tokens, n_q_heads, 192],
 *             [total_tokens, n_kv_heads, 192] (both un-rotated), [total_tokens, n_kv_heads, 128] (unscaled)
 *   k_cache   bf16 [total_cache, n_kv_heads, 192]  cached keys, ALREADY rotated at their own positions
 *   v_cache   bf16 [total_cache, n_kv_heads, 128]  cached values, unscaled
 *   sink      fp32 [n_q_heads] or NULL
 *   cu_seqlens int32 [batch + 1] device: new tokens of sequence b are cu_seqlens[b] .. cu_seqlens[b+1]-1
 *   cu_cache  int32 [batch + 1] device: sequence b's cache rows cu_cache[b] .. cu_cache[b+1]-1 are the n_b
 *             keys just before its new tokens, in position order (a sliding-window layer may keep only the
 *             last rows; rows older than the window are never read by the math, so they may be absent)
 *   positions int32 [batch] device: position of sequence b's first new token; cache row j of b sits at
 *             position positions[b] - n_b + j, new token i at positions[b] + i.  positions[b] >= n_b.
 *   max_seqlen >= every new-token count; max_position >= every positions[b] + (new tokens of b) (the RoPE
 *             table is built up to it; larger positions are clamped to its last entry)
 *   window    -1 (causal over cache and chunk) or >= 0 (each new token sees itself plus `window` previous
 *             keys, cache rows included)
 *   out       bf16 [total_tokens, n_q_heads, 128];  lse fp32 [n_q_heads, total_tokens] or NULL
 *   workspace at least mimo_attn_prefill_cached_workspace_size() bytes of device memory (the prepared key
 *             stream: cache rows and the chunk's rotated keys per sequence)
 * With positions[b] = n_b, new token i of sequence b gets the row that mimo_attn_fwd gives token n_b + i of
 * the whole sequence whose first n_b tokens are the cache; with no cache rows and positions 0 this is
 * mimo_attn_fwd.
 * The cache is read, never written. */
mimo_status_t mimo_attn_prefill_cached(const void *q, const void *k, const void *v, const void *k_cache,
                                       const void *v_cache, const float *sink, const int32_t *cu_seqlens,
                                       const int32_t *cu_cache, const int32_t *positions, int32_t batch,
                                       int32_t total_tokens, int32_t total_cache, int32_t max_seqlen,
                                       int32_t max_position, int32_t window, double rope_base,
                                       int32_t n_q_heads, int32_t n_kv_heads, void *out, float *lse,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Paged KV cache (page size 1: one token per pool row).  Source: SGLang cookbook page "MiMo-V2.6", section 2
 * "Configuration tips", "Context length and memory" (page size 1; decode batches up to 64); miles docs
 * "MiMo-V2.6-Flash" section 3.2 (sliding-window layers keep their own KV pools).
 *
 * A pool is k_pool bf16 [pool_rows, n_kv_heads, 192] (keys ALREADY rotated at their own positions) and
 * v_pool bf16 [pool_rows, n_kv_heads, 128] (unscaled).  A sequence's cache is a list of pool rows: entries
 * page_table[cu_pages[b]] .. page_table[cu_pages[b+1]-1] (int32, device), in position order.  Every pool row
 * a table names must lie in [0, pool_rows); nothing on the device checks it. */

/* Write n_tokens new tokens into a pool: token i's key (bf16 [n_tokens, n_kv_heads, 192], un-rotated) is
 * rotated at positions[i] and stored, with its value (bf16 [n_tokens, n_kv_heads, 128], unscaled), in pool
 * row slots[i] (int32 device arrays).  The rotated key is bit-identical to the one the forward computes for
 * the same token and position.  Slots outside [0, pool_rows) are skipped; duplicate slots race. */
mimo_status_t mimo_attn_cache_append(const void *k, const void *v, const int32_t *positions, const int32_t *slots,
                                     int32_t n_tokens, int32_t n_kv_heads, int32_t pool_rows, double rope_base,
                                     void *k_pool, void *v_pool, void *stream);

/* mimo_attn_decode over a paged cache: cache row r of sequence b is pool row page_table[cu_pages[b] + r];
 * max_cache_len >= every cu_pages[b+1] - cu_pages[b].  Everything else (q, k_new, v_new, positions, sink,
 * window, out, workspace of mimo_attn_decode_workspace_size()) as mimo_attn_decode. */
mimo_status_t mimo_attn_decode_paged(const void *q, const void *k_new, const void *v_new, const void *k_pool,
                                     const void *v_pool, const int32_t *page_table, const int32_t *cu_pages,
                                     const int32_t *positions, const float *sink, int32_t batch,
                                     int32_t max_cache_len, int32_t window, double rope_base, int32_t n_q_heads,
                                     int32_t n_kv_heads, void *out, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* mimo_attn_decode_paged for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments and result as mimo_attn_decode_paged
 * minus the workspace: the split-KV partials live in a 64 MiB array that the library keeps on each device
 * it runs on until the process ends (its address is looked up once per device, on the first call there).
 * The call allocates nothing, creates no HIP events (kernel tracing skips it) and only launches kernels.
 *   - When the usual split plan's partials (batch * n_q_heads * splits * 520 bytes) exceed 64 MiB, the call
 *     uses fewer, longer splits, so its fp32 summation order (not its result beyond rounding) can differ
 *     from mimo_attn_decode_paged's; batch * n_q_heads above 129055 (one split no longer fits) returns
 *     MIMO_ERR_UNSUPPORTED.
 *   - Every call on a device shares that device's array, and calls keep nothing in it that a later call
 *     needs: calls that overlap in time on one device (other streams, other threads) race and give wrong
 *     results; calls in one stream order are safe. */
mimo_status_t mimo_attn_decode_paged_noalloc(const void *q, const void *k_new, const void *v_new, const void *k_pool,
                                             const void *v_pool, const int32_t *page_table, const int32_t *cu_pages,
                                             const int32_t *positions, const float *sink, int32_t batch,
                                             int32_t max_cache_len, int32_t window, double rope_base,
                                             int32_t n_q_heads, int32_t n_kv_heads, void *out, void *stream);

/* Bytes of device workspace mimo_attn_verify_paged needs (0 for invalid sizes). */
size_t mimo_attn_verify_workspace_size(int32_t batch, int32_t n_query, int32_t max_cache_len, int32_t n_q_heads,
                                       int32_t window);

/* The verify step of speculative decoding over a paged cache: each sequence has n_query draft tokens at
 * positions positions[b] .. positions[b] + n_query - 1 whose keys and values were already appended
 * (mimo_attn_cache_append) as the LAST n_query entries of its page-table list.  Draft token i sees the
 * table entries up to its own (entry n_b - n_query + i) and, when window >= 0, at most `window` entries
 * below it; the sink is in the denominator.  Source: SGLang cookbook page "MiMo-V2.6", section 2
 * "Configuration tips" (speculative decoding with DFlash, decode batches up to 64).
 *   q     bf16 [batch * n_query, n_q_heads, 192] un-rotated, sequence-major (row b * n_query + i)
 *   out   bf16 [batch * n_query, n_q_heads, 128]
 *   max_cache_len >= every list length (drafts included); workspace of mimo_attn_verify_workspace_size().
 * The cache is read once per KV head and split, as in decode.  n_query = 1 gives the decode of a token
 * whose key is already in the cache. */
mimo_status_t mimo_attn_verify_paged(const void *q, const void *k_pool, const void *v_pool, const int32_t *page_table,
                                     const int32_t *cu_pages, const int32_t *positions, const float *sink,
                                     int32_t batch, int32_t n_query, int32_t max_cache_len, int32_t window,
                                     double rope_base, int32_t n_q_heads, int32_t n_kv_heads, void *out,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* mimo_attn_prefill_cached over a paged cache (total_pages table entries; workspace of
 * mimo_attn_prefill_cached_workspace_size(total_tokens, total_pages, n_kv_heads)).  It copies the cache
 * rows into the workspace first: for a few tokens per sequence mimo_attn_verify_paged reads the cache
 * once instead. */
mimo_status_t mimo_attn_prefill_paged(const void *q, const void *k, const void *v, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const float *sink,
                                      const int32_t *cu_seqlens, const int32_t *cu_pages, const int32_t *positions,
                                      int32_t batch, int32_t total_tokens, int32_t total_pages, int32_t max_seqlen,
                                      int32_t max_position, int32_t window, double rope_base, int32_t n_q_heads,
                                      int32_t n_kv_heads, void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Per-kernel tracing.  While enabled, every entry point records a HIP event on the caller's stream before
 * and after each kernel it launches (the events only mark the stream; nothing is synchronised).  The
 * records accumulate until mimo_attn_trace_clear(); reading one waits for its end event.  Not thread-safe
 * with concurrent calls on other threads while enabled. */
mimo_status_t mimo_attn_trace_enable(int enable);
int32_t mimo_attn_trace_count(void);
/* Name of kernel record i (static string) and its duration in milliseconds. */
mimo_status_t mimo_attn_trace_read(int32_t i, const char **name, float *ms);
void mimo_attn_trace_clear(void);

/* Name of a status code. */
const char *mimo_attn_status_string(mimo_status_t s);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *mimo_attn_last_error(void);

/* Frees the cached RoPE tables of every device.  No call may be in flight. */
void mimo_attn_release(void);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_ATTN_H */
