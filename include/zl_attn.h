/*
 * zl_attn.h -- C ABI of the MI355X (gfx950) fused batched decode attention
 * library, libzl_attn.so.
 *
 * The operation.  In the decode stage of LLM serving every sequence of a
 * dynamically assembled batch contributes one new query token per head; that
 * query attends over the sequence's whole key/value cache.  The ZhiLight pages
 * single this out as the engine's core difference from vLLM/SGLang ("ZhiLight：
 * 知乎开源的高性能 LLM 推理加速引擎", section 4 "Tensor Core 上的 Flash
 * Attention": decode runs a tensor-core Fused Batch Attention because one new
 * token per step with small batches suits the matrix units; "ZhiLight: Zhihu's
 * CUDA Inference Engine for Llama and DeepSeek on PCIe GPUs", section "Dual
 * streams, host all-reduce and the memory model": fused batch attention for
 * decoding with tensor core instructions).  Batches are built from requests of
 * different lengths (first page, section "功能生态", dynamic batching), so the
 * cache is ragged.  The pages give no formula; the library computes the plain
 * scaled-dot-product attention for every (sequence b, query head h):
 *
 *     s_i = softmax_scale * <q[b,h,:], K[cu[b]+i, g(h), :]>,  0 <= i < L_b
 *     out[b,h,:] = sum_i exp(s_i - m) V[cu[b]+i, g(h), :] / sum_i exp(s_i - m)
 *     lse[b,h]   = m + ln(sum_i exp(s_i - m)),   m = max_i s_i
 *     L_b = 0  ->  out = 0, lse = -inf
 *
 * with g(h) = h / (num_q_heads / num_kv_heads): consecutive query heads share
 * one key/value head (grouped/multi-query attention; the third page, part 01
 * section 1, names Multi-Query Attention as a variant of multi-head attention).
 * No causal mask: the cache holds every token the new query may see.
 *
 * Conventions for every entry point.
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *    buffer; the library keeps no pointer after it returns.
 *  - Work is enqueued on `stream` (NULL = the default stream) and is
 *    asynchronous: nothing synchronises, nothing is allocated.  A decode call
 *    enqueues two kernels: the decode kernel, which splits the batch evenly
 *    over its workers and leaves fp32 partials for sequences that several
 *    workers share, and the merge kernel, which combines those partials and
 *    writes the results of empty sequences.
 *  - Host-checkable arguments are validated before any HIP call; a bad argument
 *    returns an error status and enqueues nothing.
 *  - Cache lengths are clamped inside the kernels: sequence b attends over
 *    L_b = clamp(cu[b+1] - cu[b], 0, max_seqlen_k) rows, starting at cache
 *    row cu[b] (packed caches) or at the first row of its first page (paged
 *    caches).  A length above max_seqlen_k is cut to its first max_seqlen_k
 *    rows and a negative one (cu decreasing) counts as empty, so no read
 *    leaves rows cu[b] .. cu[b] + max_seqlen_k - 1 of a packed cache or the
 *    first ceil(max_seqlen_k / page_size) entries of a block-table row.  The
 *    remaining device precondition is that those rows (packed) or the page
 *    ids in those entries (paged) exist; with cu[0] = 0, cu non-decreasing,
 *    every length at most max_seqlen_k and cu[batch] = total_tokens the
 *    clamp changes nothing.  ZL_ERR_UNSUPPORTED when batch * (max_seqlen_k +
 *    C) >= 2^31 (C = 32 for GQA, 64 for MLA; the work split numbers
 *    positions in 32 bits).
 *  - dtype arguments are ints holding a zl_dtype_t value; any other value
 *    returns ZL_ERR_INVALID_ARGUMENT (an int parameter, so that a value
 *    outside the enumeration is an error status rather than undefined
 *    behaviour in the library).  zl_status_string likewise takes any int.
 *  - 16-bit buffers (q, k, v, latent, out) must be 16-byte aligned.  Rows are
 *    dense: the layouts below have no padding.
 *  - Results are bitwise deterministic for identical inputs, arguments and
 *    device (no floating-point atomics; fixed reduction order).
 *  - Calls that share one workspace must not overlap in time (same stream, or
 *    ordered by events).
 *  - No status crosses the ABI as an exception; nothing aborts or prints.
 */
#ifndef ZL_ATTN_H
#define ZL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ZL_API __attribute__((visibility("default")))
#else
#define ZL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZL_OK = 0,
    ZL_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misalignment, ...   */
    ZL_ERR_UNSUPPORTED = 2,        /* valid but not implemented (head_dim, ...)   */
    ZL_ERR_WORKSPACE_TOO_SMALL = 3,
    ZL_ERR_HIP = 4                 /* a HIP runtime call or launch failed          */
} zl_status_t;

typedef enum {
    ZL_DTYPE_F16 = 0,              /* IEEE binary16                                */
    ZL_DTYPE_BF16 = 1              /* bfloat16                                     */
} zl_dtype_t;

/* Opaque HIP stream handle (hipStream_t); NULL means the default stream. */
typedef struct ihipStream_t *zl_stream_t;

/*
 * Bytes of device workspace that zl_decode_attn_gqa needs for these sizes
 * (host function, no HIP call).  Returns 0 for invalid sizes.  The workspace
 * holds two fp32 partial results and one int per worker; it needs no
 * initialisation and its contents are meaningless between calls.
 */
ZL_API size_t zl_decode_attn_workspace_size(int batch, int num_q_heads, int num_kv_heads,
                                     int head_dim, int max_seqlen_k, int dtype);

/*
 * Grouped-query decode attention over a packed ragged cache (the operation in
 * the file header).
 *   q          [batch, num_q_heads, head_dim]             dtype
 *   k_cache    [total_tokens, num_kv_heads, head_dim]     dtype, sequence b
 *              owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1
 *   v_cache    [total_tokens, num_kv_heads, head_dim]     dtype, same rows
 *              (k_cache / v_cache may be NULL only if every sequence is empty)
 *   cu_seqlens [batch + 1] int32 (device)
 *   batch >= 0 (0 is a no-op), num_q_heads % num_kv_heads == 0,
 *   num_q_heads / num_kv_heads <= 16 or a multiple of 16,
 *   head_dim in {64, 128} (else ZL_ERR_UNSUPPORTED),
 *   max_seqlen_k (host): the clamp on every sequence length (above),
 *   softmax_scale finite (0 allowed),
 *   out        [batch, num_q_heads, head_dim] dtype, fully overwritten
 *   lse        [batch, num_q_heads] float32, natural log; NULL = not written
 *   workspace  >= zl_decode_attn_workspace_size(...) bytes, 256-byte aligned
 */
ZL_API zl_status_t zl_decode_attn_gqa(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *cu_seqlens, int batch, int num_q_heads,
                               int num_kv_heads, int head_dim, int max_seqlen_k,
                               float softmax_scale, int dtype, void *out, float *lse,
                               void *workspace, size_t workspace_bytes, zl_stream_t stream);

/*
 * zl_decode_attn_gqa for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and kernels, with no workspace
 * argument.  The workspace is a fixed 16 MiB array in device memory that the
 * library holds on every GPU it runs on until the process ends (the default
 * worker counts need at most 12.4 MiB, for D = 64 and 128 alike).  A call whose
 * workspace would exceed it returns ZL_ERR_WORKSPACE_TOO_SMALL; sizes the
 * plain call rejects get its status.  The first call on a device looks up the
 * array's device address (one hipGetSymbolAddress); nothing is allocated,
 * nothing is cleared (the workspace needs no initialisation).  All calls on
 * one GPU share the array: calls that overlap in time on one GPU race, so
 * keep them on one stream or order them with events.
 */
ZL_API zl_status_t zl_decode_attn_gqa_no_alloc(const void *q, const void *k_cache, const void *v_cache,
                                               const int32_t *cu_seqlens, int batch, int num_q_heads,
                                               int num_kv_heads, int head_dim, int max_seqlen_k,
                                               float softmax_scale, int dtype, void *out, float *lse,
                                               zl_stream_t stream);

/*
 * Bytes of device workspace that zl_decode_attn_mla needs (host function,
 * as above).  Returns 0 for invalid sizes.
 */
ZL_API size_t zl_decode_attn_mla_workspace_size(int batch, int num_q_heads, int kv_lora_rank,
                                         int rope_dim, int max_seqlen_k, int dtype);

/*
 * Absorbed multi-head latent attention decode (DeepSeek-V2 MLA, which the
 * ZhiLight pages list as natively supported: first page, sections "技术架构"
 * (flash_mla) and "功能生态"; second page, section "Dual streams, host
 * all-reduce and the memory model").  Every query head attends over one shared
 * latent row per token; the query is already multiplied into latent space
 * (its first kv_lora_rank values) and carries its rotary part in the last
 * rope_dim values; the value is the first kv_lora_rank columns of the same
 * row, and the output stays in latent space (the up-projection is applied
 * after this call).  It is the operation of the file header with one
 * key/value head, K = row[0 : rank+rope], V = row[0 : rank].
 *   q          [batch, num_q_heads, kv_lora_rank + rope_dim]  dtype
 *   kv_cache   [total_tokens, kv_lora_rank + rope_dim]        dtype (NULL only if
 *              every sequence is empty)
 *   cu_seqlens [batch + 1] int32 (device)
 *   kv_lora_rank == 512 and rope_dim == 64 (else ZL_ERR_UNSUPPORTED),
 *   1 <= num_q_heads, num_q_heads <= 16 or a multiple of 16,
 *   out        [batch, num_q_heads, kv_lora_rank] dtype
 *   lse        [batch, num_q_heads] float32 or NULL
 *   workspace  as for zl_decode_attn_gqa, sized by
 *              zl_decode_attn_mla_workspace_size
 */
ZL_API zl_status_t zl_decode_attn_mla(const void *q, const void *kv_cache, const int32_t *cu_seqlens,
                               int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                               int max_seqlen_k, float softmax_scale, int dtype,
                               void *out, float *lse, void *workspace, size_t workspace_bytes,
                               zl_stream_t stream);

/*
 * Log-sum-exp combine of split partial results (the merge step that makes
 * split-KV "flash decoding" exact; the first page names flash_decoding among
 * the engine's third-party kernels, section "技术架构").  Each split s holds
 * the attention result of a disjoint subset of one row's tokens:
 *   partial_out [num_splits, rows, head_dim_v] float32, normalised (O_s / l_s)
 *   partial_lse [num_splits, rows] float32, natural log; -inf = empty split
 * with rows = batch * num_heads.  Writes
 *   M = max_s lse_s,  w_s = exp(lse_s - M),
 *   out[r,:] = sum_s w_s O_s / sum_s w_s    (out_dtype, [rows, head_dim_v])
 *   lse[r]   = M + ln(sum_s w_s)           (float32 or NULL)
 * All splits empty -> out = 0, lse = -inf.  1 <= num_splits <= 1024,
 * head_dim_v % 4 == 0, partial buffers 16-byte aligned.
 */
ZL_API zl_status_t zl_attn_combine(const float *partial_out, const float *partial_lse, int num_splits,
                            int batch, int num_heads, int head_dim_v, int out_dtype,
                            void *out, float *lse, zl_stream_t stream);

/*
 * The same two decode calls with an explicit number of workers (the units
 * that split the batch's (kv-head, token) rows evenly; a multiple of 8,
 * 8 .. 65536; 0 = the default for the layout) and the matching workspace
 * sizes.  The result is the same attention for any worker count, up to the
 * fp32 rounding of how tokens are grouped; tests use this to vary the split,
 * and it lets a caller trade split overhead against parallelism.
 * `phases` selects the kernels to enqueue: 1 = the decode kernel only, 2 = the
 * merge kernel only, 3 = both (what the plain entry points do).  Phase 2 must
 * follow phase 1 of the same arguments on the same workspace, stream-ordered;
 * splitting a call lets a caller time or place the two launches separately.
 */
ZL_API size_t zl_decode_attn_workspace_size_ex(int batch, int num_q_heads, int num_kv_heads,
                                        int head_dim, int max_seqlen_k, int dtype,
                                        int num_workers);
ZL_API zl_status_t zl_decode_attn_gqa_ex(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *cu_seqlens, int batch, int num_q_heads,
                                  int num_kv_heads, int head_dim, int max_seqlen_k,
                                  float softmax_scale, int dtype, void *out, float *lse,
                                  int num_workers, int phases, void *workspace,
                                  size_t workspace_bytes, zl_stream_t stream);
ZL_API size_t zl_decode_attn_mla_workspace_size_ex(int batch, int num_q_heads, int kv_lora_rank,
                                            int rope_dim, int max_seqlen_k, int dtype,
                                            int num_workers);
ZL_API zl_status_t zl_decode_attn_mla_ex(const void *q, const void *kv_cache, const int32_t *cu_seqlens,
                                  int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                  int max_seqlen_k, float softmax_scale, int dtype,
                                  void *out, float *lse, int num_workers, int phases,
                                  void *workspace, size_t workspace_bytes, zl_stream_t stream);

/*
 * Paged caches.  Requests that share a prompt prefix can share its key/value
 * rows when the cache is kept in fixed-size pages: the first ZhiLight page
 * lists a prefix cache among the engine's features (section "功能生态") and
 * places it in the C++ runtime's batch generator (section "技术架构"); the
 * second page lists it beside fused batch attention for decoding (section
 * "Dual streams, host all-reduce and the memory model").  The attention is
 * the operation in the file header; only where a token's row lives changes:
 *   token i of sequence b is row (i % page_size) of page
 *   block_table[b * max_pages_per_seq + i / page_size]
 *   k_pages, v_pages [num_pages, page_size, num_kv_heads, head_dim]  dtype
 *   kv_pages         [num_pages, page_size, kv_lora_rank + rope_dim] dtype
 *   block_table      [batch, max_pages_per_seq] int32 (device), every entry a
 *                    sequence uses (i / page_size for i < L_b) is a valid
 *                    page id (precondition)
 *   cu_seqlens       as above: the prefix sums of the sequence lengths (a
 *                    logical numbering; no cache row sits at those indices)
 *   page_size        a power of two, 16 .. 256 (else ZL_ERR_UNSUPPORTED)
 *   max_seqlen_k <= max_pages_per_seq * page_size
 * The workspace is sized by the same functions as for packed caches.  The
 * _ex forms take num_workers and phases as above.
 */
ZL_API zl_status_t zl_decode_attn_gqa_paged(const void *q, const void *k_pages, const void *v_pages,
                                            const int32_t *block_table, int max_pages_per_seq, int page_size,
                                            const int32_t *cu_seqlens, int batch, int num_q_heads,
                                            int num_kv_heads, int head_dim, int max_seqlen_k,
                                            float softmax_scale, int dtype, void *out, float *lse,
                                            void *workspace, size_t workspace_bytes, zl_stream_t stream);
ZL_API zl_status_t zl_decode_attn_gqa_paged_ex(const void *q, const void *k_pages, const void *v_pages,
                                               const int32_t *block_table, int max_pages_per_seq,
                                               int page_size, const int32_t *cu_seqlens, int batch,
                                               int num_q_heads, int num_kv_heads, int head_dim,
                                               int max_seqlen_k, float softmax_scale, int dtype,
                                               void *out, float *lse, int num_workers, int phases,
                                               void *workspace, size_t workspace_bytes, zl_stream_t stream);
ZL_API zl_status_t zl_decode_attn_mla_paged(const void *q, const void *kv_pages, const int32_t *block_table,
                                            int max_pages_per_seq, int page_size, const int32_t *cu_seqlens,
                                            int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                            int max_seqlen_k, float softmax_scale, int dtype,
                                            void *out, float *lse, void *workspace, size_t workspace_bytes,
                                            zl_stream_t stream);
ZL_API zl_status_t zl_decode_attn_mla_paged_ex(const void *q, const void *kv_pages, const int32_t *block_table,
                                               int max_pages_per_seq, int page_size, const int32_t *cu_seqlens,
                                               int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                               int max_seqlen_k, float softmax_scale, int dtype,
                                               void *out, float *lse, int num_workers, int phases,
                                               void *workspace, size_t workspace_bytes, zl_stream_t stream);

/*
 * Several new query tokens per sequence: chunked prefill (the first ZhiLight
 * page lists it among the engine's features, section "功能生态": a long
 * prompt's prefill is split into chunks; the second page lists it beside
 * flash-attention prefill, section "Dual streams, host all-reduce and the
 * memory model"), and several draft tokens checked in one step.  Sequence b
 * has nq = cu_seqlens_q[b+1] - cu_seqlens_q[b] new query tokens, whose keys
 * and values are already the last nq of its lk = cu_seqlens_k[b+1] -
 * cu_seqlens_k[b] cached rows (lk clamped to [0, max_seqlen_k] as above;
 * nq below 0 counts as 0).  New token i (0 <= i < nq) sits at cache
 * position lk - nq + i; with causal = 1 it attends to cache rows
 * 0 .. lk - nq + i (none if that is negative: out 0, lse -inf), with
 * causal = 0 to all lk rows.  Each (token, head) row is the attention in the
 * file header over its visible rows.
 *   q            [total_q, num_q_heads, head_dim]              dtype
 *   k/v_cache    [cu_seqlens_k[batch], num_kv_heads, head_dim]  dtype (GQA)
 *   kv_cache     [cu_seqlens_k[batch], kv_lora_rank + rope_dim] dtype (MLA;
 *                V = the first kv_lora_rank columns)
 *   cu_seqlens_q [batch + 1] int32 (device), cu_seqlens_q[0] = 0,
 *                non-decreasing, cu_seqlens_q[batch] = total_q (precondition)
 *   cu_seqlens_k [batch + 1] int32 (device), as cu_seqlens above
 *   total_q      rows of q (host); 0 is a no-op
 *   out          [total_q, num_q_heads, Dv] dtype;  lse [total_q, num_q_heads]
 * The kernels cut each sequence's (token, head) rows of one key/value head
 * into blocks of R rows (R = 16 for GQA, 32 for MLA) and stream the
 * sequence's rows once per block, so the key/value bytes read are those of a
 * decode step times ceil(nq * group / R).  ZL_ERR_UNSUPPORTED when
 * ceil((total_q * group + (R - 1) * batch) / R) * (max_seqlen_k + C) >= 2^31,
 * C = 32 (GQA) or 64 (MLA).
 * The workspace is sized by zl_decode_attn_workspace_size(_ex) (GQA) or
 * zl_decode_attn_mla_workspace_size(_ex) (MLA) with the same arguments; the
 * _ex forms take num_workers and phases as above.
 */
ZL_API zl_status_t zl_attn_varlen_gqa(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int batch,
                                      int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                      int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                      void *out, float *lse, void *workspace, size_t workspace_bytes,
                                      zl_stream_t stream);
ZL_API zl_status_t zl_attn_varlen_gqa_ex(const void *q, const void *k_cache, const void *v_cache,
                                         const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int batch,
                                         int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                         int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                         void *out, float *lse, int num_workers, int phases, void *workspace,
                                         size_t workspace_bytes, zl_stream_t stream);
ZL_API zl_status_t zl_attn_varlen_mla(const void *q, const void *kv_cache, const int32_t *cu_seqlens_q,
                                      const int32_t *cu_seqlens_k, int batch, int total_q, int num_q_heads,
                                      int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale,
                                      int causal, int dtype, void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, zl_stream_t stream);
ZL_API zl_status_t zl_attn_varlen_mla_ex(const void *q, const void *kv_cache, const int32_t *cu_seqlens_q,
                                         const int32_t *cu_seqlens_k, int batch, int total_q, int num_q_heads,
                                         int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale,
                                         int causal, int dtype, void *out, float *lse, int num_workers,
                                         int phases, void *workspace, size_t workspace_bytes,
                                         zl_stream_t stream);

/*
 * Several new tokens per sequence over paged caches: the prefix cache the
 * ZhiLight pages describe keeps key/value rows in blocks (first page,
 * sections "技术架构" and "功能生态"), and chunked prefill or draft-token
 * verification then attends over those blocks (same sections).  The
 * operation, query/output layouts, mask and checks are those of
 * zl_attn_varlen_gqa / zl_attn_varlen_mla; the caches are page pools as for
 * zl_decode_attn_gqa_paged / zl_decode_attn_mla_paged: row i of sequence b
 * (i < cu_seqlens_k[b+1] - cu_seqlens_k[b]) is row i % page_size of page
 * block_table[b * max_pages_per_seq + i / page_size].  cu_seqlens_k gives
 * only the lengths here (its values are not row indices into the pools).
 * Preconditions as for the paged decode calls (every page id names a page
 * of the pools, max_seqlen_k <= max_pages_per_seq * page_size).  A null
 * cu_seqlens_q or block_table returns ZL_ERR_INVALID_ARGUMENT (the packed or
 * one-token calls serve those cases); every other check and status is that
 * of the varlen and paged calls.  Outputs, lse and workspace are owned by the
 * caller; the call is asynchronous on `stream`.
 */
ZL_API zl_status_t zl_attn_varlen_gqa_paged(const void *q, const void *k_pages, const void *v_pages,
                                            const int32_t *block_table, int max_pages_per_seq, int page_size,
                                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int batch,
                                            int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                            int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                            void *out, float *lse, void *workspace, size_t workspace_bytes,
                                            zl_stream_t stream);
ZL_API zl_status_t zl_attn_varlen_gqa_paged_ex(const void *q, const void *k_pages, const void *v_pages,
                                               const int32_t *block_table, int max_pages_per_seq, int page_size,
                                               const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                               int batch, int total_q, int num_q_heads, int num_kv_heads,
                                               int head_dim, int max_seqlen_k, float softmax_scale, int causal,
                                               int dtype, void *out, float *lse, int num_workers,
                                               int phases, void *workspace, size_t workspace_bytes,
                                               zl_stream_t stream);
ZL_API zl_status_t zl_attn_varlen_mla_paged(const void *q, const void *kv_pages, const int32_t *block_table,
                                            int max_pages_per_seq, int page_size, const int32_t *cu_seqlens_q,
                                            const int32_t *cu_seqlens_k, int batch, int total_q, int num_q_heads,
                                            int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale,
                                            int causal, int dtype, void *out, float *lse, void *workspace,
                                            size_t workspace_bytes, zl_stream_t stream);
ZL_API zl_status_t zl_attn_varlen_mla_paged_ex(const void *q, const void *kv_pages, const int32_t *block_table,
                                               int max_pages_per_seq, int page_size, const int32_t *cu_seqlens_q,
                                               const int32_t *cu_seqlens_k, int batch, int total_q,
                                               int num_q_heads, int kv_lora_rank, int rope_dim, int max_seqlen_k,
                                               float softmax_scale, int causal, int dtype, void *out,
                                               float *lse, int num_workers, int phases, void *workspace,
                                               size_t workspace_bytes, zl_stream_t stream);

/*
 * Long runs of new tokens: prefill and large prefill chunks (the first
 * ZhiLight page lists flash-attention prefill and chunked prefill, sections
 * "技术架构" and "功能生态"; the second page lists them in section "Dual
 * streams, host all-reduce and the memory model").  The operation, layouts and
 * argument checks are those of zl_attn_varlen_gqa; only the kernel differs: it
 * reads every key/value row the block's query rows can see once per 128 query
 * rows of one key/value head (for the causal mask, only the keys up to the
 * block's last token), so it suits many new tokens per sequence; for a few
 * new tokens per sequence zl_attn_varlen_gqa streams fewer bytes.  No
 * workspace.  ZL_ERR_UNSUPPORTED when num_kv_heads *
 * ceil((total_q * group + 127 * batch) / 128) >= 2^31.
 */
ZL_API zl_status_t zl_attn_prefill_gqa(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int batch,
                                       int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                       int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                       void *out, float *lse, zl_stream_t stream);

/*
 * zl_attn_prefill_gqa over page pools: long prompt chunks attending over a
 * prefix cache kept in fixed-size blocks (the first ZhiLight page lists
 * Prefix Cache and chunked prefill among the engine's features, sections
 * "技术架构" and "功能生态"; the second page lists chunked prefill with the
 * paged memory model, section "Dual streams, host all-reduce and the memory
 * model").  Operation, query / output layouts, mask and checks are those of
 * zl_attn_prefill_gqa; the caches are the pools of zl_decode_attn_gqa_paged:
 *   k_pages, v_pages [num_pages, page_size, num_kv_heads, head_dim] dtype;
 *   row i of sequence b (i < its clamped length) is row i % page_size of
 *   page block_table[b * max_pages_per_seq + i / page_size];
 *   cu_seqlens_k gives the cache lengths only (no row indices).
 * page_size a power of two, 16 .. 256 (else ZL_ERR_UNSUPPORTED);
 * max_seqlen_k <= max_pages_per_seq * page_size and a null or unaligned
 * block_table give ZL_ERR_INVALID_ARGUMENT.  Precondition: every table entry
 * a sequence uses names a page of the pools.  No workspace; asynchronous on
 * `stream`.
 */
ZL_API zl_status_t zl_attn_prefill_gqa_paged(const void *q, const void *k_pages, const void *v_pages,
                                             const int32_t *block_table, int max_pages_per_seq, int page_size,
                                             const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int batch,
                                             int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                             int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                             void *out, float *lse, zl_stream_t stream);

/*
 * INT8 coding of an all-reduce payload: the single-GPU half of the INT8
 * all-reduce (the first ZhiLight page, section 1: the all-reduce of tensor
 * parallelism can move INT8 data to cut the bytes between GPUs; the second
 * page, section "Dual streams, host all-reduce and the memory model": an
 * Int8-quantized all-reduce cuts the bytes per collective).  The pages give
 * no scheme; this library codes chunks of `chunk` consecutive elements
 * (256, 512 or 1024, else ZL_ERR_UNSUPPORTED), each with one fp32 scale, 127
 * levels per sign:
 *   amax = max |x| over the chunk,  code = rint(x * (127 / amax)) (ties to
 *   even; 0 when amax = 0),  scale = amax / 127,  value = code * scale
 * in fp32 with every product, sum and quotient rounded on its own (a short
 * last chunk is coded on its own).  The payload values are finite (a NaN or
 * an infinity leaves its chunk's codes and scale unspecified; nothing is
 * read or written out of bounds).  All pointers are device pointers; the
 * 16-bit arrays and the codes must be 16-byte aligned, the scales 4-byte
 * aligned; n == 0 is a no-op.  The collective itself (moving the codes
 * between GPUs) is not part of this library.
 *   zl_int8_quantize:   x [n] dtype -> codes [n] int8, scales [ceil(n/chunk)] fp32
 *   zl_int8_dequantize: codes, scales -> out [n] dtype (value rounded to dtype)
 *   zl_int8_reduce_step: one hop of a ring all-reduce: y = code_in *
 *     scale_in + local (fp32); codes_out/scales_out = y coded again (both or
 *     neither given), sum_out = y rounded to dtype (optional; at least one of
 *     codes_out and sum_out).
 */
ZL_API zl_status_t zl_int8_quantize(const void *x, int dtype, long long n, int chunk, int8_t *codes,
                                    float *scales, zl_stream_t stream);
ZL_API zl_status_t zl_int8_dequantize(const int8_t *codes, const float *scales, long long n, int chunk,
                                      int dtype, void *out, zl_stream_t stream);
ZL_API zl_status_t zl_int8_reduce_step(const int8_t *codes_in, const float *scales_in, const void *local,
                                       int dtype, long long n, int chunk, int8_t *codes_out,
                                       float *scales_out, void *sum_out, zl_stream_t stream);

/*
 * Measurement aid, no attention arithmetic: a plain streaming read of `bytes`
 * of `src` (only whole 1 KB blocks; bytes < 1024 is a no-op) at the launch
 * shape of a decode kernel -- head_dim_k 64 or 128 selects the GQA kernel's
 * shape (one-wave workgroups, 8 or 16 KB items), 576 the MLA kernel's
 * (four-wave workgroups, 36 KB items); other values give ZL_ERR_UNSUPPORTED --
 * with the decode kernels' load path (coalesced 16-byte loads into registers,
 * two items in flight per wave), each workgroup reading an equal contiguous
 * share.  Decode attention is bound by its HBM reads (the first ZhiLight page
 * names HBM traffic as the cost its fused kernels cut, section 3 "自研 Fusion
 * Kernel"), so this read of the same bytes with nothing else to do is the
 * ceiling a decode kernel of that shape is measured against.
 *   src         16-byte aligned device buffer of at least `bytes` bytes
 *   workgroups  0 = the decode kernel's default worker count, else a multiple
 *               of 8 in 8 .. 65536
 *   sink        [workgroups] uint32 (device); gives the loads a use: a word
 *               is written only if a workgroup's checksum of its bytes
 *               equals a fixed key (its contents are meaningless)
 * Asynchronous on `stream`; allocates nothing.
 */
ZL_API zl_status_t zl_hbm_read_probe(const void *src, size_t bytes, int head_dim_k, int workgroups,
                                     uint32_t *sink, zl_stream_t stream);

/* Static, human-readable name of a status code (host).  Takes any int (a
 * zl_status_t value converts to it); values that name no status give
 * "unknown zl_status_t". */
ZL_API const char *zl_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ZL_ATTN_H */
