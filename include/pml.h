/*
 * pml.h - C ABI of the paged MQA-logits library for AMD Instinct MI355X (gfx950).
 *
 * The library scores query rows of DeepSeek-style sparse-attention indexers
 * against an fp8 or MXFP4 key cache and selects the top-k keys per row:
 *
 *     logit[r, s] = sum_h w[r,h] * max(0, scale_k[s] * <q[r,h,:], k[s,:]>)
 *
 * for the key tokens s that row r may see, and -inf for the rest. The calls
 * follow the decode path of the vLLM sparse-attention indexer page
 * ("vllm.model_executor.layers.sparse_attn_indexer", _varlen_decode_rows:
 * get_paged_mqa_logits_metadata -> fp8_fp4_paged_mqa_logits -> top-k
 * selector) and its prefill path (mqa_logits over [ks, ke) bounds).
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless stated otherwise. All buffers are
 *     owned by the caller; the library keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; no call synchronises or allocates memory.
 *   - Every call returns a status (PML_OK = 0). Arguments are validated on
 *     the host before anything is launched; on error nothing is launched.
 *     PML_ERR_HIP means a launch failed; the HIP error stays readable with
 *     hipGetLastError(). Faults inside a kernel surface at the caller's next
 *     synchronisation of `stream`.
 *   - Contracts that depend on device data (lengths within max_ctx, sorted
 *     bounds, ...) are not checked on the host. Where a kernel can detect a
 *     violation cheaply it writes NaN instead of reading out of bounds.
 *   - fp8 means OCP E4M3 ("fn": max 448, no infinity), the native fp8 of gfx950.
 */
#ifndef PML_H
#define PML_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pml_status {
    PML_OK = 0,
    PML_ERR_NULL = 1,          /* a required pointer is NULL                          */
    PML_ERR_SHAPE = 2,         /* unsupported heads / head_dim, or a negative size     */
    PML_ERR_BLOCK_KV = 3,      /* block_kv is not 32 or 64                             */
    PML_ERR_VARLEN_NEXT_N = 4, /* indices given together with next_n != 1              */
    PML_ERR_STRIDE = 5,        /* page stride, table or output leading dim too small   */
    PML_ERR_ALIGN = 6,         /* a pointer or stride breaks the 16-byte alignment     */
    PML_ERR_K = 7,             /* top-k k outside [1, 4096]                           */
    PML_ERR_WORKSPACE = 8,     /* workspace missing or smaller than required           */
    PML_ERR_FORMAT = 9,        /* kv_format is neither PML_KV_FP8 nor PML_KV_MXFP4      */
    PML_ERR_UNSUPPORTED = 10,  /* an argument combination this version does not handle */
    PML_ERR_HIP = 11,          /* a kernel launch failed                               */
    PML_ERR_SCRATCH = 12       /* input larger than the allocation-free call's scratch */
};

/* Key-cache formats (sparse_attn_indexer page, _gather_workspace_shapes and
 * kv_cache_as_quant_view). A page holds block_kv tokens:
 *   PML_KV_FP8:   values [block_kv][D] fp8, then scales [block_kv] fp32
 *                 (little-endian); page_bytes = block_kv * (D + 4).
 *   PML_KV_MXFP4: values [block_kv][D/2] packed e2m1 (element 2i in the low
 *                 nibble of byte i), then scales [block_kv][D/32] e8m0;
 *                 page_bytes = block_kv * (D/2 + D/32). No per-token fp32 scale.
 * Page p starts at kv_cache + p * page_stride_bytes; the stride may exceed
 * page_bytes (a per-layer view into a larger allocation). fp8 per-token
 * scales must be non-negative (they are quantisation scales). */
enum pml_kv_format { PML_KV_FP8 = 0, PML_KV_MXFP4 = 1 };

/* Heads and head dimension this version supports. */
#define PML_HEADS 64
#define PML_HEAD_DIM 128
/* Largest top-k. */
#define PML_MAX_TOPK 4096

/*
 * paged_mqa_logits_metadata - split the paged-logits work over persistent
 * workgroups ("get_paged_mqa_logits_metadata(context_lens, block_kv, num_SMs,
 * indices=)", [Attention][DSA] Route SM100 sparse-indexer decode ... , Purpose
 * and Changes; the schedule has one row per worker plus one, the caller reads
 * the worker count back as schedule.shape[0] - 1, and a row slice gets its own
 * schedule, sparse_attn_indexer page, _varlen_decode_rows).
 *
 *   context_lens     int32. With indices or next_n == 1: [num_rows], the
 *                    tokens each row sees. Otherwise [num_rows / next_n]
 *                    full lengths (row j of entry b sees len[b]-next_n+j+1),
 *                    or, with context_lens_2d, [num_rows / next_n][next_n]
 *                    per-row lengths.
 *   num_rows         flattened query rows (>= 0); a multiple of next_n.
 *   next_n           rows per batch entry when indices is NULL (>= 1).
 *   indices          int32 [num_rows] request id per row, or NULL. Rows with
 *                    equal CONSECUTIVE ids form one group whose key blocks are
 *                    read once for all of them ("[Bugfix][GLM-5.3-Flash] ...",
 *                    Purpose). Grouping changes speed, never the result.
 *                    Requires next_n == 1 (else PML_ERR_VARLEN_NEXT_N).
 *   block_kv         tokens per cache page: 32 or 64 (else PML_ERR_BLOCK_KV).
 *   num_CUs          number of persistent workgroups the logits call will
 *                    launch (1 .. 2^20, else PML_ERR_SHAPE; e.g. 2 per
 *                    compute unit).
 *   schedule         int32 [num_CUs + 1][2] output, 16-B aligned (else
 *                    PML_ERR_ALIGN). The (row-piece, key-block) units, ordered
 *                    by piece then block, are cut into num_CUs ranges of about
 *                    equal cost; entry c < num_CUs is the (first row of its
 *                    row-piece, block offset) where range c starts, and entry
 *                    num_CUs is (num_rows, 0). A row-piece is at most 8
 *                    consecutive rows of one group; a key block is a step of
 *                    max(block_kv, 64) tokens (a 32-token cache is scored two
 *                    pages per step); units are weighted by (4 + rows in the
 *                    piece) so ranges cost about the same.
 *                    The logits calls only read it, so one schedule serves any
 *                    number of calls, concurrent ones included.
 * The schedule is valid only for the same context_lens, indices, next_n,
 * block_kv and num_CUs.
 */
int paged_mqa_logits_metadata(const int32_t *context_lens, int num_rows, int next_n,
                              int context_lens_2d, const int32_t *indices, int block_kv,
                              int num_CUs, int32_t *schedule, void *stream);

/* Rows of [2] int32 entries in the schedule for num_CUs workgroups (host
 * only, no GPU call): num_CUs + 1. -1 when num_CUs is outside 1 .. 2^20. */
int paged_mqa_logits_schedule_rows(int num_CUs);

/*
 * fp8_fp4_paged_mqa_logits - score every visible token of a paged key cache
 * ("fp8_fp4_paged_mqa_logits((q, q_scale), kv_cache, weights, seq_lens,
 * block_table, schedule, max_model_len, indices)", sparse_attn_indexer page,
 * _varlen_decode_rows; FP8 q with its per-token scale folded into weights and
 * FP4 q as a (values, scales) pair, forward_cuda).
 *
 *   q                16-B aligned. With q_scale NULL: fp8 codes
 *                    [num_rows][num_heads][head_dim]. With q_scale: packed
 *                    e2m1 values [num_rows][num_heads][head_dim / 2], element
 *                    2i in the low nibble of byte i (the MXFP4 key layout
 *                    applied to q, this library's reading of the FP4 pair).
 *   q_scale          NULL (fp8 q), or e8m0 [num_rows][num_heads][head_dim / 32],
 *                    one per 32 consecutive elements, 16-B aligned (else
 *                    PML_ERR_ALIGN); requires kv_format PML_KV_MXFP4 (else
 *                    PML_ERR_UNSUPPORTED).
 *   num_rows, next_n, context_lens, context_lens_2d, indices
 *                    as for the metadata call (same values it was given).
 *   num_heads        must be 64; head_dim must be 128 (else PML_ERR_SHAPE).
 *   kv_cache         paged key cache, 16-B aligned; kv_format PML_KV_FP8 or
 *                    PML_KV_MXFP4; block_kv 32 or 64.
 *   page_stride_bytes >= page bytes and a multiple of 16 (else PML_ERR_STRIDE).
 *   num_pages        pages in kv_cache (>= 1). A visible block whose table
 *                    entry is outside [0, num_pages) scores NaN.
 *   weights          fp32 [num_rows][num_heads].
 *   block_table      int32 [table rows][block_table_ld]; row r reads table row
 *                    r / next_n (with indices: its own row, and rows of one
 *                    group must hold the same entries). Entries of blocks a
 *                    row does not see are never used (a few past a row's last
 *                    visible block may be read ahead, within block_table_cols).
 *                    block_table_cols (<= ld) bounds the block index; beyond it
 *                    a block scores NaN.
 *   schedule, num_CUs the metadata call's output (read only) and its num_CUs
 *                    (schedule 16-B aligned); the kernel launches num_CUs
 *                    workgroups, workgroup c scoring schedule range c.
 *   max_ctx          output columns (>= every visible length).
 *   logits           fp32 [num_rows][logits_ld] output, 16-B aligned,
 *                    logits_ld >= max_ctx and a multiple of 4. Columns
 *                    [0, vis(r)) get the score, [vis(r), max_ctx) get -inf,
 *                    [max_ctx, logits_ld) are not written.
 *   workspace        device scratch of at least
 *                    fp8_fp4_paged_mqa_logits_workspace_size(num_rows, num_CUs)
 *                    bytes, 256-B aligned (else PML_ERR_WORKSPACE /
 *                    PML_ERR_ALIGN). Its contents need no initialisation and
 *                    are garbage afterwards. Calls that run at the same time
 *                    need separate workspaces (they may share the schedule).
 *                    The call first writes, per row, u = sum_h w[h] q[h] as
 *                    four scaled fp8 pieces into it (codes [num_rows][4][128],
 *                    then e8m0 scales [num_rows][4][4]): the scores' linear
 *                    half, sum_h w_h <q_h, k>, runs on the matrix core as
 *                    <u, k>.
 */
size_t fp8_fp4_paged_mqa_logits_workspace_size(int num_rows, int num_CUs);
int fp8_fp4_paged_mqa_logits(const void *q, const uint8_t *q_scale, int num_rows, int next_n,
                             int num_heads, int head_dim, const void *kv_cache, int kv_format,
                             int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                             const float *weights, const int32_t *context_lens, int context_lens_2d,
                             const int32_t *block_table, int64_t block_table_ld,
                             int block_table_cols, const int32_t *schedule, int num_CUs,
                             const int32_t *indices, int max_ctx, float *logits, int64_t logits_ld,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * mqa_logits - non-paged (ragged prefill) logits: a dense [M][N] matrix whose
 * row r is scored on keys [cu_seqlen_ks[r], cu_seqlen_ke[r]) and -inf
 * elsewhere (sparse_attn_indexer page: the dense M*N logits tensor that
 * prefill chunking bounds, and forward_cpu's per-row lengths ke - ks).
 *
 *   q        fp8 codes [M][num_heads][head_dim], 16-B aligned.
 *   k        fp8 codes [N][head_dim] contiguous keys, 16-B aligned.
 *   k_scale  fp32 [N] per-key scale (non-negative), 4-B aligned.
 *   weights  fp32 [M][num_heads], 16-B aligned.
 *   cu_seqlen_ks, cu_seqlen_ke  int32 [M]; bounds are clamped to [0, N].
 *   logits   fp32 [M][logits_ld], logits_ld >= N, a multiple of 4, 16-B aligned.
 *            Columns [0, N) of every row are written; [N, logits_ld) are not.
 * M <= 524280 and N <= 2^31 - 257 (else PML_ERR_SHAPE). M == 0 or N == 0
 * returns PML_OK and launches nothing.
 */
int mqa_logits(const void *q, int M, int num_heads, int head_dim, const void *k,
               const float *k_scale, int N, const float *weights, const int32_t *cu_seqlen_ks,
               const int32_t *cu_seqlen_ke, float *logits, int64_t logits_ld, void *stream);

/*
 * top_k_per_row - the k largest logits of each row among its valid columns
 * (the indexer's top-k selector, "selector(logits, seq_lens, next_n, out,
 * topk_tokens, max_seq_len)", sparse_attn_indexer page, _varlen_decode_rows;
 * int32 output preset to -1 and request-local positions, forward_cpu).
 *
 *   logits     fp32 [num_rows][logits_ld], 16-B aligned, logits_ld a multiple
 *              of 4 (else PML_ERR_ALIGN / PML_ERR_STRIDE), as the logits calls
 *              write them.
 *   ks         int32 [num_rows] first valid column per row, or NULL (= 0).
 *   ke         int32 end of the valid columns: [num_rows] when next_n == 1 or
 *              ks != NULL; else [num_rows / next_n] full lengths and row j of
 *              entry b ends at ke[b] - next_n + j + 1. Bounds are clamped to
 *              [0, logits_ld].
 *   next_n     >= 1; must be 1 when ks is given.
 *   k          1..4096 (else PML_ERR_K).
 *   max_width  upper bound of ke - ks over all rows (the selector's
 *              max_seq_len). With max_width <= 8192 every row takes a variant
 *              that keeps the whole row in registers. Wider rows are an error
 *              of the caller and are cut to max_width.
 *   out        int32 [num_rows][out_ld], out_ld >= k: per row the selected
 *              positions minus ks in ascending order, then -1 up to k.
 *              Order of selection: larger value first, equal values by lower
 *              position (-0.0 equals +0.0).
 *   workspace  device scratch of at least top_k_per_row_workspace_size()
 *              bytes, 16-B aligned (may be NULL when that size is 0; this
 *              version needs none).
 */
size_t top_k_per_row_workspace_size(int num_rows, int max_width, int k);
int top_k_per_row(const float *logits, int num_rows, int64_t logits_ld, const int32_t *ks,
                  const int32_t *ke, int next_n, int k, int max_width, int32_t *out,
                  int64_t out_ld, void *workspace, size_t workspace_bytes, void *stream);

/*
 * top_k_per_row_bf16 - top_k_per_row over bf16 logits (as
 * fp8_fp4_paged_mqa_logits_bf16 writes them; the SM100 kernel's logits dtype,
 * sparse_attn_indexer page, the logits buffer of _varlen_decode_rows), with no
 * fp32 copy in between.
 *
 *   logits     bf16 bits [num_rows][logits_ld] (uint16_t), 16-B aligned,
 *              logits_ld a multiple of 8 (else PML_ERR_ALIGN /
 *              PML_ERR_STRIDE).
 *
 * Every other argument, check and result is as for top_k_per_row: the
 * selection is that of top_k_per_row over the exact fp32 values of the bf16
 * logits (as_fp32_logits), bit for bit.
 */
int top_k_per_row_bf16(const uint16_t *logits, int num_rows, int64_t logits_ld, const int32_t *ks,
                       const int32_t *ke, int next_n, int k, int max_width, int32_t *out,
                       int64_t out_ld, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp8_fp4_paged_mqa_logits_noalloc - fp8_fp4_paged_mqa_logits without the
 * workspace arguments, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it). The
 * call's scratch is a static array in device memory, one per GPU, held until
 * the process ends; this call allocates nothing. Limits: num_rows <= 4096 and
 * num_CUs <= 4096 (else PML_ERR_SCRATCH, nothing launched). All calls on one
 * GPU share the array, so calls that overlap on one GPU (on different streams)
 * race; calls in stream order do not. Every other argument, check and result
 * is as for fp8_fp4_paged_mqa_logits.
 */
int fp8_fp4_paged_mqa_logits_noalloc(const void *q, const uint8_t *q_scale, int num_rows, int next_n,
                                     int num_heads, int head_dim, const void *kv_cache, int kv_format,
                                     int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                     const float *weights, const int32_t *context_lens,
                                     int context_lens_2d, const int32_t *block_table,
                                     int64_t block_table_ld, int block_table_cols,
                                     const int32_t *schedule, int num_CUs, const int32_t *indices,
                                     int max_ctx, float *logits, int64_t logits_ld, void *stream);

/*
 * fp8_fp4_paged_mqa_logits_bf16 - the same call as fp8_fp4_paged_mqa_logits
 * with fp8 q (no q_scale argument), writing bf16 logits (the SM100 kernel's
 * output type; sparse_attn_indexer page, as_fp32_logits and
 * _varlen_decode_rows). Every argument means what it means there, except:
 *   logits     bf16 bits [num_rows][logits_ld] (uint16_t), 16-B aligned;
 *              logits_ld >= max_ctx and a multiple of 8 (else
 *              PML_ERR_STRIDE). Each value is the fp32 logit rounded to the
 *              nearest bf16, ties to even; -inf stays -inf (0xff80), NaN stays
 *              a NaN.
 * The scores are computed exactly as in the fp32 call; only the store differs,
 * so the bf16 output equals the fp32 output rounded to bf16, bit for bit.
 */
int fp8_fp4_paged_mqa_logits_bf16(const void *q, int num_rows, int next_n, int num_heads,
                                  int head_dim, const void *kv_cache, int kv_format,
                                  int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                  const float *weights, const int32_t *context_lens,
                                  int context_lens_2d, const int32_t *block_table,
                                  int64_t block_table_ld, int block_table_cols,
                                  const int32_t *schedule, int num_CUs,
                                  const int32_t *indices, int max_ctx, uint16_t *logits,
                                  int64_t logits_ld, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * fp8_fp4_paged_mqa_logits_fp4q - fp8_fp4_paged_mqa_logits with the fp4 q
 * pair required (q_scales NULL with rows is PML_ERR_NULL); a thin alias.
 */
int fp8_fp4_paged_mqa_logits_fp4q(const uint8_t *q_values, const uint8_t *q_scales, int num_rows,
                                  int next_n, int num_heads, int head_dim, const void *kv_cache,
                                  int kv_format, int block_kv, int64_t page_stride_bytes,
                                  int64_t num_pages, const float *weights,
                                  const int32_t *context_lens, int context_lens_2d,
                                  const int32_t *block_table, int64_t block_table_ld,
                                  int block_table_cols, const int32_t *schedule, int num_CUs,
                                  const int32_t *indices, int max_ctx, float *logits,
                                  int64_t logits_ld, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * fp8_fp4_paged_mqa_logits_topk - the paged logits and their per-row top-k in
 * one call, the top-k taken from candidates the logits kernel keeps instead of
 * a second full pass over the rows (the indexer page names a fused prefill
 * top-k and bounds the logits it materialises: sparse_attn_indexer page,
 * _decode_chunk_ranges; the fused form here is this library's). The first
 * arguments through logits_ld mean what they mean for
 * fp8_fp4_paged_mqa_logits (fp8 q), and the fp32 logits are written as that
 * call writes them. Then:
 *   k          1..4096 (else PML_ERR_K).
 *   topk       int32 [num_rows][topk_ld], topk_ld >= k: what top_k_per_row
 *              writes for these logits with ke = the rows' visible lengths
 *              (context_lens read as for the logits) and max_width = max_ctx,
 *              bit for bit.
 *   workspace  device scratch of at least
 *              fp8_fp4_paged_mqa_logits_topk_workspace_size(num_rows, max_ctx,
 *              block_kv, k, num_CUs) bytes, 256-B aligned (else
 *              PML_ERR_WORKSPACE / PML_ERR_ALIGN). Its contents need no
 *              initialisation and are garbage afterwards. Layout: the logits
 *              call's workspace, then, each region 256-B aligned: thresholds
 *              fp32 [num_rows], widths int32 [num_rows], done flags int32
 *              [num_rows], candidate counts int32 [num_rows][nb], then
 *              candidate lists fp32 [num_rows][nb * S][2], with
 *              S = max(block_kv, 64) tokens per step and nb = ceil(max_ctx / S).
 * How: a first kernel scores an evenly spaced sample of each wide row's blocks
 * and sets a threshold that about 2k of the row's columns are expected to
 * reach (rows of at most 4k columns take every finite logit). The logits
 * kernel also writes, per row and key block, the columns at or above the
 * threshold. A selection kernel takes the k best of a row's candidates when
 * there are k to 4k of them; every other row goes through the full top-k over
 * the written logits, so the result is exact for any data.
 */
size_t fp8_fp4_paged_mqa_logits_topk_workspace_size(int num_rows, int max_ctx, int block_kv, int k,
                                                     int num_CUs);
int fp8_fp4_paged_mqa_logits_topk(const void *q, int num_rows, int next_n, int num_heads,
                                  int head_dim, const void *kv_cache, int kv_format,
                                  int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                  const float *weights, const int32_t *context_lens,
                                  int context_lens_2d, const int32_t *block_table,
                                  int64_t block_table_ld, int block_table_cols,
                                  const int32_t *schedule, int num_CUs,
                                  const int32_t *indices, int max_ctx, float *logits,
                                  int64_t logits_ld, int k, int32_t *topk, int64_t topk_ld,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * as_fp32_logits - fp32 copy of bf16 logits over each row's valid span, for
 * the fp32 top-k (sparse_attn_indexer page, as_fp32_logits: only columns below
 * the row's end are converted, and the row stride is kept).
 *   logits     bf16 bits [num_rows][logits_ld], 16-B aligned, logits_ld a
 *              multiple of 8 and >= cols.
 *   cols       the logits width (max_ctx), at most 134215680 (65535 chunks of
 *              2048 columns; else PML_ERR_SHAPE); row ends are clamped to
 *              [0, cols].
 *   row_ends   int32 [num_rows].
 *   out        fp32 [num_rows][out_ld], 16-B aligned, out_ld a multiple of 4
 *              and >= cols. Columns [0, row_end) receive the exact fp32 value
 *              of each bf16 (the bits shifted up by 16); the other columns are
 *              not written.
 */
int as_fp32_logits(const uint16_t *logits, int num_rows, int64_t logits_ld, int cols,
                   const int32_t *row_ends, float *out, int64_t out_ld, void *stream);

/*
 * Exact top-k over key tokens sharded across decode-context-parallel ranks
 * ("vllm.model_executor.layers.sparse_attn_indexer", _merge_dcp_topk_global:
 * each rank packs its local top-k as (score, global token id) float32 pairs,
 * the ranks all-gather them along the leading dimension, and a stable top-k
 * over the gathered pairs gives the global top-k). The merge loses nothing: a
 * token of the global top-k has fewer than k tokens ahead of it overall, hence
 * fewer than k on its own rank, so it is in that rank's local top-k.
 *
 * Token placement: runs of `interleave` consecutive tokens of a request go to
 * ranks 0, 1, ..., world - 1 in turn, so local position p of rank r holds
 * global token (p / interleave) * world * interleave + r * interleave
 * + p % interleave. (The page names only the interleave size; this is the
 * library's reading of it.)
 *
 * pack_dcp_topk_candidates - one rank's pairs from its local top-k.
 *   logits      fp32 [num_rows][logits_ld]: this rank's logits.
 *   row_starts  int32 [num_rows] column of each row's local position 0, or
 *               NULL (= 0); clamped to [0, logits_ld] as in top_k_per_row.
 *   topk        int32 [num_rows][topk_ld], topk_ld >= k: local positions as
 *               top_k_per_row writes them (relative to row_starts, -1 padded).
 *   rank, world 0 <= rank < world; interleave >= 1.
 *   packed      fp32 [num_rows][k][2], 8-B aligned: for slot j with local
 *               position p, 0 <= p < logits_ld - row_start, the pair
 *               (logits[row][row_start + p], global id of p as a float);
 *               any other entry packs as (-inf, -1).
 *   Ids must stay exact in float32: PML_ERR_SHAPE when the global id of local
 *   position logits_ld - 1 reaches 2^24. k in [1, 4096] (else PML_ERR_K).
 *
 * stable_topk_from_gathered_candidates - the merge.
 *   gathered    fp32 [world][num_rows][k][2], 8-B aligned, rank-major as the
 *               all-gather leaves it. A pair is a candidate when its id field
 *               f has 0 <= f < 2^24; its id is f truncated. Candidate ids of a
 *               row must be distinct (otherwise which duplicates are kept is
 *               unspecified; at most k ids are still written).
 *   k           [1, 4096] (else PML_ERR_K); world * k <= 32768 (else
 *               PML_ERR_SHAPE).
 *   out         int32 [num_rows][out_ld], out_ld >= k: per row the ids of the
 *               k best candidates in ascending order, then -1 when the row has
 *               fewer than k. Order of selection: larger score first (NaN after
 *               every number, -0.0 equal to +0.0), equal scores by lower id --
 *               the order of top_k_per_row, so with the placement above the
 *               merge of every rank's packed top_k_per_row output equals
 *               top_k_per_row over the unsharded row.
 */
int pack_dcp_topk_candidates(const float *logits, int num_rows, int64_t logits_ld,
                             const int32_t *row_starts, const int32_t *topk, int64_t topk_ld,
                             int k, int rank, int world, int interleave, float *packed,
                             void *stream);
int stable_topk_from_gathered_candidates(const float *gathered, int world, int num_rows, int k,
                                         int32_t *out, int64_t out_ld, void *stream);

/* Text of a status code (static storage). */
const char *pml_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int pml_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PML_H */
