/*
 * dsa.h -- C ABI of libdsa, the DeepSeek Sparse Attention (DSA) hot path for AMD MI355X (gfx950).
 *
 * The path has three steps, each with its own entry point, and one entry point that runs all three:
 *
 *   dsa_indexer_scores  the lightning indexer: for every query token t and every visible past token s
 *                       S[t,s] = scale * k_scale[s] * sum_j w'[t,j] * max(0, q[t,j,:] . k[s,:]),
 *                       w'[t,j] = weights[t,j] * q_scale[t,j]
 *                       (page "一文讀懂DeepSeek-V3.2核心技術DSA", section "DSA 的四步工作流程", the
 *                       indexer-scoring step: Q.K over a small 128-dim key cache, mask and scale, then
 *                       the per-head weights; page "DeepSeek 稀疏注意力路线（V3 / V3.2 / V4）",
 *                       section "两阶段流程", item 1: ReLU-type activation, FP8, heads aggregated).
 *   dsa_topk            per query, the k positions with the largest scores, ties to the lower position;
 *                       every position when the context has at most k tokens (same page, top-k step,
 *                       and its special case that a short context selects everything).
 *   dsa_sparse_mla      attention of every query head over the selected 576-dim latent rows only, in
 *                       MQA form: keys are the whole 576-dim row (512 latent + 64 decoupled-RoPE dims),
 *                       values its first 512 dims (same page, the sparse-MLA step and the 512-dim key
 *                       cache of the second component; page "DeepSeek-V3.2加速技术详解", section 3.1
 *                       "MHA版MLA VS MQA版MLA": the attention runs on the shared latent vectors and the
 *                       value up-projection is applied afterwards, outside this library).
 *   dsa_forward         indexer -> top-k -> sparse MLA; queries whose context is at most k skip the
 *                       indexer and take every position.
 *
 * Conventions shared by every call
 *   - All array pointers are DEVICE pointers unless marked "host"; the structs themselves live in host
 *     memory and are read during the call only.  The caller owns every buffer; the library allocates
 *     no device memory.  Scratch space comes from the caller's `workspace`, sized by
 *     dsa_workspace_size().
 *   - Work is enqueued on `stream` and the call returns without waiting for it.  Buffers must stay
 *     valid until the stream has run the work.
 *   - Argument errors are reported synchronously, before anything is launched, as DSA_ERR_INVALID_ARG
 *     or DSA_ERR_UNSUPPORTED; a failed launch is DSA_ERR_HIP.  dsa_last_error() then holds a
 *     per-thread message.  No C++ exception crosses this interface.
 *   - The library keeps no global mutable state apart from that per-thread message and, for
 *     dsa_forward_noalloc only, its static scratch array and that array's device address per GPU.
 *   - Results are deterministic: the same inputs give bitwise identical outputs.
 *   - Token positions are LOGICAL positions 0..n-1 within a sequence, independent of paging.
 *   - Device-side index data (q_len, q_seq, cu_q, page tables, selected indices) is bounds-checked
 *     where it is used: a length above max_len is read as max_len, a query whose sequence number is out
 *     of range is skipped, a selected index outside [0, n_t) is skipped, and a physical page number
 *     outside [0, num_pages) reads as an all-zero row.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,   /* a pointer, size or layout argument is wrong */
    DSA_ERR_UNSUPPORTED = 2,   /* a valid request the library does not implement */
    DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than dsa_workspace_size() */
    DSA_ERR_HIP = 4            /* the HIP runtime reported an error */
} dsa_status;

typedef enum {
    DSA_F32 = 0,
    DSA_BF16 = 1,
    DSA_FP8_E4M3 = 2           /* OCP e4m3fn: bias 7, no infinities, max 448 */
} dsa_dtype;

/* A per-token cache: either contiguous, token s of sequence b at row b*seq_stride + s, or paged,
 * token s of sequence b at row page_table[b*page_table_stride + s/page_size]*page_size + s%page_size. */
typedef struct {
    const void* data;            /* device, [num_rows][dim] elements of `dtype` */
    const float* scale;          /* device, one float per row (fp8 only), or NULL for all-ones */
    int32_t dtype;               /* dsa_dtype */
    int32_t dim;                 /* elements per row: 128 (indexer keys) or 576 (latent) */
    int64_t num_rows;            /* rows addressable through `data` (used to check the layout) */
    int64_t seq_stride;          /* contiguous layout: rows between consecutive sequences */
    const int32_t* page_table;   /* device [num_seqs][page_table_stride], or NULL for contiguous */
    int32_t page_table_stride;   /* entries per sequence in page_table */
    int32_t page_size;           /* tokens per page (paged layout) */
} dsa_cache;

/* A batch of query tokens grouped by sequence (queries of a sequence are consecutive). */
typedef struct {
    int32_t num_queries;         /* T */
    int32_t num_seqs;            /* B, 1 .. 65535 */
    const int32_t* cu_q;         /* device [B+1]: queries of sequence b are cu_q[b] .. cu_q[b+1]-1 */
    const int32_t* q_seq;        /* device [T]: sequence of each query */
    const int32_t* q_len;        /* device [T]: n_t, query t sees its sequence's tokens 0..n_t-1
                                    (causal; a token sees itself, so in prefill n_t = position + 1) */
    int32_t max_len;             /* host: an upper bound of every n_t (sizes grids and score rows),
                                    at most 65535 * 256 = 16776960 */
    int32_t max_q;               /* host: an upper bound of the queries of one sequence */
} dsa_batch;

/* Lightning-indexer scores.
 *   q        [T][n_heads][head_dim] in q_dtype (F32, BF16 or FP8_E4M3)
 *   q_scale  [T][n_heads] floats (one per 128-wide fp8 row) or NULL for all-ones; must be >= 0
 *   weights  [T][n_heads] floats (any sign)
 *   k_cache  the 128-dim indexer key cache, dtype F32, BF16 or FP8_E4M3 (fp8 scales >= 0)
 *   scale    scalar multiplier of every score
 *   scores   [T][ld] floats, ld >= max_len: every entry of row t is written -- the score for
 *            s < n_t, -inf for n_t <= s < ld (the masked positions of the indexer-scoring step) --
 *            except rows of queries the batch does not reach (a sequence number outside
 *            [0, num_seqs), or a query outside its sequence's cu_q range), which are left untouched
 * head_dim must be 128; q_dtype must equal k_cache->dtype.  (dsa_forward keeps its scores in the
 * workspace and writes no masked entries: the top-k step reads positions s < n_t only.) */
dsa_status dsa_indexer_scores(const void* q, int32_t q_dtype, const float* q_scale, const float* weights,
                              int32_t n_heads, int32_t head_dim, const dsa_cache* k_cache,
                              const dsa_batch* batch, float scale, float* scores, int64_t ld,
                              hipStream_t stream);

/* Top-k positions per query from the score rows.
 *   scores   [T][ld] floats; only entries s < n_t of row t are read
 *   indices  [T][k] int32: the selected positions in ascending order, then -1 padding (n_t < k)
 * Scores are compared as real numbers (+0 == -0); equal scores go to the lower position.  NaN scores
 * are not supported.  workspace may be NULL: then each row is selected by one workgroup.  With a
 * workspace of dsa_workspace_size(DSA_OP_TOPK, ...) bytes (non-zero for rows longer than 32768),
 * long rows go through two passes -- slices of the row each keep their best k (key, position)
 * candidates, then one workgroup per row selects from those -- with the same result. */
dsa_status dsa_topk(const float* scores, int64_t ld, const dsa_batch* batch, int32_t k, int32_t* indices,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The indexer and the top-k step in one call: the selection of dsa_indexer_scores followed by
 * dsa_topk, bit for bit, without handing the scores to the caller (page "DeepSeek 稀疏注意力路线（V3 /
 * V3.2 / V4）", section "两阶段流程", items 1-2: every past token is scored and only the top-k of those
 * scores are kept).  Arguments as in dsa_indexer_scores, plus
 *   k        1 <= k <= 65536
 *   indices  [T][k] int32: the selected positions in ascending order, then -1 padding
 *   workspace  device memory of dsa_workspace_size(DSA_OP_INDEXER_TOPK, ...) bytes
 * When the rows are longer than 32768 positions, the queries are fp8 with 32 or 64 heads, a sequence
 * has at most two queries and pages (if any) hold at least 16 tokens, the scores never leave the chip:
 * each workgroup scores one slice of a sequence's positions into LDS and keeps only the slice's best k
 * as candidates, and a second pass selects each row's k from its slices' candidates; rows of at most
 * 32768 positions (16384 with two queries per sequence) are scored and selected whole by one
 * workgroup.  Otherwise the scores go through the workspace (queries with n_t <= k are not scored:
 * they select every position).  The fused pass pays where its workgroups fill the GPU (e.g. 64
 * sequences at 131072 positions); dsa_forward takes it only there. */
dsa_status dsa_indexer_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* weights,
                            int32_t n_heads, int32_t head_dim, const dsa_cache* k_cache, const dsa_batch* batch,
                            float scale, int32_t k, int32_t* indices, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Selection variants of the top-k step (page "DeepSeek-V3.2推理加速引擎深度剖析", closing outlook:
 * a K chosen per query, and the sliding-window branch combined with the selection; page
 * "DeepSeek-V3.2加速技术详解": the third, sliding-window branch).
 *   k_per_query  device [T] int32, or NULL: query t selects its best min(max(k_per_query[t], 0), k)
 *                positions (k when NULL) by the order of dsa_topk, or all n_t positions when n_t is
 *                not larger
 *   window       W >= 0: the W most recent positions n_t - W .. n_t - 1 join the selection (set union)
 *   indices      [T][k + window] int32: the union in ascending order, then -1 padding; it feeds
 *                dsa_sparse_mla with k + window as its k
 * 1 <= k and k + window <= 65536.  With k_per_query NULL and window 0 this is dsa_topk.  The
 * workspace is used as in dsa_topk (NULL allowed). */
dsa_status dsa_topk_select(const float* scores, int64_t ld, const dsa_batch* batch, int32_t k,
                           const int32_t* k_per_query, int32_t window, int32_t* indices, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Sparse MLA in MQA form over the selected latent rows.
 *   q        [T][n_heads][d_qk] bf16 (d_qk = 576)
 *   latent   the latent cache, BF16, dim 576; values are the first d_v = 512 dims of each row
 *   indices  [T][k] int32 logical positions; entries outside [0, n_t) (e.g. -1 padding) are skipped;
 *            valid entries must be distinct
 *   out      [T][n_heads][d_v] bf16: sum_j softmax_j(softmax_scale * q.c_j) * c_j[:d_v]
 *   lse      [T][n_heads] floats (natural-log log-sum-exp of the scaled logits) or NULL
 * A query with no valid index gets out = 0 and lse = -inf.  1 <= n_heads <= 128; softmax_scale must be
 * positive and finite. */
dsa_status dsa_sparse_mla(const void* q, int32_t n_heads, int32_t d_qk, int32_t d_v, const dsa_cache* latent,
                          const dsa_batch* batch, const int32_t* indices, int32_t k, float softmax_scale,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Indexer -> top-k -> sparse MLA for one batch (arguments as in the three calls above).
 * indices_out may be NULL (the selection then lives in the workspace). */
dsa_status dsa_forward(const void* q_idx, int32_t q_idx_dtype, const float* q_idx_scale,
                       const float* weights, int32_t idx_heads, const dsa_cache* k_cache, float idx_scale,
                       int32_t k,
                       const void* q, int32_t n_heads, const dsa_cache* latent, float softmax_scale,
                       const dsa_batch* batch, int32_t* indices_out, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* dsa_forward for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Arguments as in dsa_forward, without the
 * workspace: the call uses a scratch array of 96 MiB that the library holds in each GPU's memory
 * from the time its code is loaded on that GPU until the process ends, and it calls no allocator.
 * A batch whose dsa_workspace_size(DSA_OP_FORWARD, ...) exceeds 96 MiB is rejected with
 * DSA_ERR_WORKSPACE before anything is launched (64 decode queries fit up to about 96K context each;
 * long prefills do not fit: use dsa_forward there).  Every call on one GPU shares that GPU's array:
 * calls that can overlap on one GPU -- on different streams, or from different threads without
 * ordering -- race and must be serialised by the caller (one stream, or events).  The first call on
 * a device looks up the array's device address (hipGetSymbolAddress) with that device current. */
dsa_status dsa_forward_noalloc(const void* q_idx, int32_t q_idx_dtype, const float* q_idx_scale,
                               const float* weights, int32_t idx_heads, const dsa_cache* k_cache, float idx_scale,
                               int32_t k, const void* q, int32_t n_heads, const dsa_cache* latent,
                               float softmax_scale, const dsa_batch* batch, int32_t* indices_out, void* out,
                               float* lse, hipStream_t stream);

/* Value restore after sparse MLA in MQA form (page "DeepSeek-V3.2加速技术详解", section 3.1
 * "MHA版MLA VS MQA版MLA": attention runs on the shared latent vectors and each head's value is
 * restored only afterwards):
 *     out[t][h][n] = sum_{k < 512} latent_out[t][h][k] * w_uv[h][n][k],   n < d_h
 *   latent_out  [num_tokens][n_heads][512] bf16 (the out of dsa_sparse_mla)
 *   w_uv        [n_heads][d_h][512] bf16: row n of head h holds output dim n's 512 weights
 *   out         [num_tokens][n_heads][d_h] bf16 (fp32 accumulation, round to nearest even)
 * d_h is 128, 256, 384 or 512; 1 <= n_heads <= 128; the three pointers are 16-byte aligned. */
dsa_status dsa_value_restore(const void* latent_out, const void* w_uv, int32_t num_tokens, int32_t n_heads,
                             int32_t d_h, void* out, hipStream_t stream);

/* ---- cache write path -------------------------------------------------------------------------
 * The step before the three above: page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程",
 * first step (the query and key projections carry rotary position information); page "DeepSeek
 * 稀疏注意力路线", section "DeepSeek-V3：MLA 基座", "核心机制（直觉）" (MLA's position information
 * travels in a decoupled channel: the 64 dims after the 512 latent dims of a row) and "两阶段流程"
 * item 1 (the indexer runs in fp8).  The pages give no rotation formula; the standard one is used.
 *
 * Numerics: each rotated value is computed in double (angle, cosine, sine, rotation) and rounded once
 * to binary32; that value is stored as f32, as bf16 (round to nearest even), or as e4m3 with one scale
 * per 128-wide row: s = max(amax, 1e-12) / 448 (binary32), code = e4m3(x / s) rounded to nearest
 * even and saturating at 448.  Elements outside the rotated span are converted the same way. */

/* Rotation of the span [offset, offset + dim) of a row: pair i turns by position * base^(-2i/dim)
 * radians; the pairs are (offset + 2i, offset + 2i + 1) when interleaved, else (offset + i,
 * offset + i + dim/2).  dim == 0 (or a NULL dsa_rope*) turns the rotation off. */
typedef struct {
    int32_t offset;        /* first rotated element of a row */
    int32_t dim;           /* rotated elements, even */
    int32_t interleaved;   /* 1: adjacent pairs; 0: the two halves of the span */
    double base;           /* > 0 and finite */
} dsa_rope;

/* Append num_tokens new tokens to the indexer key cache and to the latent cache.
 *   k_new        [num_tokens][128] F32 or BF16 (un-rotated indexer keys), or NULL (k_cache untouched)
 *   latent_new   [num_tokens][576] F32 or BF16 (un-rotated latent rows), or NULL (latent_cache untouched)
 *   seq, pos     device [num_tokens]: token i is position pos[i] of sequence seq[i]
 *   num_seqs     sequences addressable through the caches (the page tables have num_seqs rows)
 *   k_rope, latent_rope  rotations of the two rows (for DeepSeek-V3.2's latent: offset 512, dim 64)
 *   k_cache      the 128-dim indexer key cache (F32, BF16, or FP8_E4M3 with a writable scale array);
 *   latent_cache the 576-dim BF16 latent cache; the `data` (and fp8 `scale`) arrays of both are WRITTEN
 * Token i goes to the row its layout assigns to (seq[i], pos[i]), rotated at position pos[i].  A token
 * whose sequence is outside [0, num_seqs), whose position is negative or past its sequence's rows
 * (contiguous: seq_stride; paged: page_table_stride pages), whose page number is negative, or whose
 * row is outside [0, num_rows) is not written.  Two tokens of one call must not share a row. */
dsa_status dsa_cache_append(const void* k_new, int32_t k_new_dtype, const void* latent_new,
                            int32_t latent_new_dtype, const int32_t* seq, const int32_t* pos,
                            int32_t num_tokens, int32_t num_seqs, const dsa_rope* k_rope,
                            const dsa_rope* latent_rope, const dsa_cache* k_cache,
                            const dsa_cache* latent_cache, hipStream_t stream);

/* Rotate the query blocks of num_tokens tokens at positions pos (device [num_tokens]).
 *   q_idx_in     [num_tokens][idx_heads][128] F32 or BF16, or NULL (indexer queries skipped)
 *   q_idx_out    [num_tokens][idx_heads][128] in q_idx_out_dtype (F32, BF16 or FP8_E4M3);
 *                for FP8_E4M3, q_idx_scale_out [num_tokens][idx_heads] receives the row scales
 *                (the q_scale of dsa_indexer_scores)
 *   q_mla        [num_tokens][n_heads][576] BF16, rotated IN PLACE on mla_rope's span only, or NULL
 * 1 <= idx_heads, n_heads <= 128.  q_idx_out must not overlap q_idx_in. */
dsa_status dsa_rope_queries(const void* q_idx_in, int32_t q_idx_in_dtype, int32_t idx_heads, void* q_idx_out,
                            int32_t q_idx_out_dtype, float* q_idx_scale_out, const dsa_rope* idx_rope,
                            void* q_mla, int32_t n_heads, const dsa_rope* mla_rope, const int32_t* pos,
                            int32_t num_tokens, hipStream_t stream);

/* Operations for dsa_workspace_size. */
enum { DSA_OP_INDEXER = 0, DSA_OP_TOPK = 1, DSA_OP_SPARSE_MLA = 2, DSA_OP_FORWARD = 3, DSA_OP_INDEXER_TOPK = 4 };

/* Bytes of workspace the operation needs for this batch (0 if none).  For DSA_OP_FORWARD, `k` is the
 * top-k size and indices_out is assumed NULL (the worst case). */
size_t dsa_workspace_size(int32_t op, const dsa_batch* batch, int32_t k, int32_t n_heads, int32_t d_v);

const char* dsa_status_string(dsa_status s);
const char* dsa_last_error(void);   /* message of this thread's last failed call ("" if none) */
const char* dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
