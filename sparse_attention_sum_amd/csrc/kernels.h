// kernels.h -- internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace dsa {

struct BatchView {
    int32_t T, B;
    const int32_t* cu_q;
    const int32_t* q_seq;
    const int32_t* q_len;
    int32_t max_len, max_q;
};

// Lightning indexer.  skip_le > 0: queries with n_t <= skip_le need no scores and may be skipped.
// mask != 0: entries [n_t, ld) of every row are written -inf as well (skip_le is then ignored).
hipError_t launch_indexer(const void* q, int dtype, const float* q_scale, const float* w, int H,
                          const CacheView& kc, const BatchView& bv, float scale, float* scores,
                          int64_t ld, int skip_le, int mask, hipStream_t st);

// Top-k per query row (ascending positions, -1 padded), rows of k + window entries: query t's best
// clamp(kq[t], 0, k) positions (k when kq is null) united with its last `window` positions.
// A workspace of topk_workspace_bytes() (0 when not useful) lets long rows go through two passes
// (slices of the row, then a merge of their candidates); without it, one workgroup per row.
size_t topk_workspace_bytes(const BatchView& bv, int k);
// The merge pass alone: each row's selection from the slices' candidates in ws (written by the
// first pass of launch_topk or by the fused indexer -> top-k pass), nslices slices of slice_len.
hipError_t launch_topk_merge(const BatchView& bv, int k, void* ws, int nslices, int slice_len, int32_t* idx,
                             hipStream_t st);

// The lightning indexer fused with the top-k's first pass for long decode rows: fp8 queries and
// keys, 32 or 64 heads, at most two queries per sequence, rows longer than 32768, pages of at least
// 16 tokens.  indexer_topk_plan() tells whether a batch qualifies and how it is sliced (ws bytes in
// *ws_bytes); launch_indexer_topk() then runs the fused pass and the merge, writing idx [T][k].
bool indexer_topk_plan(int dtype, int H, const CacheView& kc, const BatchView& bv, int k, int* nslices,
                       int* slice_len, size_t* ws_bytes);
// true when the batch's rows are longer than one fused slice holds (a merge pass is needed anyway)
bool indexer_topk_rows_exceed_slice(const BatchView& bv);
size_t indexer_topk_workspace_bound(const BatchView& bv, int k);   // the largest plan's bytes
hipError_t launch_indexer_topk(const uint8_t* q, const float* q_scale, const float* w, int H, const CacheView& kc,
                               const BatchView& bv, float scale, int k, int32_t* idx, void* ws, hipStream_t st);
hipError_t launch_topk(const float* scores, int64_t ld, const BatchView& bv, int k, const int32_t* kq, int window,
                       int32_t* idx, void* ws, size_t ws_bytes, hipStream_t st);

// Sparse MLA.  `splits` partitions the k index slots; partial results go to the workspace when
// splits > 1.  mla_splits() is the split count the library uses for a batch.
int mla_splits(int T, int k);
size_t mla_workspace_bytes(int T, int k, int H);
hipError_t launch_sparse_mla(const uint16_t* q, int H, const CacheView& lat, const BatchView& bv,
                             const int32_t* idx, int k, float softmax_scale, uint16_t* out, float* lse,
                             void* ws, hipStream_t st);

// Rotary embedding of the span [off, off + dim) of a row (dim == 0: no rotation); pair i turns by
// position * base^(-2i/dim), pairs (off + 2i, off + 2i + 1) when inter, else (off + i, off + i + dim/2).
struct RopeView {
    int off, dim, inter;
    double base;
};

// Cache write path: rotate, store in the caches' formats and append new tokens (either source may be
// null); rotate the query blocks (indexer out of place, MLA in place on its span).
hipError_t launch_cache_append(const void* k_new, int k_dtype, const void* lat_new, int lat_dtype,
                               const int32_t* seq, const int32_t* pos, int T, int num_seqs, const RopeView& k_rope,
                               const RopeView& lat_rope, const CacheView& kc, int kc_dtype, const CacheView& lc,
                               hipStream_t st);
hipError_t launch_rope_queries(const void* qi_in, int qi_dtype, int Hi, void* qi_out, int qo_dtype, float* qo_scale,
                               const RopeView& ri, uint16_t* qm, int Hm, const RopeView& rm, const int32_t* pos,
                               int T, hipStream_t st);

// Value restore after sparse MLA (MQA form): out[t][h][:dh] = o[t][h][:512] . W[h]^T, W [H][dh][512].
hipError_t launch_value_restore(const uint16_t* o, const uint16_t* w, int T, int H, int dh, uint16_t* out,
                                hipStream_t st);

}  // namespace dsa
