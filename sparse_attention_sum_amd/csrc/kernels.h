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
hipError_t launch_indexer(const void* q, int dtype, const float* q_scale, const float* w, int H,
                          const CacheView& kc, const BatchView& bv, float scale, float* scores,
                          int64_t ld, int skip_le, hipStream_t st);

// Top-k per query row (ascending positions, -1 padded).
hipError_t launch_topk(const float* scores, int64_t ld, const BatchView& bv, int k, int32_t* idx,
                       hipStream_t st);

// Sparse MLA.  `splits` partitions the k index slots; partial results go to the workspace when
// splits > 1.  mla_splits() is the split count the library uses for a batch.
int mla_splits(int T, int k);
size_t mla_workspace_bytes(int T, int k, int H);
hipError_t launch_sparse_mla(const uint16_t* q, int H, const CacheView& lat, const BatchView& bv,
                             const int32_t* idx, int k, float softmax_scale, uint16_t* out, float* lse,
                             void* ws, hipStream_t st);

}  // namespace dsa
