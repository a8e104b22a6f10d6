// api.hip -- the libdsa C ABI: argument checks, workspace layout, kernel launches.
//
// Every entry point validates its arguments on the host and returns before launching anything when
// they are wrong.  Kernels are enqueued on the caller's stream; nothing here waits for the device.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <cstdarg>
#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

dsa_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return DSA_OK;
    return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxK = 65536;
constexpr int kMaxHeads = 128;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t score_ld(const dsa_batch* b) { return ((int64_t)b->max_len + 63) & ~(int64_t)63; }

constexpr int kMaxSeqs = 65535;
constexpr int kMaxLen = 65535 * 256;

dsa_status check_batch(const dsa_batch* b) {
    if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is NULL");
    if (b->num_queries < 0 || b->num_seqs < 1) return fail(DSA_ERR_INVALID_ARG, "batch: num_queries < 0 or num_seqs < 1");
    if (b->max_len < 0) return fail(DSA_ERR_INVALID_ARG, "batch: max_len < 0");
    // launch grids take one sequence per row of their second or third dimension, and the indexer's
    // 256-position blocks of a row along a second dimension (at most 65535 each)
    if (b->num_seqs > kMaxSeqs) return fail(DSA_ERR_INVALID_ARG, "batch: num_seqs %d > %d", b->num_seqs, kMaxSeqs);
    if (b->max_len > kMaxLen) return fail(DSA_ERR_INVALID_ARG, "batch: max_len %d > %d", b->max_len, kMaxLen);
    if (b->num_queries > 0) {
        if (!b->cu_q || !b->q_seq || !b->q_len) return fail(DSA_ERR_INVALID_ARG, "batch: cu_q / q_seq / q_len is NULL");
        if (b->max_q < 1 || b->max_q > b->num_queries)
            return fail(DSA_ERR_INVALID_ARG, "batch: max_q must be in [1, num_queries]");
    }
    return DSA_OK;
}

dsa_status check_cache(const dsa_cache* c, const dsa_batch* b, int dim, const char* name) {
    if (!c) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!c->data) return fail(DSA_ERR_INVALID_ARG, "%s: data is NULL", name);
    if (c->dim != dim) return fail(DSA_ERR_UNSUPPORTED, "%s: dim %d, expected %d", name, c->dim, dim);
    if (c->dtype != DSA_F32 && c->dtype != DSA_BF16 && c->dtype != DSA_FP8_E4M3)
        return fail(DSA_ERR_INVALID_ARG, "%s: unknown dtype %d", name, c->dtype);
    if (c->num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: num_rows < 0", name);
    if (c->page_table) {
        if (c->page_size < 1) return fail(DSA_ERR_INVALID_ARG, "%s: page_size < 1", name);
        const int64_t need = ((int64_t)b->max_len + c->page_size - 1) / c->page_size;
        if (c->page_table_stride < need)
            return fail(DSA_ERR_INVALID_ARG, "%s: page_table_stride %d < %lld pages for max_len", name,
                        c->page_table_stride, (long long)need);
        if (c->num_rows < c->page_size) return fail(DSA_ERR_INVALID_ARG, "%s: fewer rows than one page", name);
    } else {
        if (c->seq_stride < b->max_len)
            return fail(DSA_ERR_INVALID_ARG, "%s: seq_stride %lld < max_len %d", name, (long long)c->seq_stride,
                        b->max_len);
        if ((int64_t)b->num_seqs * c->seq_stride > c->num_rows)
            return fail(DSA_ERR_INVALID_ARG, "%s: num_seqs * seq_stride exceeds num_rows", name);
    }
    return DSA_OK;
}

dsa::CacheView view(const dsa_cache* c) {
    dsa::CacheView v;
    v.data = c->data;
    v.scale = c->scale;
    v.num_rows = c->num_rows;
    v.seq_stride = c->seq_stride;
    v.page_table = c->page_table;
    v.pt_stride = c->page_table_stride;
    v.page_size = c->page_size > 0 ? c->page_size : 1;
    return v;
}

dsa::BatchView view(const dsa_batch* b) {
    dsa::BatchView v;
    v.T = b->num_queries;
    v.B = b->num_seqs;
    v.cu_q = b->cu_q;
    v.q_seq = b->q_seq;
    v.q_len = b->q_len;
    v.max_len = b->max_len;
    v.max_q = b->max_q;
    return v;
}

dsa_status check_indexer(const void* q, int32_t q_dtype, const float* weights, int32_t n_heads, int32_t head_dim,
                         const dsa_cache* k_cache, const dsa_batch* batch) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if (batch->num_queries > 0 && (!q || !weights)) return fail(DSA_ERR_INVALID_ARG, "indexer: q or weights is NULL");
    if (head_dim != dsa::kIdxDim) return fail(DSA_ERR_UNSUPPORTED, "indexer: head_dim %d (only 128)", head_dim);
    if (n_heads < 1 || n_heads > kMaxHeads) return fail(DSA_ERR_UNSUPPORTED, "indexer: n_heads %d not in [1,128]", n_heads);
    if (q_dtype != DSA_F32 && q_dtype != DSA_BF16 && q_dtype != DSA_FP8_E4M3)
        return fail(DSA_ERR_INVALID_ARG, "indexer: unknown q dtype %d", q_dtype);
    s = check_cache(k_cache, batch, dsa::kIdxDim, "k_cache");
    if (s != DSA_OK) return s;
    if (k_cache->dtype != q_dtype) return fail(DSA_ERR_UNSUPPORTED, "indexer: q and k_cache dtypes differ");
    return DSA_OK;
}

dsa_status check_mla(const void* q, int32_t n_heads, int32_t d_qk, int32_t d_v, const dsa_cache* latent,
                     const dsa_batch* batch, int32_t k, void* out, float softmax_scale) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if (batch->num_queries > 0 && (!q || !out)) return fail(DSA_ERR_INVALID_ARG, "sparse_mla: q or out is NULL");
    if (d_qk != dsa::kDqk || d_v != dsa::kDv)
        return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: d_qk/d_v %d/%d (only 576/512)", d_qk, d_v);
    if (n_heads < 1 || n_heads > kMaxHeads) return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: n_heads %d not in [1,128]", n_heads);
    if (k < 1 || k > kMaxK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, %d]", k, kMaxK);
    s = check_cache(latent, batch, dsa::kDqk, "latent");
    if (s != DSA_OK) return s;
    if (latent->dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: latent cache must be bf16");
    if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY)
        return fail(DSA_ERR_INVALID_ARG, "sparse_mla: softmax_scale must be positive and finite");
    return DSA_OK;
}

dsa_status check_rope(const dsa_rope* r, int width, const char* name, dsa::RopeView& v) {
    v.off = 0; v.dim = 0; v.inter = 1; v.base = 1.0;
    if (!r || r->dim == 0) return DSA_OK;
    if (r->dim < 0 || (r->dim & 1) || r->offset < 0 || r->offset + r->dim > width)
        return fail(DSA_ERR_INVALID_ARG, "%s: span [%d, %d + %d) must be even and inside the row of %d", name,
                    r->offset, r->offset, r->dim, width);
    if (!(r->base > 0.0) || !std::isfinite(r->base)) return fail(DSA_ERR_INVALID_ARG, "%s: base must be positive and finite", name);
    v.off = r->offset; v.dim = r->dim; v.inter = r->interleaved ? 1 : 0; v.base = r->base;
    return DSA_OK;
}

// A cache that the write path fills: layout fields only (the readers' max_len checks do not apply).
dsa_status check_write_cache(const dsa_cache* c, int dim, const char* name) {
    if (!c) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!c->data) return fail(DSA_ERR_INVALID_ARG, "%s: data is NULL", name);
    if (c->dim != dim) return fail(DSA_ERR_UNSUPPORTED, "%s: dim %d, expected %d", name, c->dim, dim);
    if (c->dtype != DSA_F32 && c->dtype != DSA_BF16 && c->dtype != DSA_FP8_E4M3)
        return fail(DSA_ERR_INVALID_ARG, "%s: unknown dtype %d", name, c->dtype);
    if (c->dtype == DSA_FP8_E4M3 && !c->scale) return fail(DSA_ERR_INVALID_ARG, "%s: fp8 cache needs a scale array", name);
    if (c->num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: num_rows < 0", name);
    if (c->page_table) {
        if (c->page_size < 1 || c->page_table_stride < 1)
            return fail(DSA_ERR_INVALID_ARG, "%s: page_size and page_table_stride must be >= 1", name);
    } else if (c->seq_stride < 0) {
        return fail(DSA_ERR_INVALID_ARG, "%s: seq_stride < 0", name);
    }
    return DSA_OK;
}

bool src_dtype_ok(int32_t d) { return d == DSA_F32 || d == DSA_BF16; }

// ---- the forward: argument checks and workspace size, then the launches ----

// The workspace region that the top-k's candidates (unfused or fused first pass) and, after them, the
// MLA split partials share.
size_t forward_shared_bytes(const dsa_batch* batch, int32_t k, int32_t n_heads) {
    const int T = batch->num_queries;
    return std::max(std::max(align256(dsa::mla_workspace_bytes(T, k, n_heads)),
                             align256(dsa::topk_workspace_bytes(view(batch), k))),
                    align256(dsa::indexer_topk_workspace_bound(view(batch), k)));
}

// dsa_indexer_topk's workspace: the fused pass's candidates, or the scores then the top-k's candidates
// (whichever is larger: the dtype and cache layout that decide between them are not known here).
size_t indexer_topk_bytes(const dsa_batch* batch, int32_t k) {
    const int T = batch->num_queries;
    if (T <= 0 || batch->max_len <= k) return 0;
    const size_t unfused = align256((size_t)T * score_ld(batch) * sizeof(float)) +
                           align256(dsa::topk_workspace_bytes(view(batch), k));
    return std::max(unfused, align256(dsa::indexer_topk_workspace_bound(view(batch), k)));
}

// The forward takes the fused indexer -> top-k pass where it measured faster than the unfused one:
// rows longer than one slice, over slices that give a workgroup to every CU, with one or two queries
// per sequence.  (Measured, indexer + top-k: 64 x 131072 229 us fused against 275 us; 64 x 65536 129
// against 148; two queries per sequence at 32 x 65536 104 against 120 paged, 100 against 109
// contiguous; but 16 x 131072 117 against 100: fewer workgroups leave CUs idle that the unfused
// indexer keeps busy.  Rows that fit one slice, split into four at 64 x 32768: the merge of the
// slices' 8192 candidates per row, 14 us, takes back what the fused scoring saves inside the forward.)
bool forward_fuses(int32_t q_idx_dtype, int32_t idx_heads, const dsa_cache* k_cache, const dsa_batch* batch,
                   int32_t k) {
    int ns = 0, slen = 0;
    size_t bytes = 0;
    if (batch->max_q > 2 || !dsa::indexer_topk_rows_exceed_slice(view(batch))) return false;
    if (!dsa::indexer_topk_plan(q_idx_dtype, idx_heads, view(k_cache), view(batch), k, &ns, &slen, &bytes))
        return false;
    return (int64_t)batch->num_seqs * ns >= 256;
}

// Checks the forward's arguments; *need receives the workspace bytes the batch needs.
dsa_status forward_check(const void* q_idx, int32_t q_idx_dtype, const float* weights, int32_t idx_heads,
                         const dsa_cache* k_cache, int32_t k, const void* q, int32_t n_heads, const dsa_cache* latent,
                         float softmax_scale, const dsa_batch* batch, int32_t* indices_out, void* out, size_t* need) {
    dsa_status s = check_mla(q, n_heads, dsa::kDqk, dsa::kDv, latent, batch, k, out, softmax_scale);
    if (s != DSA_OK) return s;
    if (batch->max_len > k) {
        s = check_indexer(q_idx, q_idx_dtype, weights, idx_heads, dsa::kIdxDim, k_cache, batch);
        if (s != DSA_OK) return s;
    }
    const int T = batch->num_queries;
    *need = 0;
    if (T == 0) return DSA_OK;
    const size_t score_bytes = batch->max_len > k ? align256((size_t)T * score_ld(batch) * sizeof(float)) : 0;
    const size_t idx_bytes = indices_out ? 0 : align256((size_t)T * k * sizeof(int32_t));
    *need = score_bytes + idx_bytes + forward_shared_bytes(batch, k, n_heads);
    return DSA_OK;
}

// Indexer (queries with n_t <= k skipped) -> top-k -> sparse MLA on `stream`, with the workspace
// laid out as [scores][indices (unless indices_out)][top-k candidates, later the MLA split partials].
dsa_status forward_launch(const void* q_idx, int32_t q_idx_dtype, const float* q_idx_scale, const float* weights,
                          int32_t idx_heads, const dsa_cache* k_cache, float idx_scale, int32_t k, const void* q,
                          int32_t n_heads, const dsa_cache* latent, float softmax_scale, const dsa_batch* batch,
                          int32_t* indices_out, void* out, float* lse, void* workspace, hipStream_t stream) {
    const int T = batch->num_queries;
    const bool need_scores = batch->max_len > k;
    const int64_t ld = score_ld(batch);
    const size_t score_bytes = need_scores ? align256((size_t)T * ld * sizeof(float)) : 0;
    const size_t idx_bytes = indices_out ? 0 : align256((size_t)T * k * sizeof(int32_t));
    const size_t mla_bytes = dsa::mla_workspace_bytes(T, k, n_heads);
    const size_t topk_bytes = dsa::topk_workspace_bytes(view(batch), k);
    uint8_t* ws = (uint8_t*)workspace;
    float* scores = need_scores ? (float*)ws : nullptr;
    int32_t* idx = indices_out ? indices_out : (int32_t*)(ws + score_bytes);
    void* mla_ws = mla_bytes ? (void*)(ws + score_bytes + idx_bytes) : nullptr;
    void* topk_ws = topk_bytes ? (void*)(ws + score_bytes + idx_bytes) : nullptr;

    const dsa::BatchView bv = view(batch);
    dsa_status s = DSA_OK;
    if (need_scores && forward_fuses(q_idx_dtype, idx_heads, k_cache, batch, k)) {
        s = hip_status(dsa::launch_indexer_topk((const uint8_t*)q_idx, q_idx_scale, weights, idx_heads, view(k_cache),
                                                bv, idx_scale, k, idx, ws + score_bytes + idx_bytes, stream),
                       "forward: fused indexer -> top-k launch");
        if (s != DSA_OK) return s;
        return hip_status(dsa::launch_sparse_mla((const uint16_t*)q, n_heads, view(latent), bv, idx, k, softmax_scale,
                                                 (uint16_t*)out, lse, mla_ws, stream),
                          "forward: sparse_mla launch");
    }
    if (need_scores) {
        s = hip_status(dsa::launch_indexer(q_idx, q_idx_dtype, q_idx_scale, weights, idx_heads, view(k_cache), bv,
                                           idx_scale, scores, ld, k, 0, stream),
                       "forward: indexer launch");
        if (s != DSA_OK) return s;
    }
    s = hip_status(dsa::launch_topk(scores, ld, bv, k, nullptr, 0, idx, topk_ws, topk_bytes, stream),
                   "forward: topk launch");
    if (s != DSA_OK) return s;
    return hip_status(dsa::launch_sparse_mla((const uint16_t*)q, n_heads, view(latent), bv, idx, k, softmax_scale,
                                             (uint16_t*)out, lse, mla_ws, stream),
                      "forward: sparse_mla launch");
}

// ---- the forward's static scratch (dsa_forward_noalloc) ----
//
// One array per GPU, in the library's own device memory (it is allocated when the library's code
// is loaded on a device and held until the process ends), so that dsa_forward_noalloc calls no
// allocator.  In host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and only
// that address is handed to kernels.  Nothing in the forward's workspace has to start at zero
// (every word a kernel reads was written earlier in the same call), so the array is never cleared.
constexpr size_t kScratchBytes = (size_t)96 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

dsa_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "forward_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "forward_noalloc: hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(DSA_ERR_HIP, "forward_noalloc: no device address for the scratch array");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
    switch (s) {
        case DSA_OK: return "ok";
        case DSA_ERR_INVALID_ARG: return "invalid argument";
        case DSA_ERR_UNSUPPORTED: return "unsupported";
        case DSA_ERR_WORKSPACE: return "workspace too small";
        case DSA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* dsa_last_error(void) { return g_err; }

const char* dsa_version(void) { return "libdsa 0.1 (gfx950)"; }

size_t dsa_workspace_size(int32_t op, const dsa_batch* batch, int32_t k, int32_t n_heads, int32_t d_v) {
    (void)d_v;
    if (!batch || batch->num_queries <= 0) return 0;
    const int T = batch->num_queries;
    switch (op) {
        case DSA_OP_INDEXER:
            return 0;
        case DSA_OP_TOPK:
            return k > 0 ? dsa::topk_workspace_bytes(view(batch), k) : 0;
        case DSA_OP_SPARSE_MLA:
            return k > 0 ? dsa::mla_workspace_bytes(T, k, n_heads) : 0;
        case DSA_OP_FORWARD: {
            if (k <= 0) return 0;
            size_t bytes = 0;
            if (batch->max_len > k) bytes += align256((size_t)T * score_ld(batch) * sizeof(float));
            bytes += align256((size_t)T * k * sizeof(int32_t));
            // the top-k candidates and the MLA partials share one region (used one after the other)
            return bytes + forward_shared_bytes(batch, k, n_heads);
        }
        case DSA_OP_INDEXER_TOPK:
            return k > 0 ? indexer_topk_bytes(batch, k) : 0;
    }
    return 0;
}

dsa_status dsa_indexer_scores(const void* q, int32_t q_dtype, const float* q_scale, const float* weights,
                              int32_t n_heads, int32_t head_dim, const dsa_cache* k_cache, const dsa_batch* batch,
                              float scale, float* scores, int64_t ld, hipStream_t stream) {
    dsa_status s = check_indexer(q, q_dtype, weights, n_heads, head_dim, k_cache, batch);
    if (s != DSA_OK) return s;
    if (batch->num_queries > 0 && !scores) return fail(DSA_ERR_INVALID_ARG, "indexer: scores is NULL");
    if (ld < batch->max_len) return fail(DSA_ERR_INVALID_ARG, "indexer: ld %lld < max_len %d", (long long)ld, batch->max_len);
    return hip_status(dsa::launch_indexer(q, q_dtype, q_scale, weights, n_heads, view(k_cache), view(batch), scale,
                                          scores, ld, 0, 1, stream),
                      "indexer launch");
}

dsa_status dsa_indexer_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* weights,
                            int32_t n_heads, int32_t head_dim, const dsa_cache* k_cache, const dsa_batch* batch,
                            float scale, int32_t k, int32_t* indices, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    dsa_status s = check_indexer(q, q_dtype, weights, n_heads, head_dim, k_cache, batch);
    if (s != DSA_OK) return s;
    if (k < 1 || k > kMaxK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, %d]", k, kMaxK);
    if (batch->num_queries > 0 && !indices) return fail(DSA_ERR_INVALID_ARG, "indexer_topk: indices is NULL");
    if (batch->num_queries == 0) return DSA_OK;
    const dsa::BatchView bv = view(batch);
    const dsa::CacheView kc = view(k_cache);
    int ns = 0, slen = 0;
    size_t fbytes = 0;
    if (dsa::indexer_topk_plan(q_dtype, n_heads, kc, bv, k, &ns, &slen, &fbytes)) {
        if (!workspace || workspace_bytes < fbytes)
            return fail(DSA_ERR_WORKSPACE, "indexer_topk: workspace of %zu bytes needed, %zu given", fbytes,
                        workspace_bytes);
        return hip_status(dsa::launch_indexer_topk((const uint8_t*)q, q_scale, weights, n_heads, kc, bv, scale, k,
                                                   indices, workspace, stream),
                          "indexer_topk launch");
    }
    // unfused: the scores of the rows longer than k in the workspace, then the top-k
    const bool need_scores = batch->max_len > k;
    const int64_t ld = score_ld(batch);
    const size_t score_bytes = need_scores ? align256((size_t)batch->num_queries * ld * sizeof(float)) : 0;
    const size_t topk_bytes = dsa::topk_workspace_bytes(bv, k);
    if (score_bytes + topk_bytes > 0 && (!workspace || workspace_bytes < score_bytes + topk_bytes))
        return fail(DSA_ERR_WORKSPACE, "indexer_topk: workspace of %zu bytes needed, %zu given",
                    score_bytes + topk_bytes, workspace_bytes);
    float* scores = need_scores ? (float*)workspace : nullptr;
    if (need_scores) {
        s = hip_status(dsa::launch_indexer(q, q_dtype, q_scale, weights, n_heads, kc, bv, scale, scores, ld, k, 0,
                                           stream),
                       "indexer_topk: indexer launch");
        if (s != DSA_OK) return s;
    }
    return hip_status(dsa::launch_topk(scores, ld, bv, k, nullptr, 0, indices,
                                       topk_bytes ? (uint8_t*)workspace + score_bytes : nullptr, topk_bytes, stream),
                      "indexer_topk: topk launch");
}

dsa_status dsa_topk(const float* scores, int64_t ld, const dsa_batch* batch, int32_t k, int32_t* indices,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if (k < 1 || k > kMaxK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, %d]", k, kMaxK);
    if (batch->num_queries > 0 && (!indices || (!scores && batch->max_len > k)))
        return fail(DSA_ERR_INVALID_ARG, "topk: scores or indices is NULL");
    if (ld < batch->max_len) return fail(DSA_ERR_INVALID_ARG, "topk: ld %lld < max_len %d", (long long)ld, batch->max_len);
    return hip_status(dsa::launch_topk(scores, ld, view(batch), k, nullptr, 0, indices, workspace, workspace_bytes, stream),
                      "topk launch");
}

dsa_status dsa_topk_select(const float* scores, int64_t ld, const dsa_batch* batch, int32_t k,
                           const int32_t* k_per_query, int32_t window, int32_t* indices, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if (k < 1 || k > kMaxK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, %d]", k, kMaxK);
    if (window < 0 || (int64_t)k + window > kMaxK)
        return fail(DSA_ERR_INVALID_ARG, "window %d: must be >= 0 with k + window <= %d", window, kMaxK);
    if (batch->num_queries > 0 && (!scores || !indices))
        return fail(DSA_ERR_INVALID_ARG, "topk_select: scores or indices is NULL");
    if (ld < batch->max_len) return fail(DSA_ERR_INVALID_ARG, "topk_select: ld %lld < max_len %d", (long long)ld, batch->max_len);
    if (batch->num_queries == 0) return DSA_OK;
    return hip_status(dsa::launch_topk(scores, ld, view(batch), k, k_per_query, window, indices, workspace,
                                       workspace_bytes, stream),
                      "topk_select launch");
}

dsa_status dsa_sparse_mla(const void* q, int32_t n_heads, int32_t d_qk, int32_t d_v, const dsa_cache* latent,
                          const dsa_batch* batch, const int32_t* indices, int32_t k, float softmax_scale, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    dsa_status s = check_mla(q, n_heads, d_qk, d_v, latent, batch, k, out, softmax_scale);
    if (s != DSA_OK) return s;
    if (batch->num_queries > 0 && !indices) return fail(DSA_ERR_INVALID_ARG, "sparse_mla: indices is NULL");
    const size_t need = dsa::mla_workspace_bytes(batch->num_queries, k, n_heads);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "sparse_mla: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    return hip_status(dsa::launch_sparse_mla((const uint16_t*)q, n_heads, view(latent), view(batch), indices, k,
                                             softmax_scale, (uint16_t*)out, lse, workspace, stream),
                      "sparse_mla launch");
}

dsa_status dsa_forward(const void* q_idx, int32_t q_idx_dtype, const float* q_idx_scale, const float* weights,
                       int32_t idx_heads, const dsa_cache* k_cache, float idx_scale, int32_t k, const void* q,
                       int32_t n_heads, const dsa_cache* latent, float softmax_scale, const dsa_batch* batch,
                       int32_t* indices_out, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    size_t need = 0;
    dsa_status s = forward_check(q_idx, q_idx_dtype, weights, idx_heads, k_cache, k, q, n_heads, latent,
                                 softmax_scale, batch, indices_out, out, &need);
    if (s != DSA_OK || batch->num_queries == 0) return s;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "forward: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    return forward_launch(q_idx, q_idx_dtype, q_idx_scale, weights, idx_heads, k_cache, idx_scale, k, q, n_heads,
                          latent, softmax_scale, batch, indices_out, out, lse, workspace, stream);
}

dsa_status dsa_forward_noalloc(const void* q_idx, int32_t q_idx_dtype, const float* q_idx_scale,
                               const float* weights, int32_t idx_heads, const dsa_cache* k_cache, float idx_scale,
                               int32_t k, const void* q, int32_t n_heads, const dsa_cache* latent,
                               float softmax_scale, const dsa_batch* batch, int32_t* indices_out, void* out,
                               float* lse, hipStream_t stream) {
    size_t need = 0;
    dsa_status s = forward_check(q_idx, q_idx_dtype, weights, idx_heads, k_cache, k, q, n_heads, latent,
                                 softmax_scale, batch, indices_out, out, &need);
    if (s != DSA_OK || batch->num_queries == 0) return s;
    if (need > kScratchBytes)
        return fail(DSA_ERR_WORKSPACE,
                    "forward_noalloc: this batch needs %zu bytes of scratch, the library's static scratch holds %zu "
                    "(use dsa_forward with a workspace)", need, kScratchBytes);
    void* ws = nullptr;
    s = scratch_on_current_device(&ws);
    if (s != DSA_OK) return s;
    return forward_launch(q_idx, q_idx_dtype, q_idx_scale, weights, idx_heads, k_cache, idx_scale, k, q, n_heads,
                          latent, softmax_scale, batch, indices_out, out, lse, ws, stream);
}

dsa_status dsa_cache_append(const void* k_new, int32_t k_new_dtype, const void* latent_new,
                            int32_t latent_new_dtype, const int32_t* seq, const int32_t* pos,
                            int32_t num_tokens, int32_t num_seqs, const dsa_rope* k_rope,
                            const dsa_rope* latent_rope, const dsa_cache* k_cache,
                            const dsa_cache* latent_cache, hipStream_t stream) {
    if (num_tokens < 0 || num_seqs < 0) return fail(DSA_ERR_INVALID_ARG, "cache_append: num_tokens or num_seqs < 0");
    if (num_tokens > 0 && (!seq || !pos)) return fail(DSA_ERR_INVALID_ARG, "cache_append: seq or pos is NULL");
    dsa::RopeView kr, lr;
    dsa_status s = check_rope(k_rope, dsa::kIdxDim, "k_rope", kr);
    if (s != DSA_OK) return s;
    s = check_rope(latent_rope, dsa::kDqk, "latent_rope", lr);
    if (s != DSA_OK) return s;
    dsa::CacheView kc{}, lc{};
    int kc_dtype = DSA_F32;
    if (k_new) {
        if (!src_dtype_ok(k_new_dtype)) return fail(DSA_ERR_UNSUPPORTED, "cache_append: k_new dtype must be F32 or BF16");
        s = check_write_cache(k_cache, dsa::kIdxDim, "k_cache");
        if (s != DSA_OK) return s;
        kc = view(k_cache);
        kc_dtype = k_cache->dtype;
    }
    if (latent_new) {
        if (!src_dtype_ok(latent_new_dtype))
            return fail(DSA_ERR_UNSUPPORTED, "cache_append: latent_new dtype must be F32 or BF16");
        s = check_write_cache(latent_cache, dsa::kDqk, "latent_cache");
        if (s != DSA_OK) return s;
        if (latent_cache->dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "cache_append: latent cache must be bf16");
        lc = view(latent_cache);
    }
    if (!k_new && !latent_new) return DSA_OK;
    return hip_status(dsa::launch_cache_append(k_new, k_new_dtype, latent_new, latent_new_dtype, seq, pos, num_tokens,
                                               num_seqs, kr, lr, kc, kc_dtype, lc, stream),
                      "cache_append launch");
}

dsa_status dsa_rope_queries(const void* q_idx_in, int32_t q_idx_in_dtype, int32_t idx_heads, void* q_idx_out,
                            int32_t q_idx_out_dtype, float* q_idx_scale_out, const dsa_rope* idx_rope,
                            void* q_mla, int32_t n_heads, const dsa_rope* mla_rope, const int32_t* pos,
                            int32_t num_tokens, hipStream_t stream) {
    if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "rope_queries: num_tokens < 0");
    if (num_tokens > 0 && !pos) return fail(DSA_ERR_INVALID_ARG, "rope_queries: pos is NULL");
    dsa::RopeView ri, rm;
    dsa_status s = check_rope(idx_rope, dsa::kIdxDim, "idx_rope", ri);
    if (s != DSA_OK) return s;
    s = check_rope(mla_rope, dsa::kDqk, "mla_rope", rm);
    if (s != DSA_OK) return s;
    if (q_idx_in) {
        if (!src_dtype_ok(q_idx_in_dtype)) return fail(DSA_ERR_UNSUPPORTED, "rope_queries: q_idx_in dtype must be F32 or BF16");
        if (q_idx_out_dtype != DSA_F32 && q_idx_out_dtype != DSA_BF16 && q_idx_out_dtype != DSA_FP8_E4M3)
            return fail(DSA_ERR_INVALID_ARG, "rope_queries: unknown q_idx_out dtype %d", q_idx_out_dtype);
        if (!q_idx_out) return fail(DSA_ERR_INVALID_ARG, "rope_queries: q_idx_out is NULL");
        if (q_idx_out_dtype == DSA_FP8_E4M3 && !q_idx_scale_out)
            return fail(DSA_ERR_INVALID_ARG, "rope_queries: fp8 output needs q_idx_scale_out");
        if (idx_heads < 1 || idx_heads > kMaxHeads) return fail(DSA_ERR_UNSUPPORTED, "rope_queries: idx_heads %d not in [1,128]", idx_heads);
    }
    if (q_mla && (n_heads < 1 || n_heads > kMaxHeads))
        return fail(DSA_ERR_UNSUPPORTED, "rope_queries: n_heads %d not in [1,128]", n_heads);
    if (!q_idx_in && (!q_mla || rm.dim == 0)) return DSA_OK;
    return hip_status(dsa::launch_rope_queries(q_idx_in, q_idx_in_dtype, q_idx_in ? idx_heads : 0, q_idx_out,
                                               q_idx_out_dtype, q_idx_scale_out, ri, (uint16_t*)q_mla,
                                               q_mla ? n_heads : 0, rm, pos, num_tokens, stream),
                      "rope_queries launch");
}

dsa_status dsa_value_restore(const void* latent_out, const void* w_uv, int32_t num_tokens, int32_t n_heads,
                             int32_t d_h, void* out, hipStream_t stream) {
    if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "value_restore: num_tokens < 0");
    if (n_heads < 1 || n_heads > kMaxHeads) return fail(DSA_ERR_UNSUPPORTED, "value_restore: n_heads %d not in [1,128]", n_heads);
    if (d_h < 128 || d_h > 512 || d_h % 128 != 0)
        return fail(DSA_ERR_UNSUPPORTED, "value_restore: d_h %d must be 128, 256, 384 or 512", d_h);
    if (num_tokens == 0) return DSA_OK;
    if (!latent_out || !w_uv || !out) return fail(DSA_ERR_INVALID_ARG, "value_restore: a pointer is NULL");
    if (((uintptr_t)latent_out | (uintptr_t)w_uv | (uintptr_t)out) & 15)
        return fail(DSA_ERR_INVALID_ARG, "value_restore: pointers must be 16-byte aligned");
    return hip_status(dsa::launch_value_restore((const uint16_t*)latent_out, (const uint16_t*)w_uv, num_tokens, n_heads,
                                                d_h, (uint16_t*)out, stream),
                      "value_restore launch");
}

}  // extern "C"
