/*
 * oracle.c -- plain, slow CPU oracle of the DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or load this file;
 * it is used by tests/, by the smoke check and by the benchmark's CPU-baseline leg.
 * It shares no code, header, table or constant with the GPU library.
 *
 * What it computes (the plain definition, in double precision):
 *   1. Lightning indexer   (page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程",
 *      second step "索引器評分": dot products Q.K over a 128-dim key cache, mask and scale,
 *      then multiplied by per-head weights; page "DeepSeek 稀疏注意力路线", "两阶段流程" item 1:
 *      a ReLU-type non-negative activation, then the heads are aggregated):
 *          S[t,s] = scale * sum_j w[t,j] * max(0, sum_i qhat[t,j,i] * khat[b,s,i])   for s < n_t
 *          S[t,s] = -inf                                                            for s >= n_t
 *      with qhat = dec(q) * q_scale[t,j] and khat = dec(k) * k_scale[row] when fp8 scales are given.
 *   2. Top-k selection     (same page, third step "Top-k 選擇", including the special case that a
 *      context no longer than k selects every token): if n_t <= k the set {0..n_t-1}; otherwise the
 *      first k of s in [0,n_t) ordered by (S descending, s ascending).
 *   3. Sparse MLA in MQA form (same page, fourth step "執行稀疏 MLA"; page "DeepSeek-V3.2加速技术详解",
 *      section 3.1 "MHA版MLA VS MQA版MLA": attention is computed on the shared latent vectors and the
 *      value is restored only afterwards): for each head h,
 *          z_j = softmax_scale * sum_{i<Dqk} q[t,h,i] * c[b,I_j,i]
 *          p   = softmax(z)            o[t,h,v] = sum_j p_j c[b,I_j,v]  (v < Dv)
 *          lse = max z + ln sum_j exp(z_j - max z)
 *      over the listed indices I of query t that lie in [0, n_t); other entries (-1 padding) are skipped.
 *
 * Number formats are decoded exactly from their definitions:
 *   bf16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits (the top half of an IEEE binary32).
 *   fp8 e4m3 (OCP "E4M3FN"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at
 *   exponent field 0, no infinities, S.1111.111 is NaN, largest finite magnitude 448.
 *
 * Threads: queries are independent; a pthread pool hands out query numbers, nothing else is split.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };

/* ------------------------------------------------------------------------------------------ */
/* number formats                                                                             */

double orc_bf16_value(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xff;
    int m = bits & 0x7f;
    double v;
    if (e == 0xff) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -126 - 7);               /* subnormal: 0.m * 2^-126 */
    } else {
        v = ldexp(1.0 + (double)m / 128.0, e - 127);  /* normal: 1.m * 2^(e-127) */
    }
    return sign ? -v : v;
}

double orc_e4m3_value(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xf;
    int m = bits & 0x7;
    double v;
    if (e == 0xf && m == 0x7) {
        v = NAN;                                      /* the only NaN encodings; no infinities */
    } else if (e == 0) {
        v = ldexp((double)m, -6 - 3);                 /* subnormal: 0.m * 2^-6 */
    } else {
        v = ldexp(1.0 + (double)m / 8.0, e - 7);      /* normal: 1.m * 2^(e-7) */
    }
    return sign ? -v : v;
}

static double elem_value(const void* base, int dtype, int64_t i) {
    if (dtype == ORC_F32) return (double)((const float*)base)[i];
    if (dtype == ORC_BF16) return orc_bf16_value(((const uint16_t*)base)[i]);
    return orc_e4m3_value(((const uint8_t*)base)[i]);
}

/* Decode n elements of the given format (used by the tests to pin the decoders). */
void orc_decode(const void* src, int dtype, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; i++) dst[i] = elem_value(src, dtype, i);
}

/* ------------------------------------------------------------------------------------------ */
/* token caches: contiguous [B][seq_stride][dim] or paged [pages][page_size][dim]             */

typedef struct {
    const void* data;
    int dtype;
    const float* scale;          /* one value per stored row, or NULL */
    int64_t seq_stride;          /* contiguous: rows between sequences */
    const int32_t* page_table;   /* NULL: contiguous */
    int32_t pt_stride;
    int32_t page_size;
    int32_t dim;
} orc_cache;

/* Storage row that holds token s of sequence b. */
static int64_t cache_row(const orc_cache* c, int32_t b, int64_t s) {
    if (c->page_table == NULL) return (int64_t)b * c->seq_stride + s;
    int64_t page = c->page_table[(int64_t)b * c->pt_stride + s / c->page_size];
    return page * c->page_size + s % c->page_size;
}

/* ------------------------------------------------------------------------------------------ */
/* a minimal pool: worker i takes query numbers i, i+nthreads, ...                             */

typedef struct {
    void (*fn)(void* ctx, int64_t item);
    void* ctx;
    int64_t nitems;
    int nthreads;
    int id;
} orc_job;

static void* orc_worker(void* p) {
    orc_job* j = (orc_job*)p;
    for (int64_t it = j->id; it < j->nitems; it += j->nthreads) j->fn(j->ctx, it);
    return NULL;
}

static void orc_parallel(void (*fn)(void*, int64_t), void* ctx, int64_t nitems, int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    if ((int64_t)nthreads > nitems) nthreads = (int)(nitems > 0 ? nitems : 1);
    pthread_t th[512];
    orc_job jobs[512];
    for (int i = 0; i < nthreads; i++) {
        jobs[i].fn = fn; jobs[i].ctx = ctx; jobs[i].nitems = nitems;
        jobs[i].nthreads = nthreads; jobs[i].id = i;
    }
    for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, orc_worker, &jobs[i]);
    orc_worker(&jobs[0]);
    for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------------------------------ */
/* 1. lightning indexer                                                                       */

typedef struct {
    const void* q; int q_dtype; const float* q_scale; const float* w;
    int32_t H, D;
    orc_cache k;
    const int32_t* q_seq; const int32_t* q_len;
    const int32_t* qsel;
    double scale;
    double* scores; int64_t ld;
} idx_ctx;

static void indexer_one(void* p, int64_t r) {
    idx_ctx* c = (idx_ctx*)p;
    int64_t t = c->qsel ? c->qsel[r] : r;
    int32_t b = c->q_seq[t];
    int64_t n = c->q_len[t];
    int32_t H = c->H, D = c->D;
    double* out = c->scores + r * c->ld;

    /* qhat[j][i] = dec(q[t,j,i]) * q_scale[t,j] */
    double* qh = (double*)malloc(sizeof(double) * (size_t)H * D);
    double* kh = (double*)malloc(sizeof(double) * (size_t)D);
    for (int j = 0; j < H; j++) {
        double qs = c->q_scale ? (double)c->q_scale[t * H + j] : 1.0;
        for (int i = 0; i < D; i++) qh[j * D + i] = elem_value(c->q, c->q_dtype, (t * H + j) * (int64_t)D + i) * qs;
    }
    for (int64_t s = 0; s < c->ld; s++) {
        if (s >= n) { out[s] = -INFINITY; continue; }          /* causal mask */
        int64_t row = cache_row(&c->k, b, s);
        double ks = c->k.scale ? (double)c->k.scale[row] : 1.0;
        for (int i = 0; i < D; i++) kh[i] = elem_value(c->k.data, c->k.dtype, row * D + i) * ks;
        double total = 0.0;
        for (int j = 0; j < H; j++) {
            double dot = 0.0;
            for (int i = 0; i < D; i++) dot += qh[j * D + i] * kh[i];
            double act = dot > 0.0 ? dot : 0.0;                 /* ReLU per head */
            total += (double)c->w[t * H + j] * act;             /* per-head weight, summed over heads */
        }
        out[s] = c->scale * total;
    }
    free(qh);
    free(kh);
}

/* scores: [nsel or T][ld] doubles. Returns 0. */
int orc_indexer(const void* q, int q_dtype, const float* q_scale, const float* w,
                int32_t T, int32_t H, int32_t D,
                const void* k, int k_dtype, const float* k_scale, int64_t k_seq_stride,
                const int32_t* page_table, int32_t pt_stride, int32_t page_size,
                const int32_t* q_seq, const int32_t* q_len,
                const int32_t* qsel, int32_t nsel,
                double scale, double* scores, int64_t ld, int nthreads) {
    idx_ctx c;
    c.q = q; c.q_dtype = q_dtype; c.q_scale = q_scale; c.w = w; c.H = H; c.D = D;
    c.k.data = k; c.k.dtype = k_dtype; c.k.scale = k_scale; c.k.seq_stride = k_seq_stride;
    c.k.page_table = page_table; c.k.pt_stride = pt_stride; c.k.page_size = page_size; c.k.dim = D;
    c.q_seq = q_seq; c.q_len = q_len; c.qsel = qsel; c.scale = scale; c.scores = scores; c.ld = ld;
    orc_parallel(indexer_one, &c, qsel ? nsel : T, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 2. top-k selection                                                                         */

typedef struct { double v; int64_t s; } scored;

/* order: larger score first; equal scores -> lower position first (a total order, so the
   result of the sort does not depend on the sorting algorithm) */
static int by_score_then_pos(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s) ? 1 : 0;
}

typedef struct {
    const double* scores; int64_t ld;
    const int32_t* q_len; const int32_t* rows;
    int32_t k;
    int32_t* idx;
} topk_ctx;

static void topk_one(void* p, int64_t r) {
    topk_ctx* c = (topk_ctx*)p;
    int64_t n = c->q_len[c->rows ? c->rows[r] : r];
    const double* row = c->scores + r * c->ld;
    int32_t* out = c->idx + r * (int64_t)c->k;
    for (int32_t i = 0; i < c->k; i++) out[i] = -1;
    if (n <= c->k) {                          /* short context: every token is selected */
        for (int64_t s = 0; s < n; s++) out[s] = (int32_t)s;
        return;
    }
    scored* all = (scored*)malloc(sizeof(scored) * (size_t)n);
    for (int64_t s = 0; s < n; s++) { all[s].v = row[s]; all[s].s = s; }
    qsort(all, (size_t)n, sizeof(scored), by_score_then_pos);
    for (int32_t i = 0; i < c->k; i++) out[i] = (int32_t)all[i].s;
    free(all);
}

/* scores: [R][ld] doubles, row r belongs to query rows[r] (or r); idx: [R][k], -1 padded. */
int orc_topk(const double* scores, int64_t ld, int32_t R, const int32_t* q_len, const int32_t* rows,
             int32_t k, int32_t* idx, int nthreads) {
    topk_ctx c;
    c.scores = scores; c.ld = ld; c.q_len = q_len; c.rows = rows; c.k = k; c.idx = idx;
    orc_parallel(topk_one, &c, R, nthreads);
    return 0;
}

/* Selection variants (page "DeepSeek-V3.2推理加速引擎深度剖析", closing outlook: a K chosen per
   query, and the sliding-window branch combined with the selection; page "DeepSeek-V3.2加速技术详解",
   the third, sliding-window branch): query t takes its own k_t = clamp(kq[t], 0, k) (k when kq is
   NULL) best positions by the same order (all n_t when n_t <= k_t), and the set union with the W
   most recent positions n_t - W .. n_t - 1; the result is listed in ascending position order,
   -1 padded to k + W entries. */
typedef struct {
    const double* scores; int64_t ld;
    const int32_t* q_len; const int32_t* rows;
    int32_t k; const int32_t* kq; int32_t window;
    int32_t* idx;
} select_ctx;

static void select_one(void* p, int64_t r) {
    select_ctx* c = (select_ctx*)p;
    const int64_t t = c->rows ? c->rows[r] : r;
    const int64_t n = c->q_len[t];
    const int32_t width = c->k + c->window;
    int64_t kt = c->kq ? c->kq[t] : c->k;
    if (kt < 0) kt = 0;
    if (kt > c->k) kt = c->k;
    const double* row = c->scores + r * c->ld;
    int32_t* out = c->idx + r * (int64_t)width;
    char* chosen = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
    if (n <= kt) {
        for (int64_t s = 0; s < n; s++) chosen[s] = 1;
    } else {
        scored* all = (scored*)malloc(sizeof(scored) * (size_t)n);
        for (int64_t s = 0; s < n; s++) { all[s].v = row[s]; all[s].s = s; }
        qsort(all, (size_t)n, sizeof(scored), by_score_then_pos);
        for (int64_t i = 0; i < kt; i++) chosen[all[i].s] = 1;
        free(all);
    }
    for (int64_t s = n - c->window; s < n; s++)
        if (s >= 0) chosen[s] = 1;
    int32_t m = 0;
    for (int64_t s = 0; s < n; s++)
        if (chosen[s]) out[m++] = (int32_t)s;
    for (; m < width; m++) out[m] = -1;
    free(chosen);
}

/* scores: [R][ld] doubles, row r of query rows[r] (or r); kq: [T] or NULL; idx: [R][k + window]. */
int orc_topk_select(const double* scores, int64_t ld, int32_t R, const int32_t* q_len, const int32_t* rows,
                    int32_t k, const int32_t* kq, int32_t window, int32_t* idx, int nthreads) {
    select_ctx c;
    c.scores = scores; c.ld = ld; c.q_len = q_len; c.rows = rows; c.k = k; c.kq = kq; c.window = window; c.idx = idx;
    orc_parallel(select_one, &c, R, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 3. sparse MLA, MQA form                                                                    */

typedef struct {
    const uint16_t* q; int32_t H, Dqk, Dv;
    orc_cache c;
    const int32_t* q_seq; const int32_t* q_len;
    const int32_t* idx; int32_t k;
    const int32_t* qsel;
    double softmax_scale;
    double* out; double* lse;
} mla_ctx;

static void mla_one(void* p, int64_t r) {
    mla_ctx* m = (mla_ctx*)p;
    int64_t t = m->qsel ? m->qsel[r] : r;
    int32_t b = m->q_seq[t];
    int64_t n = m->q_len[t];
    int32_t H = m->H, Dqk = m->Dqk, Dv = m->Dv;
    const int32_t* I = m->idx + r * (int64_t)m->k;

    /* the selected latent rows, decoded once */
    int32_t cnt = 0;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(m->k > 0 ? m->k : 1));
    for (int32_t j = 0; j < m->k; j++)
        if (I[j] >= 0 && I[j] < n) rows[cnt++] = cache_row(&m->c, b, I[j]);
    double* cr = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1) * Dqk);
    for (int32_t j = 0; j < cnt; j++)
        for (int i = 0; i < Dqk; i++) cr[(int64_t)j * Dqk + i] = orc_bf16_value(((const uint16_t*)m->c.data)[rows[j] * Dqk + i]);

    double* z = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
    double* qv = (double*)malloc(sizeof(double) * (size_t)Dqk);
    for (int h = 0; h < H; h++) {
        double* o = m->out + (r * H + h) * (int64_t)Dv;
        for (int v = 0; v < Dv; v++) o[v] = 0.0;
        if (cnt == 0) {                              /* nothing selected: zero output, lse = -inf */
            if (m->lse) m->lse[r * H + h] = -INFINITY;
            continue;
        }
        for (int i = 0; i < Dqk; i++) qv[i] = orc_bf16_value(m->q[(t * H + h) * (int64_t)Dqk + i]);
        double zmax = -INFINITY;
        for (int32_t j = 0; j < cnt; j++) {
            double dot = 0.0;
            for (int i = 0; i < Dqk; i++) dot += qv[i] * cr[(int64_t)j * Dqk + i];
            z[j] = m->softmax_scale * dot;
            if (z[j] > zmax) zmax = z[j];
        }
        double denom = 0.0;
        for (int32_t j = 0; j < cnt; j++) { z[j] = exp(z[j] - zmax); denom += z[j]; }
        for (int32_t j = 0; j < cnt; j++) {
            double pj = z[j] / denom;
            for (int v = 0; v < Dv; v++) o[v] += pj * cr[(int64_t)j * Dqk + v];   /* value = first Dv dims */
        }
        if (m->lse) m->lse[r * H + h] = zmax + log(denom);
    }
    free(rows); free(cr); free(z); free(qv);
}

/* q: bf16 [T][H][Dqk]; latent: bf16 rows of Dqk; idx: [nsel or T][k];
   out: [nsel or T][H][Dv] doubles; lse: [nsel or T][H] doubles or NULL. */
int orc_sparse_mla(const uint16_t* q, int32_t T, int32_t H, int32_t Dqk, int32_t Dv,
                   const uint16_t* latent, int64_t seq_stride,
                   const int32_t* page_table, int32_t pt_stride, int32_t page_size,
                   const int32_t* q_seq, const int32_t* q_len,
                   const int32_t* idx, int32_t k,
                   const int32_t* qsel, int32_t nsel,
                   double softmax_scale, double* out, double* lse, int nthreads) {
    mla_ctx m;
    m.q = q; m.H = H; m.Dqk = Dqk; m.Dv = Dv;
    m.c.data = latent; m.c.dtype = ORC_BF16; m.c.scale = NULL; m.c.seq_stride = seq_stride;
    m.c.page_table = page_table; m.c.pt_stride = pt_stride; m.c.page_size = page_size; m.c.dim = Dqk;
    m.q_seq = q_seq; m.q_len = q_len; m.idx = idx; m.k = k; m.qsel = qsel;
    m.softmax_scale = softmax_scale; m.out = out; m.lse = lse;
    orc_parallel(mla_one, &m, qsel ? nsel : T, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 4. cache write path: rotary position embedding, quantisation and cache append               */
/*
 * Rotary embedding (page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程", first step: the
 * query and key projections carry rotary position information; page "DeepSeek 稀疏注意力路线",
 * section "DeepSeek-V3：MLA 基座", subsection "核心机制（直觉）": MLA's position information travels in a channel
 * of its own, the 64 dims after the 512 latent dims).  The pages give no formula; this is the
 * standard rotation: pair i of the rotated span [off, off + d) of a row at position p turns by the
 * angle p * base^(-2i/d),
 *     x_a' = x_a cos - x_b sin,   x_b' = x_a sin + x_b cos,
 * with the pair (a, b) = (off + 2i, off + 2i + 1) (interleaved) or (off + i, off + i + d/2) (split).
 * Everything is computed in double; each result is then rounded once to binary32 (round to nearest
 * even), and that value is stored:
 *   f32  as is;
 *   bf16 round to nearest, ties to the even code;
 *   fp8  one scale per row (the 1x128 per-token tile of the page on the V3 report), s = max(amax,
 *        1e-12) / 448 in binary32 arithmetic, amax the largest |value| of the row; code = the e4m3
 *        value nearest to x / s (binary32 division), ties to the even code, |x / s| > 448 saturating
 *        to 448; a negative value (or -0) keeps the sign bit.
 */

/* bf16 code nearest to a binary32 value (finite): the two codes around it by truncation of the
   magnitude, then the nearer one, the even one on a tie. */
uint16_t orc_bf16_encode(float x) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint16_t lo = (uint16_t)(bits >> 16), hi = (uint16_t)(lo + 1);   /* same sign, next magnitude */
    double v = (double)x, vl = orc_bf16_value(lo), vh = orc_bf16_value(hi);
    double dl = fabs(v - vl), dh = fabs(vh - v);
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

/* e4m3 code nearest to a value, by search over the 127 finite magnitudes; ties to the even code;
   magnitudes above 448 saturate to 448. */
uint8_t orc_e4m3_encode(double x) {
    const int neg = signbit(x) ? 1 : 0;
    const double a = fabs(x);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7e; c++) {
        const double d = fabs(orc_e4m3_value((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    if (a > 448.0) best = 0x7e;
    return (uint8_t)(neg ? (best | 0x80) : best);
}

/* Rotate a row (values in double) in place at position p. */
static void rope_row(double* x, int width, int64_t p, int off, int d, int interleaved, double base) {
    if (d <= 0) return;
    double* y = (double*)malloc(sizeof(double) * (size_t)width);
    memcpy(y, x, sizeof(double) * (size_t)width);
    for (int i = 0; i < d / 2; i++) {
        const int a = interleaved ? off + 2 * i : off + i;
        const int b = interleaved ? off + 2 * i + 1 : off + i + d / 2;
        const double ang = (double)p * pow(base, -2.0 * i / d);
        const double c = cos(ang), s = sin(ang);
        y[a] = x[a] * c - x[b] * s;
        y[b] = x[a] * s + x[b] * c;
    }
    memcpy(x, y, sizeof(double) * (size_t)width);
    free(y);
}

/* Store a row of binary32 values in dtype at dst (row r of a [rows][width] array); fp8 also
   writes scale[r]. */
static void store_row(const float* v, int width, int dtype, void* dst, int64_t r, float* scale) {
    if (dtype == ORC_F32) {
        memcpy((float*)dst + r * width, v, sizeof(float) * (size_t)width);
    } else if (dtype == ORC_BF16) {
        for (int i = 0; i < width; i++) ((uint16_t*)dst)[r * width + i] = orc_bf16_encode(v[i]);
    } else {
        float amax = 0.0f;
        for (int i = 0; i < width; i++) amax = fmaxf(amax, fabsf(v[i]));
        const float s = fmaxf(amax, 1e-12f) / 448.0f;
        for (int i = 0; i < width; i++) ((uint8_t*)dst)[r * width + i] = orc_e4m3_encode((double)(v[i] / s));
        scale[r] = s;
    }
}

/* Rotate rows in double and round to binary32: x [R][width] in src_dtype (f32 / bf16),
   pos [R] (row r at position pos[r]), out [R][width] floats. */
int orc_rope_rows(const void* x, int src_dtype, int64_t R, int width, const int32_t* pos, int off, int d,
                  int interleaved, double base, float* out) {
    double* row = (double*)malloc(sizeof(double) * (size_t)width);
    for (int64_t r = 0; r < R; r++) {
        for (int i = 0; i < width; i++) row[i] = elem_value(x, src_dtype, r * width + i);
        rope_row(row, width, pos[r], off, d, interleaved, base);
        for (int i = 0; i < width; i++) out[r * width + i] = (float)row[i];
    }
    free(row);
    return 0;
}

/* Rotate and store rows: x [R][width] (f32 / bf16) -> dst [R][width] in dst_dtype (f32 / bf16 /
   fp8 with scale [R]); row r at position pos[r / heads] (heads rows per token). */
int orc_rope_store(const void* x, int src_dtype, int64_t R, int width, int heads, const int32_t* pos,
                   int off, int d, int interleaved, double base, void* dst, int dst_dtype, float* scale) {
    double* row = (double*)malloc(sizeof(double) * (size_t)width);
    float* v = (float*)malloc(sizeof(float) * (size_t)width);
    for (int64_t r = 0; r < R; r++) {
        for (int i = 0; i < width; i++) row[i] = elem_value(x, src_dtype, r * width + i);
        rope_row(row, width, pos[r / heads], off, d, interleaved, base);
        for (int i = 0; i < width; i++) v[i] = (float)row[i];
        store_row(v, width, dst_dtype, dst, r, scale);
    }
    free(row); free(v);
    return 0;
}

/* Append T tokens to a cache: token i of sequence seq[i] at position pos[i] goes to the storage
   row that the cache layout assigns to it (contiguous: seq * seq_stride + pos; paged: through the
   page table), rotated and stored in the cache's dtype.  A token whose sequence is outside
   [0, num_seqs), whose position is negative or past its sequence's rows (contiguous: seq_stride;
   paged: the page table's width), or whose row falls outside [0, num_rows) is not written. */
int orc_cache_append(const void* x, int src_dtype, int32_t T, int width, const int32_t* seq,
                     const int32_t* pos, int32_t num_seqs, int off, int d, int interleaved, double base,
                     void* cache, int cache_dtype, float* cache_scale, int64_t num_rows, int64_t seq_stride,
                     const int32_t* page_table, int32_t pt_stride, int32_t page_size) {
    double* row = (double*)malloc(sizeof(double) * (size_t)width);
    float* v = (float*)malloc(sizeof(float) * (size_t)width);
    for (int32_t i = 0; i < T; i++) {
        const int32_t b = seq[i], p = pos[i];
        if (b < 0 || b >= num_seqs || p < 0) continue;
        int64_t r;
        if (page_table == NULL) {
            if (p >= seq_stride) continue;
            r = (int64_t)b * seq_stride + p;
        } else {
            if (p / page_size >= pt_stride) continue;
            const int64_t page = page_table[(int64_t)b * pt_stride + p / page_size];
            if (page < 0) continue;
            r = page * page_size + p % page_size;
        }
        if (r >= num_rows) continue;
        for (int j = 0; j < width; j++) row[j] = elem_value(x, src_dtype, (int64_t)i * width + j);
        rope_row(row, width, p, off, d, interleaved, base);
        for (int j = 0; j < width; j++) v[j] = (float)row[j];
        store_row(v, width, cache_dtype, cache, r, cache_scale);
    }
    free(row); free(v);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 5. value restore after sparse MLA in MQA form                                              */
/* Page "DeepSeek-V3.2加速技术详解", section 3.1 "MHA版MLA VS MQA版MLA": attention runs on the
   latent vectors and each head's value is restored afterwards:
       out[t][h][n] = sum_{k < 512} o[t][h][k] * W[h][n][k]      (n < dh)
   o: bf16 [T][H][512]; W: bf16 [H][dh][512]; out: doubles [T][H][dh]. */
typedef struct { const uint16_t* o; const uint16_t* w; int32_t H, dh; double* out; } vr_ctx;

static void vr_one(void* p, int64_t t) {
    vr_ctx* c = (vr_ctx*)p;
    double* ov = (double*)malloc(sizeof(double) * 512);
    for (int32_t h = 0; h < c->H; h++) {
        for (int k = 0; k < 512; k++) ov[k] = orc_bf16_value(c->o[(t * c->H + h) * 512 + k]);
        for (int32_t n = 0; n < c->dh; n++) {
            const uint16_t* wr = c->w + ((int64_t)h * c->dh + n) * 512;
            double s = 0.0;
            for (int k = 0; k < 512; k++) s += ov[k] * orc_bf16_value(wr[k]);
            c->out[(t * c->H + h) * (int64_t)c->dh + n] = s;
        }
    }
    free(ov);
}

int orc_value_restore(const uint16_t* o, const uint16_t* w, int32_t T, int32_t H, int32_t dh, double* out,
                      int nthreads) {
    vr_ctx c;
    c.o = o; c.w = w; c.H = H; c.dh = dh; c.out = out;
    orc_parallel(vr_one, &c, T, nthreads);
    return 0;
}
