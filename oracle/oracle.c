/*
 * Differential-attention CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, double-precision C.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load this library; the GPU product path
 * never links, calls or reads it, and it shares no code with the GPU sources.
 *
 * What it computes, and where the pages define it:
 *
 *  - Two softmax attention maps over split query/key halves,
 *      A1 = softmax(Q1 K1^T / sqrt(d)),  A2 = softmax(Q2 K2^T / sqrt(d)),
 *    and the differential output (A1 - lambda * A2) V.
 *      Page "差分注意力" (aiknowledge.cn), part 一, subsection "差分思路"
 *      (the three displayed formulas) and part 二, Step 2; page
 *      "Understanding Differential Transformer Unchains Pretrained
 *      Self-Attentions" (Paper-Notes), 方法详解 / 关键设计 (A_diff = A1 - lambda A2).
 *  - The softmax weight of one key, exp(q.k_i/sqrt d) / sum_j exp(q.k_j/sqrt d),
 *    with d the length of the dot product.
 *      Page "差分注意力", part 一, subsection "Softmax 的噪声底".
 *  - lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init, a per-head scalar that
 *    may be negative.
 *      Page "差分注意力", part 一 "差分思路" and part 二 Step 4.
 *  - lambda_init = 0.8 - 0.6 exp(-0.3 (layer - 1)).
 *      Page "【架构革新】Differential Transformer：用“差分降噪”重塑LLM注意力机制"
 *      (mcipr.com), section 3 (engineering practice).
 *  - A per-head RMS normalisation applied after the difference in the V1
 *    layout, and the V2 layout (twice the query heads over unchanged KV heads).
 *      Page "差分注意力", part 一, subsection "V1 到 V2 的 diff".
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes): causal masking means key j is visible to query i iff j <= i;
 * the RMS normalisation is y_c = o_c / sqrt(mean_c o_c^2 + eps) * w_c * s
 * with the scale s = (1 - lambda_init) supplied by the caller; in the V2
 * decode layout, pair p takes query head 2p for A1 and 2p+1 for A2, both over
 * KV head floor(2p / (Hq/Hkv)).
 *
 * Arithmetic: every input element is widened to double exactly (fp32 or the
 * upper 16 bits of an fp32 for bf16); all sums, exponentials and products are
 * done in double in the plain order of the definition: scores, row maximum,
 * exponentials, normaliser, weights, weighted sum of value rows.  The maximum
 * shift inside the softmax is the usual exact identity softmax(x) =
 * softmax(x - c); it changes nothing but overflow behaviour.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_FP32 0
#define ORACLE_BF16 1

/* One element of an fp32 or bf16 array, widened to double without rounding. */
static double elem(const void* base, int dtype, int64_t idx) {
    if (dtype == ORACLE_FP32) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* lambda_init = 0.8 - 0.6 exp(-0.3 (layer - 1)); page "【架构革新】...", section 3. */
double oracle_lambda_init(int layer) {
    return 0.8 - 0.6 * exp(-0.3 * (double)(layer - 1));
}

/*
 * lambda_h = exp(lq1_h . lk1_h) - exp(lq2_h . lk2_h) + lambda_init(layer),
 * page "差分注意力", part 二 Step 4 (re-parameterisation), with lambda_init from
 * the depth schedule.  Inputs are fp32 [H][dim]; each dot product is summed in
 * double in index order (a product of two fp32 values is exact in double), and
 * the double result is rounded once to fp32.
 */
void oracle_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                   int H, int dim, int layer, float* lambda_out) {
    double init = oracle_lambda_init(layer);
    for (int h = 0; h < H; ++h) {
        double d1 = 0.0, d2 = 0.0;
        for (int i = 0; i < dim; ++i) {
            d1 += (double)lq1[(int64_t)h * dim + i] * (double)lk1[(int64_t)h * dim + i];
            d2 += (double)lq2[(int64_t)h * dim + i] * (double)lk2[(int64_t)h * dim + i];
        }
        lambda_out[h] = (float)(exp(d1) - exp(d2) + init);
    }
}

/* ------------------------------------------------------------------------ */
/* One query row of differential attention.                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    int dtype;
    const void *q1, *q2, *k1, *k2, *v;
    int64_t q_off;              /* element offset of this query row in q1/q2 */
    int64_t k_off;              /* element offset of key 0 in k1/k2 */
    int64_t v_off;              /* element offset of value row 0 in v */
    int64_t ldk, ldv;           /* elements between consecutive keys / value rows */
    int nkeys, d, dv;
    double lambda;
} row_job;

/*
 * Scores, both softmax maps, the difference weights and the weighted sum of
 * value rows for one query.  scratch holds 2*nkeys doubles.  If a1/a2 are not
 * NULL they receive the two softmax rows.
 */
static void diff_row(const row_job* r, double* scratch, double* out, double* a1, double* a2) {
    double* s1 = scratch;
    double* s2 = scratch + r->nkeys;
    double inv_sqrt_d = 1.0 / sqrt((double)r->d);
    for (int j = 0; j < r->nkeys; ++j) {
        double dot1 = 0.0, dot2 = 0.0;
        for (int c = 0; c < r->d; ++c) {
            dot1 += elem(r->q1, r->dtype, r->q_off + c) *
                    elem(r->k1, r->dtype, r->k_off + (int64_t)j * r->ldk + c);
            dot2 += elem(r->q2, r->dtype, r->q_off + c) *
                    elem(r->k2, r->dtype, r->k_off + (int64_t)j * r->ldk + c);
        }
        s1[j] = dot1 * inv_sqrt_d;
        s2[j] = dot2 * inv_sqrt_d;
    }
    double m1 = -INFINITY, m2 = -INFINITY;
    for (int j = 0; j < r->nkeys; ++j) {
        if (s1[j] > m1) m1 = s1[j];
        if (s2[j] > m2) m2 = s2[j];
    }
    double z1 = 0.0, z2 = 0.0;
    for (int j = 0; j < r->nkeys; ++j) {
        s1[j] = exp(s1[j] - m1);
        s2[j] = exp(s2[j] - m2);
        z1 += s1[j];
        z2 += s2[j];
    }
    for (int c = 0; c < r->dv; ++c) out[c] = 0.0;
    for (int j = 0; j < r->nkeys; ++j) {
        double w1 = s1[j] / z1;
        double w2 = s2[j] / z2;
        if (a1) a1[j] = w1;
        if (a2) a2[j] = w2;
        double w = w1 - r->lambda * w2;
        for (int c = 0; c < r->dv; ++c)
            out[c] += w * elem(r->v, r->dtype, r->v_off + (int64_t)j * r->ldv + c);
    }
}

/* y_c = o_c / sqrt(mean_c o_c^2 + eps) * w_c * scale (per head, per row). */
static void rms_norm(double* o, int dv, double eps, double scale, const float* weight) {
    double ms = 0.0;
    for (int c = 0; c < dv; ++c) ms += o[c] * o[c];
    ms /= (double)dv;
    double r = 1.0 / sqrt(ms + eps);
    for (int c = 0; c < dv; ++c) o[c] = o[c] * r * (weight ? (double)weight[c] : 1.0) * scale;
}

/* ------------------------------------------------------------------------ */
/* A tiny worker pool: threads pull row indices from a shared counter.        */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t n;
    int64_t next;
    pthread_mutex_t mu;
    void (*fn)(void* ctx, int64_t item, double* scratch);
    void* ctx;
    int64_t scratch_len;
} pool;

static void* pool_worker(void* arg) {
    pool* p = (pool*)arg;
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(p->scratch_len > 0 ? p->scratch_len : 1));
    if (!scratch) return (void*)1;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int64_t item = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (item >= p->n) break;
        p->fn(p->ctx, item, scratch);
    }
    free(scratch);
    return NULL;
}

int oracle_default_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run_pool(int64_t n, int nthreads, int64_t scratch_len,
                    void (*fn)(void*, int64_t, double*), void* ctx) {
    pool p;
    p.n = n;
    p.next = 0;
    p.fn = fn;
    p.ctx = ctx;
    p.scratch_len = scratch_len;
    pthread_mutex_init(&p.mu, NULL);
    if (nthreads <= 0) nthreads = oracle_default_threads();
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tids) return -3;
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, pool_worker, &p) != 0) { rc = -3; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void* ret = NULL;
        pthread_join(tids[t], &ret);
        if (ret) rc = -3;
    }
    free(tids);
    pthread_mutex_destroy(&p.mu);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Prefill: all rows, or a caller-chosen list of rows.                       */
/* ------------------------------------------------------------------------ */

typedef struct {
    int dtype;
    const void *q1, *q2, *k1, *k2, *v;
    int64_t ldq, ldk, ldv;
    int B, H, N, d, dv, causal;
    const float* lambda;
    int rmsnorm;
    double eps, norm_scale;
    const float* norm_weight;
    const int64_t* rows;
    double* out;
} prefill_ctx;

static void prefill_item(void* vctx, int64_t item, double* scratch) {
    const prefill_ctx* c = (const prefill_ctx*)vctx;
    int64_t row = c->rows ? c->rows[item] : item;      /* (b*H + h)*N + i */
    int64_t bh = row / c->N;
    int i = (int)(row % c->N);
    int h = (int)(bh % c->H);
    row_job r;
    r.dtype = c->dtype;
    r.q1 = c->q1; r.q2 = c->q2; r.k1 = c->k1; r.k2 = c->k2; r.v = c->v;
    r.q_off = row * c->ldq;
    r.k_off = bh * (int64_t)c->N * c->ldk;
    r.v_off = bh * (int64_t)c->N * c->ldv;
    r.ldk = c->ldk;
    r.ldv = c->ldv;
    r.nkeys = c->causal ? i + 1 : c->N;
    r.d = c->d;
    r.dv = c->dv;
    r.lambda = (double)c->lambda[h];
    double* o = c->out + item * (int64_t)c->dv;
    diff_row(&r, scratch, o, NULL, NULL);
    if (c->rmsnorm) rms_norm(o, c->dv, c->eps, c->norm_scale, c->norm_weight);
}

/*
 * Differential-attention prefill over [B][H][N] query rows.
 *   q1, q2: [B][H][N][ldq] (a packed [B][H][N][2d] tensor passes q2 = q1 + d)
 *   k1, k2: [B][H][N][ldk], v: [B][H][N][ldv]; element type fp32 or bf16 bits.
 *   lambda: fp32 [H].  rows: NULL for every row in (b,h,i) order, or nrows
 *   flat indices (b*H + h)*N + i.  out: double [nrows][dv].
 * Returns 0, or a negative value for invalid arguments / thread failure.
 */
int oracle_prefill(int dtype, const void* q1, const void* q2, const void* k1, const void* k2,
                   const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                   int B, int H, int N, int d, int dv, int causal, const float* lambda,
                   int rmsnorm, double eps, double norm_scale, const float* norm_weight,
                   const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    if (!q1 || !q2 || !k1 || !k2 || !v || !lambda || !out) return -1;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || dv <= 0) return -1;
    if (dtype != ORACLE_FP32 && dtype != ORACLE_BF16) return -1;
    int64_t total = (int64_t)B * H * N;
    if (!rows) nrows = total;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= total) return -2;
    prefill_ctx c;
    c.dtype = dtype;
    c.q1 = q1; c.q2 = q2; c.k1 = k1; c.k2 = k2; c.v = v;
    c.ldq = ldq; c.ldk = ldk; c.ldv = ldv;
    c.B = B; c.H = H; c.N = N; c.d = d; c.dv = dv; c.causal = causal;
    c.lambda = lambda;
    c.rmsnorm = rmsnorm; c.eps = eps; c.norm_scale = norm_scale; c.norm_weight = norm_weight;
    c.rows = rows;
    c.out = out;
    return run_pool(nrows, nthreads, 2 * (int64_t)N, prefill_item, &c);
}

/*
 * The two softmax rows A1[i,:] and A2[i,:] of one query (b,h,i), for the
 * signal-to-noise measurement of page "差分注意力", part 二 Step 3.  Masked
 * keys get weight 0.  a1, a2: double [N].
 */
int oracle_prefill_weights(int dtype, const void* q1, const void* q2, const void* k1,
                           const void* k2, int64_t ldq, int64_t ldk, int B, int H, int N,
                           int d, int causal, int b, int h, int i, double* a1, double* a2) {
    if (!q1 || !q2 || !k1 || !k2 || !a1 || !a2) return -1;
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N || d <= 0) return -1;
    int64_t bh = (int64_t)b * H + h;
    int nkeys = causal ? i + 1 : N;
    double* scratch = (double*)malloc(sizeof(double) * 2 * (size_t)N);
    if (!scratch) return -3;
    /* A value tensor of width 0 is never read; the output row is empty. */
    row_job r;
    r.dtype = dtype;
    r.q1 = q1; r.q2 = q2; r.k1 = k1; r.k2 = k2; r.v = k1;
    r.q_off = (bh * N + i) * ldq;
    r.k_off = bh * (int64_t)N * ldk;
    r.v_off = 0;
    r.ldk = ldk;
    r.ldv = 0;
    r.nkeys = nkeys;
    r.d = d;
    r.dv = 0;
    r.lambda = 0.0;
    for (int j = 0; j < N; ++j) { a1[j] = 0.0; a2[j] = 0.0; }
    diff_row(&r, scratch, NULL, a1, a2);
    free(scratch);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode in the V2 layout: one new query per sequence, KV cache shared by   */
/* the two query heads of a pair.                                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    int dtype;
    const void *q, *kc, *vc;
    const int32_t* seq_lens;
    int B, Hq, Hkv, D, Lmax;
    const float* lambda;
    double* out;
} decode_ctx;

static void decode_item(void* vctx, int64_t item, double* scratch) {
    const decode_ctx* c = (const decode_ctx*)vctx;
    int P = c->Hq / 2;
    int b = (int)(item / P);
    int p = (int)(item % P);
    int group = c->Hq / c->Hkv;
    int g = (2 * p) / group;
    int64_t kv_off = ((int64_t)b * c->Hkv + g) * (int64_t)c->Lmax * c->D;
    row_job r;
    r.dtype = c->dtype;
    r.q1 = c->q;
    /* Head 2p+1 follows head 2p in [B][Hq][D]: q2 is q shifted by one head. */
    r.q2 = (const void*)((const char*)c->q + (size_t)c->D * (c->dtype == ORACLE_FP32 ? 4 : 2));
    r.k1 = c->kc; r.k2 = c->kc; r.v = c->vc;
    r.q_off = ((int64_t)b * c->Hq + 2 * p) * c->D;    /* head 2p */
    r.k_off = kv_off;
    r.v_off = kv_off;
    r.ldk = c->D;
    r.ldv = c->D;
    r.nkeys = c->seq_lens[b];
    r.d = c->D;
    r.dv = c->D;
    r.lambda = (double)c->lambda[p];
    diff_row(&r, scratch, c->out + item * (int64_t)c->D, NULL, NULL);
}

/*
 * q: [B][Hq][D]; kc, vc: [B][Hkv][Lmax][D] (fp32 or bf16 bits); seq_lens: [B]
 * with 1 <= L_b <= Lmax; lambda: fp32 [Hq/2]; out: double [B][Hq/2][D].
 * Requires Hq % (2*Hkv) == 0 so that both heads of a pair share a KV head.
 */
int oracle_decode(int dtype, const void* q, const void* kc, const void* vc,
                  const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                  const float* lambda, double* out, int nthreads) {
    if (!q || !kc || !vc || !seq_lens || !lambda || !out) return -1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax <= 0) return -1;
    if (Hq % (2 * Hkv) != 0) return -1;
    if (dtype != ORACLE_FP32 && dtype != ORACLE_BF16) return -1;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 1 || seq_lens[b] > Lmax) return -2;
    decode_ctx c;
    c.dtype = dtype;
    c.q = q; c.kc = kc; c.vc = vc;
    c.seq_lens = seq_lens;
    c.B = B; c.Hq = Hq; c.Hkv = Hkv; c.D = D; c.Lmax = Lmax;
    c.lambda = lambda;
    c.out = out;
    return run_pool((int64_t)B * (Hq / 2), nthreads, 2 * (int64_t)Lmax, decode_item, &c);
}
