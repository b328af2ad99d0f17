/*
 * Thread-sanitizer driver for the oracle's worker pool (oracle.c): the same
 * prefill and decode computed with 1 and with 8 worker threads must agree bit
 * for bit, and the sanitizer must report no data race.  Built together with
 * oracle.c under -fsanitize=thread (and, separately, address/undefined);
 * exit status 0 iff every comparison holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_prefill(int dtype, const void* q1, const void* q2, const void* k1, const void* k2,
                   const void* v, int64_t ldq, int64_t ldk, int64_t ldv, int B, int H, int N,
                   int d, int dv, int causal, const float* lambda, int rmsnorm, double eps,
                   double norm_scale, const float* norm_weight, const int64_t* rows,
                   int64_t nrows, double* out, int nthreads);
int oracle_decode(int dtype, const void* q, const void* kc, const void* vc,
                  const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                  const float* lambda, double* out, int nthreads);
void oracle_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int H,
                   int dim, int layer, float* out);

/* xorshift64*: a deterministic input stream (uniform in [-1, 1)). */
static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static float next_uniform(void) {
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (float)((g_state * 0x2545f4914f6cdd1dull) >> 40) / (float)(1 << 23) - 1.0f;
}
static float* fill(size_t n) {
    float* a = (float*)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) a[i] = next_uniform();
    return a;
}

int main(void) {
    int fails = 0;
    /* Prefill: B=2, H=3, N=57, d=16, dv=24, causal, RMS norm; then a row subset. */
    const int B = 2, H = 3, N = 57, d = 16, dv = 24;
    const size_t nq = (size_t)B * H * N * d, nv = (size_t)B * H * N * dv;
    float *q1 = fill(nq), *q2 = fill(nq), *k1 = fill(nq), *k2 = fill(nq), *v = fill(nv);
    float lam[3] = {0.3f, -0.2f, 0.9f};
    double* a = (double*)calloc(nv, sizeof(double));
    double* b = (double*)calloc(nv, sizeof(double));
    if (oracle_prefill(0, q1, q2, k1, k2, v, d, d, dv, B, H, N, d, dv, 1, lam, 1, 1e-5, 0.4, NULL,
                       NULL, 0, a, 1) != 0 ||
        oracle_prefill(0, q1, q2, k1, k2, v, d, d, dv, B, H, N, d, dv, 1, lam, 1, 1e-5, 0.4, NULL,
                       NULL, 0, b, 8) != 0) {
        fprintf(stderr, "prefill call failed\n");
        return 1;
    }
    if (memcmp(a, b, nv * sizeof(double)) != 0) { fprintf(stderr, "prefill: threads disagree\n"); ++fails; }
    int64_t rows[5] = {0, 56, 100, 171, (int64_t)B * H * N - 1};
    double r[5 * 24];
    if (oracle_prefill(0, q1, q2, k1, k2, v, d, d, dv, B, H, N, d, dv, 1, lam, 1, 1e-5, 0.4, NULL,
                       rows, 5, r, 8) != 0) return 1;
    for (int i = 0; i < 5; ++i)
        if (memcmp(r + i * dv, a + rows[i] * dv, dv * sizeof(double)) != 0) {
            fprintf(stderr, "prefill: row %lld differs from the full run\n", (long long)rows[i]);
            ++fails;
        }

    /* Decode, V2 layout: B=5, Hq=8, Hkv=2, D=16, Lmax=40. */
    const int DB = 5, Hq = 8, Hkv = 2, D = 16, L = 40;
    float* dq = fill((size_t)DB * Hq * D);
    float* kc = fill((size_t)DB * Hkv * L * D);
    float* vc = fill((size_t)DB * Hkv * L * D);
    int32_t lens[5] = {1, 7, 40, 33, 12};
    float dl[4] = {0.1f, 0.5f, -0.3f, 0.8f};
    double da[5 * 4 * 16], db[5 * 4 * 16];
    if (oracle_decode(0, dq, kc, vc, lens, DB, Hq, Hkv, D, L, dl, da, 1) != 0 ||
        oracle_decode(0, dq, kc, vc, lens, DB, Hq, Hkv, D, L, dl, db, 8) != 0) return 1;
    if (memcmp(da, db, sizeof da) != 0) { fprintf(stderr, "decode: threads disagree\n"); ++fails; }

    float lo[3];
    oracle_lambda(q1, k1, q2, k2, 3, d, 2, lo);
    free(q1); free(q2); free(k1); free(k2); free(v); free(a); free(b);
    free(dq); free(kc); free(vc);
    printf("oracle thread check: %d failures\n", fails);
    return fails ? 1 : 0;
}
