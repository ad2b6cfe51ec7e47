/* Host sanitizer run of the CPU oracle: every entry point of losa_oracle.c on
 * small fixed inputs (ragged sequences, an empty prefix, a partial last page,
 * every reading flag), built with AddressSanitizer and UndefinedBehavior-
 * Sanitizer.  The values are not checked here (the pins do that); any
 * out-of-bounds access, leak or undefined operation aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_seq, block, n_qhead, n_kvhead, head_dim, page_size, budget_tokens, n_active;
    int32_t out_bf16, union_cap;
    int64_t kv_tokens;
    double softmax_scale;
    int32_t flags, pad_;
} oracle_shape;

void oracle_page_meta(const oracle_shape *, const float *, const int32_t *, const int32_t *,
                      float *, float *);
void oracle_locality(const oracle_shape *, const float *, const float *, float *);
void oracle_active_set(const oracle_shape *, const float *, int32_t *);
void oracle_shared_active_set(const oracle_shape *, const float *, float *, int32_t *);
float oracle_page_bound(const float *, const float *, const float *, int);
void oracle_select_pages(const oracle_shape *, const float *, const float *, const float *,
                         const int32_t *, const int32_t *, const int32_t *, int32_t *, int32_t *,
                         int32_t *, float *, int64_t);
void oracle_step(const oracle_shape *, const float *, const float *, const float *, const float *,
                 const float *, const float *, const float *, const float *, const int32_t *,
                 const int32_t *, double *, double *, float *, float *, int32_t *, int32_t *,
                 int32_t *, int32_t *);
void oracle_dense_first_step(const oracle_shape *, const float *, const float *, const float *,
                             const float *, const float *, const int32_t *, const int32_t *,
                             double *, double *, float *);
void oracle_naive_sparse_step(const oracle_shape *, const float *, const float *, const float *,
                              const float *, const float *, const float *, const float *,
                              const int32_t *, const int32_t *, double *, double *, float *);
void oracle_dense_row(const oracle_shape *, int, int, int, const float *, const float *,
                      const float *, const float *, const float *, const int32_t *,
                      const int32_t *, double *, double *, float *);

static uint64_t rng_state = 88172645463325252ull;
static float draw(void) { /* xorshift64, uniform in [-2, 2) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (float)((rng_state >> 11) * (1.0 / 9007199254740992.0) * 4.0 - 2.0);
}
static float *fill(size_t n) {
    float *a = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) a[i] = draw();
    return a;
}

static int run(int flags, int budget, int n_active) {
    const int S = 3, B = 8, Hq = 4, Hk = 2, d = 16, P = 16;
    const int32_t lens[3] = {200, 0, 37};
    int32_t off[3];
    int64_t T = 0;
    for (int s = 0; s < S; ++s) {
        off[s] = (int32_t)T;
        T += (lens[s] + P - 1) / P * P;
    }
    if (T < P) T = P;
    int max_pages = (200 + P - 1) / P;
    oracle_shape sh = {S, B, Hq, Hk, d, P, budget, n_active, 1, max_pages, T, 0.0, flags, 0};
    float *kc = fill((size_t)Hk * T * d), *vc = fill((size_t)Hk * T * d);
    float *kmin = fill((size_t)Hk * (T / P) * d), *kmax = fill((size_t)Hk * (T / P) * d);
    const size_t nq = (size_t)S * B * Hq * d, nb = (size_t)S * B * Hk * d;
    float *q0 = fill(nq), *q1 = fill(nq), *kb = fill(nb), *vb = fill(nb), *out = fill(nq);
    const size_t rows = (size_t)S * Hq * B;
    double *op = (double *)calloc(rows * d, sizeof(double));
    double *lp = (double *)calloc(rows, sizeof(double));
    float *loc = fill(rows), *tot = fill((size_t)S * B);
    const int k = budget / P;
    int32_t *act = (int32_t *)calloc((size_t)S * Hq * (n_active ? n_active : 1), sizeof(int32_t));
    int32_t *psel = (int32_t *)calloc((size_t)S * Hq * (n_active ? n_active : 1) * k, sizeof(int32_t));
    int32_t *uidx = (int32_t *)calloc((size_t)S * Hk * max_pages, sizeof(int32_t));
    int32_t *ucnt = (int32_t *)calloc((size_t)S * Hk, sizeof(int32_t));
    float *bounds = fill((size_t)S * Hk * (Hq / Hk) * (n_active ? n_active : 1) * max_pages);
    double orow[16], lrow;
    float out_row[16];

    oracle_page_meta(&sh, kc, off, lens, kmin, kmax);
    oracle_locality(&sh, q1, q0, loc);
    oracle_active_set(&sh, loc, act);
    oracle_shared_active_set(&sh, loc, tot, act);
    (void)oracle_page_bound(q1, kmin, kmax, d);
    oracle_active_set(&sh, loc, act);
    oracle_select_pages(&sh, q1, kmin, kmax, off, lens, act, psel, uidx, ucnt, bounds, max_pages);
    oracle_dense_first_step(&sh, q0, kb, vb, kc, vc, off, lens, op, lp, out);
    oracle_step(&sh, q1, q0, kb, vb, kc, vc, kmin, kmax, off, lens, op, lp, out, loc, act, psel,
                uidx, ucnt);
    oracle_naive_sparse_step(&sh, q1, kb, vb, kc, vc, kmin, kmax, off, lens, op, lp, out);
    for (int s = 0; s < S; ++s) oracle_dense_row(&sh, s, Hq - 1, B - 1, q1, kb, vb, kc, vc, off, lens, orow, &lrow, out_row);
    double chk = 0;
    for (size_t i = 0; i < nq; ++i) chk += out[i];
    free(kc); free(vc); free(kmin); free(kmax); free(q0); free(q1); free(kb); free(vb); free(out);
    free(op); free(lp); free(loc); free(tot); free(act); free(psel); free(uidx); free(ucnt); free(bounds);
    return isfinite(chk) ? 0 : 1;
}

int main(void) {
    int bad = 0;
    for (int flags = 0; flags < 8; ++flags) bad |= run(flags, 48, 3);
    bad |= run(0, 1024, 8);  /* budget past every prefix: every page selected */
    bad |= run(0, 16, 0);    /* no active token */
    printf("oracle sanitizer run: %s\n", bad ? "non-finite output" : "ok");
    return bad;
}
