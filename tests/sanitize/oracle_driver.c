/*
 * oracle_driver.c -- exercises oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by tests/test_sanitize.py).
 *
 * Every buffer is allocated at exactly the size its layout needs, so a read
 * or write one element past a tensor, a per-head window array or a row list
 * is reported.  The shapes cover what the oracle's indexing distinguishes:
 * GQA groups, Nq != Nk both ways, ragged key tiles of the streaming form,
 * row subsets, key ranges (split chunks), windows with sinks, soft-caps,
 * empty sizes, more threads than rows, and each invalid-argument return.
 * Besides memory safety it checks that the direct and the streaming forms
 * agree, that a row subset equals the same rows of the full result, and
 * that merging split chunks (oracle_combine) equals the unsplit result.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, double *lse, double *m_out, double *l_out,
                     int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                     double scale, int causal, const int32_t *head_window, double softcap,
                     int64_t sinks, int64_t key_lo, int64_t key_hi,
                     const int64_t *rows, int64_t nrows, int64_t tile, int nthreads);
int oracle_combine(const double *o_part, const double *m_part, const double *l_part,
                   double *o, double *lse, int64_t R, int64_t S, int64_t d);

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++failures;                                   \
        }                                                 \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static double uniform(void)
{
    /* xorshift64*: a deterministic stream, no relation to the method. */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

/* malloc of exactly n doubles (one byte when n == 0, so the pointer is
 * valid but any access is out of bounds). */
static double *dalloc(int64_t n)
{
    double *p = (double *)malloc(n > 0 ? (size_t)n * sizeof(double) : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    for (int64_t i = 0; i < n; ++i) p[i] = uniform();
    return p;
}

static double max_diff(const double *a, const double *b, int64_t n)
{
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        if (isinf(a[i]) && isinf(b[i]) && a[i] == b[i]) continue;
        double e = fabs(a[i] - b[i]);
        if (!(e <= m)) m = e; /* NaN propagates as a failure */
    }
    return m;
}

typedef struct {
    int64_t B, H, Hkv, Nq, Nk, d;
    int causal;
    int windowed;     /* 0: none; 1: alternate heads windowed */
    int64_t window;
    double softcap;
    int64_t sinks;
} shape_t;

static void run_shape(const shape_t *s)
{
    const int64_t R = s->B * s->H * s->Nq;
    double *q = dalloc(s->B * s->H * s->Nq * s->d);
    double *k = dalloc(s->B * s->Hkv * s->Nk * s->d);
    double *v = dalloc(s->B * s->Hkv * s->Nk * s->d);
    int32_t *hw = NULL;
    if (s->windowed) {
        hw = (int32_t *)malloc((size_t)(s->H > 0 ? s->H : 1) * sizeof(int32_t));
        for (int64_t h = 0; h < s->H; ++h) hw[h] = (h % 2 == 0) ? (int32_t)s->window : 0;
    }
    const double scale = 1.0 / sqrt((double)(s->d > 0 ? s->d : 1)) * 3.0;
    double *o = dalloc(R * s->d), *lse = dalloc(R), *m = dalloc(R), *l = dalloc(R);
    int rc = oracle_attention(q, k, v, o, lse, m, l, s->B, s->H, s->Hkv, s->Nq, s->Nk, s->d, scale,
                              s->causal, hw, s->softcap, s->sinks, 0, s->Nk, NULL, 0, 0, 3);
    CHECK(rc == 0, "direct rc %d", rc);
    for (int64_t r = 0; r < R; ++r) {
        if (isinf(lse[r])) {
            CHECK(lse[r] < 0 && l[r] == 0.0, "row %lld: empty row state", (long long)r);
            for (int64_t c = 0; c < s->d; ++c) CHECK(o[r * s->d + c] == 0.0, "row %lld: O of an empty row", (long long)r);
        } else {
            CHECK(isfinite(lse[r]) && l[r] >= 1.0, "row %lld: lse %g l %g", (long long)r, lse[r], l[r]);
        }
    }

    /* Streaming form, ragged tiles (1, 5 and more than Nk keys). */
    const int64_t tiles[3] = {1, 5, s->Nk + 3};
    for (int t = 0; t < 3; ++t) {
        double *o2 = dalloc(R * s->d), *lse2 = dalloc(R);
        rc = oracle_attention(q, k, v, o2, lse2, NULL, NULL, s->B, s->H, s->Hkv, s->Nq, s->Nk, s->d, scale,
                              s->causal, hw, s->softcap, s->sinks, 0, s->Nk, NULL, 0, tiles[t], 8);
        CHECK(rc == 0, "stream rc %d", rc);
        CHECK(max_diff(o, o2, R * s->d) <= 1e-12, "tile %lld: O differs by %g", (long long)tiles[t],
              max_diff(o, o2, R * s->d));
        CHECK(max_diff(lse, lse2, R) <= 1e-12, "tile %lld: lse differs", (long long)tiles[t]);
        free(o2);
        free(lse2);
    }

    /* A row subset in reverse order equals the same rows of the full result. */
    if (R > 0) {
        const int64_t nr = R < 7 ? R : 7;
        int64_t *rows = (int64_t *)malloc((size_t)nr * sizeof(int64_t));
        for (int64_t n = 0; n < nr; ++n) rows[n] = R - 1 - (n * (R / nr));
        double *o3 = dalloc(nr * s->d), *lse3 = dalloc(nr);
        rc = oracle_attention(q, k, v, o3, lse3, NULL, NULL, s->B, s->H, s->Hkv, s->Nq, s->Nk, s->d, scale,
                              s->causal, hw, s->softcap, s->sinks, 0, s->Nk, rows, nr, 0, 16);
        CHECK(rc == 0, "rows rc %d", rc);
        for (int64_t n = 0; n < nr; ++n) {
            CHECK(max_diff(o + rows[n] * s->d, o3 + n * s->d, s->d) == 0.0, "subset row %lld", (long long)n);
            CHECK(max_diff(lse + rows[n], lse3 + n, 1) == 0.0, "subset lse %lld", (long long)n);
        }
        free(rows);
        free(o3);
        free(lse3);
    }

    /* Split chunks of the keys merged with oracle_combine equal the whole. */
    const int64_t S = 3;
    const int64_t C = s->Nk > 0 ? (s->Nk + S - 1) / S : 0;
    double *op = dalloc(R * S * s->d), *mp = dalloc(R * S), *lp = dalloc(R * S);
    for (int64_t sp = 0; sp < S; ++sp) {
        double *oc = dalloc(R * s->d), *mc = dalloc(R), *lc = dalloc(R);
        rc = oracle_attention(q, k, v, oc, NULL, mc, lc, s->B, s->H, s->Hkv, s->Nq, s->Nk, s->d, scale, s->causal,
                              hw, s->softcap, s->sinks, sp * C, (sp + 1) * C, NULL, 0, 0, 2);
        CHECK(rc == 0, "chunk rc %d", rc);
        for (int64_t r = 0; r < R; ++r) {
            memcpy(op + (r * S + sp) * s->d, oc + r * s->d, (size_t)s->d * sizeof(double));
            mp[r * S + sp] = mc[r];
            lp[r * S + sp] = lc[r];
        }
        free(oc);
        free(mc);
        free(lc);
    }
    double *o4 = dalloc(R * s->d), *lse4 = dalloc(R);
    rc = oracle_combine(op, mp, lp, o4, lse4, R, S, s->d);
    CHECK(rc == 0, "combine rc %d", rc);
    CHECK(max_diff(o, o4, R * s->d) <= 1e-12, "combined O differs by %g", max_diff(o, o4, R * s->d));
    CHECK(max_diff(lse, lse4, R) <= 1e-12, "combined lse differs by %g", max_diff(lse, lse4, R));

    free(op); free(mp); free(lp); free(o4); free(lse4);
    free(o); free(lse); free(m); free(l);
    free(q); free(k); free(v); free(hw);
}

static void invalid_arguments(void)
{
    double *q = dalloc(2 * 2 * 4), *k = dalloc(2 * 4), *v = dalloc(2 * 4);
    double *o = dalloc(2 * 2 * 4);
    int32_t hw[2] = {3, 0};
    int64_t bad_rows[1] = {4};
    /* B=1, H=2, Hkv=1, Nq=2, Nk=2, d=2 unless varied. */
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, -1, 2, 1, 2, 2, 2, 1.0, 0, NULL, 0, 0, 0, 2, NULL, 0, 0, 1) == -1, "B<0");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 2, 0, 2, 2, 2, 1.0, 0, NULL, 0, 0, 0, 2, NULL, 0, 0, 1) == -1, "Hkv=0");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 3, 2, 2, 2, 2, 1.0, 0, NULL, 0, 0, 0, 2, NULL, 0, 0, 1) == -1, "H not a multiple of Hkv");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 2, 1, 2, 2, -2, 1.0, 0, NULL, 0, 0, 0, 2, NULL, 0, 0, 1) == -1, "d<0");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 2, 1, 2, 2, 2, 1.0, 0, hw, 0, 0, 0, 2, NULL, 0, 0, 1) == -1, "window without causal");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 2, 1, 2, 2, 2, 1.0, 1, NULL, 0, -1, 0, 2, NULL, 0, 0, 1) == -1, "sinks<0");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 2, 1, 2, 2, 2, 1.0, 1, NULL, 0, 0, 0, 2, NULL, 0, -1, 1) == -1, "tile<0");
    CHECK(oracle_attention(q, k, v, o, NULL, NULL, NULL, 1, 2, 1, 2, 2, 2, 1.0, 1, NULL, 0, 0, 0, 2, bad_rows, 1, 0, 1) == -1, "row out of range");
    CHECK(oracle_combine(o, o, o, o, o, 1, 0, 2) == -1, "S=0");
    CHECK(oracle_combine(o, o, o, o, o, -1, 1, 2) == -1, "R<0");
    free(q); free(k); free(v); free(o);
}

int main(void)
{
    const shape_t shapes[] = {
        /* B, H, Hkv, Nq, Nk, d, causal, windowed, window, softcap, sinks */
        {2, 4, 2, 13, 13, 8, 1, 0, 0, 0.0, 0},    /* causal GQA, square    */
        {1, 6, 3, 9, 21, 5, 1, 1, 4, 0.0, 2},     /* Nq < Nk, windows+sinks */
        {1, 2, 2, 17, 6, 4, 1, 0, 0, 0.0, 0},     /* Nq > Nk: rows see none */
        {2, 3, 1, 7, 11, 3, 0, 0, 0, 2.5, 0},     /* non-causal, soft-cap   */
        {1, 4, 4, 10, 10, 6, 1, 1, 1, 30.0, 3},   /* window 1, sinks, cap   */
        {1, 2, 1, 5, 0, 4, 0, 0, 0, 0.0, 0},      /* no keys                */
        {1, 2, 1, 0, 5, 4, 1, 0, 0, 0.0, 0},      /* no queries             */
        {0, 2, 1, 5, 5, 4, 1, 0, 0, 0.0, 0},      /* empty batch            */
        {1, 2, 2, 3, 4, 0, 1, 0, 0, 0.0, 0},      /* d = 0                  */
        {1, 1, 1, 1, 1, 1, 1, 1, 5, 0.0, 9},      /* window > Nk, sinks > Nk */
    };
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) run_shape(&shapes[i]);
    invalid_arguments();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle_driver: all checks passed\n");
    return 0;
}
