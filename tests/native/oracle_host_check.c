/*
 * Sanitizer run of the CPU oracle (oracle/attention.c). Test infrastructure:
 * tests/test_host_sanitizers.py builds this file with the oracle under
 * AddressSanitizer + UndefinedBehaviorSanitizer and, separately, under
 * ThreadSanitizer (the oracle's worker threads share one job record).
 *
 * Every buffer is a heap allocation of exactly the size its layout needs, so
 * a read past K, V, the mask or a row list, or a write past an output, is
 * reported. Besides running clean, each case checks properties that hold
 * whatever the inputs:
 *   - a row with no visible key has o = 0 and lse = -infinity;
 *   - o is a convex combination of the visible values (per column between
 *     their minimum and maximum);
 *   - a row that sees exactly one key returns that key's value row exactly;
 *   - one thread and several threads give bit-identical results;
 *   - invalid arguments return -1.
 * Prints "oracle ok: N rows" and exits 0 when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_rows(const double *q_rows, const int64_t *rb, const int64_t *rh,
                          const int64_t *ri, int64_t nrows, const double *k, const double *v,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                          int64_t Dqk, int64_t Dv, int causal, double scale,
                          const double *mask, int64_t mask_bstride, int64_t mask_stride,
                          double *o_rows, double *lse_rows, int nthreads);

static int failures = 0;
static int64_t rows_checked = 0;

#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAIL line %d: %s: ", __LINE__, #cond);        \
            fprintf(stderr, __VA_ARGS__);                                  \
            fprintf(stderr, "\n");                                         \
            if (++failures > 20) exit(1);                                  \
        }                                                                  \
    } while (0)

/* splitmix64, for reproducible values in [-1, 1) */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

static void *alloc(size_t elem, int64_t n) { return malloc(elem * (size_t)(n > 0 ? n : 1)); }

static double *fill(int64_t n) {
    double *p = (double *)alloc(sizeof(double), n);
    for (int64_t i = 0; i < n; ++i) p[i] = uniform();
    return p;
}

typedef struct {
    int64_t B, Hq, Hkv, Sq, Skv, Dqk, Dv;
    int causal;
    int mask_kind; /* 0 none, 1 shared over the batch, 2 per batch entry */
} shape;

static int visible(const shape *s, const double *mask, int64_t mbs, int64_t ms, int64_t b,
                   int64_t i, int64_t j) {
    if (s->causal && j > i + s->Skv - s->Sq) return 0;
    if (mask && isinf(mask[b * mbs + i * ms + j])) return 0;
    return 1;
}

static void run_case(const shape *s) {
    const int64_t nrows = s->B * s->Hq * s->Sq;
    const int64_t ms = s->Skv + 3; /* a row stride longer than the row */
    const int64_t mbs = s->mask_kind == 2 ? s->Sq * ms : 0;
    double *k = fill(s->B * s->Skv * s->Hkv * s->Dqk);
    double *v = fill(s->B * s->Skv * s->Hkv * s->Dv);
    double *mask = NULL;
    if (s->mask_kind) {
        const int64_t n = (s->mask_kind == 2 ? s->B : 1) * s->Sq * ms;
        mask = fill(n);
        /* hide some keys, and every key of query row 1 */
        for (int64_t t = 0; t < n; ++t) {
            const int64_t i = (t % (s->Sq * ms)) / ms;
            if (i == 1 || mask[t] > 0.6) mask[t] = -INFINITY;
        }
    }
    double *q = fill(nrows * s->Dqk);
    int64_t *rb = (int64_t *)alloc(sizeof(int64_t), nrows);
    int64_t *rh = (int64_t *)alloc(sizeof(int64_t), nrows);
    int64_t *ri = (int64_t *)alloc(sizeof(int64_t), nrows);
    /* rows listed in a scrambled order */
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t x = (r * 7 + 3) % nrows;
        rb[r] = x / (s->Hq * s->Sq);
        rh[r] = (x / s->Sq) % s->Hq;
        ri[r] = x % s->Sq;
    }
    double *o1 = (double *)alloc(sizeof(double), nrows * s->Dv);
    double *l1 = (double *)alloc(sizeof(double), nrows);
    double *o4 = (double *)alloc(sizeof(double), nrows * s->Dv);
    double *l4 = (double *)alloc(sizeof(double), nrows);
    const double scale = 0.37;
    int rc = oracle_attention_rows(q, rb, rh, ri, nrows, k, v, s->B, s->Hq, s->Hkv, s->Sq, s->Skv,
                                   s->Dqk, s->Dv, s->causal, scale, mask, mbs, ms, o1, l1, 1);
    CHECK(rc == 0, "rc %d", rc);
    rc = oracle_attention_rows(q, rb, rh, ri, nrows, k, v, s->B, s->Hq, s->Hkv, s->Sq, s->Skv,
                               s->Dqk, s->Dv, s->causal, scale, mask, mbs, ms, o4, l4, 4);
    CHECK(rc == 0, "rc %d", rc);
    CHECK(memcmp(o1, o4, sizeof(double) * (size_t)(nrows * s->Dv)) == 0 &&
              memcmp(l1, l4, sizeof(double) * (size_t)nrows) == 0,
          "1 and 4 threads differ");
    const int64_t G = s->Hq / s->Hkv;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rb[r], h = rh[r], i = ri[r], g = h / G;
        int64_t nvis = 0, last = -1;
        for (int64_t j = 0; j < s->Skv; ++j)
            if (visible(s, mask, mbs, ms, b, i, j)) {
                ++nvis;
                last = j;
            }
        const double *orow = o1 + r * s->Dv;
        if (nvis == 0) {
            CHECK(isinf(l1[r]) && l1[r] < 0, "row %lld: lse %g with no visible key",
                  (long long)r, l1[r]);
            for (int64_t d = 0; d < s->Dv; ++d) CHECK(orow[d] == 0.0, "row %lld o != 0", (long long)r);
            continue;
        }
        CHECK(isfinite(l1[r]), "row %lld: lse %g", (long long)r, l1[r]);
        for (int64_t d = 0; d < s->Dv; ++d) {
            double lo = INFINITY, hi = -INFINITY;
            for (int64_t j = 0; j < s->Skv; ++j)
                if (visible(s, mask, mbs, ms, b, i, j)) {
                    const double x = v[((b * s->Skv + j) * s->Hkv + g) * s->Dv + d];
                    lo = x < lo ? x : lo;
                    hi = x > hi ? x : hi;
                }
            CHECK(orow[d] >= lo - 1e-12 && orow[d] <= hi + 1e-12, "row %lld col %lld not convex",
                  (long long)r, (long long)d);
            if (nvis == 1)
                CHECK(orow[d] == v[((b * s->Skv + last) * s->Hkv + g) * s->Dv + d],
                      "row %lld: one key but o != v", (long long)r);
        }
    }
    rows_checked += nrows;
    free(k); free(v); free(mask); free(q); free(rb); free(rh); free(ri);
    free(o1); free(l1); free(o4); free(l4);
}

static void bad_arguments(void) {
    double q[8] = {0}, k[8] = {0}, v[8] = {0}, o[8], l[2];
    int64_t rb[1] = {0}, rh[1] = {0}, ri[1] = {0};
    CHECK(oracle_attention_rows(q, rb, rh, ri, 1, k, v, 1, 3, 2, 1, 1, 4, 4, 0, 1.0, NULL, 0, 0,
                                o, l, 1) == -1, "Hq %% Hkv");
    int64_t bad_b[1] = {1};
    CHECK(oracle_attention_rows(q, bad_b, rh, ri, 1, k, v, 1, 1, 1, 1, 1, 4, 4, 0, 1.0, NULL, 0,
                                0, o, l, 1) == -1, "row batch out of range");
    CHECK(oracle_attention_rows(q, rb, rh, ri, 1, k, v, 1, 1, 1, 1, 2, 4, 4, 0, 1.0, k, 0, 1, o,
                                l, 1) == -1, "mask stride < Skv");
    CHECK(oracle_attention_rows(q, rb, rh, ri, 1, k, v, 1, 1, 1, 1, 1, 0, 4, 0, 1.0, NULL, 0, 0,
                                o, l, 1) == -1, "Dqk = 0");
}

int main(void) {
    const shape cases[] = {
        {2, 4, 2, 5, 7, 16, 16, 0, 0},   /* grouped heads, no mask */
        {2, 4, 2, 5, 7, 16, 16, 1, 0},   /* causal, Sq < Skv */
        {1, 3, 1, 9, 4, 8, 8, 1, 0},     /* causal, Sq > Skv: empty leading rows */
        {2, 2, 2, 3, 0, 8, 8, 0, 0},     /* no keys at all */
        {1, 2, 1, 4, 10, 24, 16, 1, 0},  /* key width != value width */
        {3, 4, 4, 6, 13, 8, 8, 0, 1},    /* one mask shared over the batch */
        {3, 6, 2, 6, 13, 8, 8, 1, 2},    /* per-batch mask with the causal rule */
        {1, 1, 1, 1, 1, 4, 4, 0, 0},     /* one key */
        {2, 8, 1, 17, 65, 32, 32, 1, 0}, /* several hundred rows */
    };
    for (size_t c = 0; c < sizeof(cases) / sizeof(cases[0]); ++c) run_case(&cases[c]);
    bad_arguments();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle ok: %lld rows\n", (long long)rows_checked);
    return 0;
}
