/*
 * oracle_driver.c -- runs the fp64 oracle (oracle/attn_oracle.c, linked in)
 * under AddressSanitizer and UndefinedBehaviorSanitizer: every public
 * function on small inputs, every layout, mask and grouping, the thread
 * split, argument errors, and the special values (NaN, Inf, subnormals).
 * Built and run by tests/test_sanitize.py; exits non-zero on a failed check
 * (the sanitizers abort on their own findings).
 *
 * The checks here are light (the values are pinned by the Python tests);
 * what matters is that every path executes with bounds and UB checking on.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_decode(uint16_t b);
uint16_t oracle_round_bf16(double x, int mode);
void oracle_round_array(const double *x, int64_t n, int mode, uint16_t *out);
void oracle_decode_array(const uint16_t *b, int64_t n, double *out);
int oracle_attn_rows_gqa(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B, int64_t H,
                         int64_t H_kv, int64_t Sq, int64_t Sk, int layout, int mask, const int64_t *rows,
                         int64_t nrows, double *o_exact, uint16_t *o_round, double *lse, int nthreads);
int oracle_attn_rows_masked(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B, int64_t H,
                            int64_t Sq, int64_t Sk, int layout, int mask, const int64_t *rows, int64_t nrows,
                            double *o_exact, uint16_t *o_round, int nthreads);
int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B, int64_t H, int64_t Sq,
                     int64_t Sk, int layout, const int64_t *rows, int64_t nrows, double *o_exact,
                     uint16_t *o_round, int nthreads);
double oracle_softmax_row(const uint16_t *q, const uint16_t *k, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                          int layout, int64_t b, int64_t h, int64_t i, double *w);

#define D 128
static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

/* xorshift64* for inputs; values are bf16 patterns of N(0,1)-ish magnitude */
static uint64_t rng_state = 88172645463325252ull;
static uint64_t next_u64(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 2685821657736338717ull;
}
static uint16_t rand_bf16(void)
{
    /* sign, exponent 124..128 (values 1/8 .. 4), random 7-bit fraction */
    uint64_t u = next_u64();
    return (uint16_t)(((u >> 63) << 15) | ((124 + (u >> 20) % 5) << 7) | ((u >> 40) & 0x7F));
}

static uint16_t *alloc_bits(size_t n)
{
    uint16_t *p = (uint16_t *)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i)
        p[i] = rand_bf16();
    return p;
}

static void run_case(int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int layout, int mask,
                     int nthreads)
{
    uint16_t *q = alloc_bits((size_t)(B * H * Sq * D));
    uint16_t *k = alloc_bits((size_t)(B * H_kv * Sk * D));
    uint16_t *v = alloc_bits((size_t)(B * H_kv * Sk * D));
    int64_t nrows = B * H * Sq;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)nrows);
    int64_t r = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t i = 0; i < Sq; ++i, ++r)
                rows[3 * r] = b, rows[3 * r + 1] = h, rows[3 * r + 2] = i;
    double *ex = (double *)malloc(sizeof(double) * (size_t)(nrows * D));
    uint16_t *rd = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(nrows * 3 * D));
    double *lse = (double *)malloc(sizeof(double) * (size_t)nrows);
    CHECK(oracle_attn_rows_gqa(q, k, v, B, H, H_kv, Sq, Sk, layout, mask, rows, nrows, ex, rd, lse, nthreads) == 0);
    for (int64_t i = 0; i < nrows * D; ++i) {
        /* each element is a weighted mean of V values (|v| <= 4) or NaN (a row with no key) */
        CHECK(isnan(ex[i]) || fabs(ex[i]) <= 4.0);
    }
    if (H == H_kv) {
        double *ex2 = (double *)malloc(sizeof(double) * (size_t)(nrows * D));
        uint16_t *rd2 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(nrows * 3 * D));
        CHECK(oracle_attn_rows_masked(q, k, v, B, H, Sq, Sk, layout, mask, rows, nrows, ex2, rd2, 1) == 0);
        CHECK(memcmp(rd, rd2, sizeof(uint16_t) * (size_t)(nrows * 3 * D)) == 0);
        if (mask == 0) {
            CHECK(oracle_attn_rows(q, k, v, B, H, Sq, Sk, layout, rows, nrows, ex2, rd2, 3) == 0);
            CHECK(memcmp(rd, rd2, sizeof(uint16_t) * (size_t)(nrows * 3 * D)) == 0);
            double *w = (double *)malloc(sizeof(double) * (size_t)Sk);
            double l = oracle_softmax_row(q, k, B, H, Sq, Sk, layout, B - 1, H - 1, Sq - 1, w);
            double s = 0.0;
            for (int64_t j = 0; j < Sk; ++j)
                s += w[j];
            CHECK(l >= 1.0 && fabs(s - 1.0) < 1e-12);
            free(w);
        }
        free(ex2), free(rd2);
    }
    free(q), free(k), free(v), free(rows), free(ex), free(rd), free(lse);
}

int main(void)
{
    /* decode and round every bf16 pattern, and the three modes on assorted binary64 values */
    double *vals = (double *)malloc(sizeof(double) * 65536);
    uint16_t *bits = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    uint16_t *back = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    for (int i = 0; i < 65536; ++i)
        bits[i] = (uint16_t)i;
    oracle_decode_array(bits, 65536, vals);
    for (int m = 0; m < 3; ++m) {
        oracle_round_array(vals, 65536, m, back);
        for (int i = 0; i < 65536; ++i) {
            const int nan = ((i & 0x7F80) == 0x7F80) && (i & 0x7F);
            CHECK(nan ? back[i] == 0x7FC0 : back[i] == bits[i]);
        }
    }
    const double specials[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e-300, -1e-300, 1e300, -1e300,
                               3.3895313892515355e38, 3.4e38, 1.0 + 1.0 / 256, ldexp(1.5, -133), ldexp(1.0, -140)};
    for (size_t i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i)
        for (int m = 0; m < 3; ++m)
            (void)oracle_round_bf16(specials[i], m);
    CHECK(oracle_round_bf16(ldexp(1.5, -133), 0) == 0x0002 && oracle_round_bf16(ldexp(1.5, -133), 2) == 0x0001);
    for (int i = 0; i < 200000; ++i) {
        uint64_t u = next_u64();
        double x;
        memcpy(&x, &u, sizeof x);
        for (int m = 0; m < 3; ++m)
            (void)oracle_round_bf16(x, m);
    }
    free(vals), free(bits), free(back);

    /* attention rows: layouts, masks (none, top left, bottom right), grouping, threads, ragged sizes */
    for (int layout = 0; layout < 2; ++layout)
        for (int mask = 0; mask < 3; ++mask) {
            run_case(2, 3, 3, 17, 70, layout, mask, 4);
            run_case(1, 4, 2, 70, 17, layout, mask, 3);  /* Sq > Sk: bottom-right rows without a key */
            run_case(1, 2, 1, 1, 1, layout, mask, 8);
        }

    /* special values: NaN, +Inf and -Inf in K, a subnormal V */
    {
        int64_t Sq = 5, Sk = 9;
        uint16_t *q = alloc_bits((size_t)(Sq * D)), *k = alloc_bits((size_t)(Sk * D)), *v = alloc_bits((size_t)(Sk * D));
        k[3 * D + 5] = 0x7FC0, k[4 * D + 6] = 0x7F80, k[5 * D + 7] = 0xFF80, v[2 * D + 9] = 0x0001;
        int64_t rows[15];
        for (int i = 0; i < Sq; ++i)
            rows[3 * i] = 0, rows[3 * i + 1] = 0, rows[3 * i + 2] = i;
        double ex[5 * D], lse[5];
        uint16_t rd[5 * 3 * D];
        CHECK(oracle_attn_rows_gqa(q, k, v, 1, 1, 1, Sq, Sk, 0, 0, rows, Sq, ex, rd, lse, 2) == 0);
        for (int i = 0; i < Sq; ++i)
            CHECK(isnan(ex[i * D]) && isnan(lse[i]));  /* the NaN logit poisons every row */
        free(q), free(k), free(v);
    }

    /* argument errors return -1 and touch nothing */
    {
        uint16_t t[D] = {0};
        int64_t rows[3] = {0, 0, 0}, bad_rows[3] = {0, 0, 5};
        double ex[D];
        uint16_t rd[3 * D];
        CHECK(oracle_attn_rows_gqa(NULL, t, t, 1, 1, 1, 1, 1, 0, 0, rows, 1, ex, rd, NULL, 1) == -1);
        CHECK(oracle_attn_rows_gqa(t, t, t, 1, 3, 2, 1, 1, 0, 0, rows, 1, ex, rd, NULL, 1) == -1);
        CHECK(oracle_attn_rows_gqa(t, t, t, 1, 1, 1, 1, 1, 2, 0, rows, 1, ex, rd, NULL, 1) == -1);
        CHECK(oracle_attn_rows_gqa(t, t, t, 1, 1, 1, 1, 1, 0, 3, rows, 1, ex, rd, NULL, 1) == -1);
        CHECK(oracle_attn_rows_gqa(t, t, t, 1, 1, 1, 1, 1, 0, 0, bad_rows, 1, ex, rd, NULL, 1) == -1);
        CHECK(oracle_attn_rows_gqa(t, t, t, 1, 1, 1, 0, 1, 0, 0, rows, 1, ex, rd, NULL, 1) == -1);
    }
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle driver: all checks passed\n");
    return failures ? 1 : 0;
}
