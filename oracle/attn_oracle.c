/*
 * attn_oracle.c -- plain fp64 CPU oracle for bf16 forward attention, without a
 * mask or with a causal one, with as many K/V heads as query heads or fewer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the test-suite, the
 * smoke check and the CPU-baseline leg of the benchmark do.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes (the definition, not an algorithm for speed):
 *
 *   O = softmax(Q K^T / sqrt(d)) V,   d = 128, per (batch b, head h, query i)
 *
 * as stated on the snilld.dk page "Open source attention kernel in HIP beats
 * AITER v3 on MI300X" (section "Hvordan kernen arbejder" / How the kernel
 * works), for the BSHD and BHSD layouts, head_dim 128, any query and key
 * lengths (section "Hvad er udgivet" / What was released), followed by one
 * rounding of each output element to bf16 in the mode the caller asks for
 * (RTNE, RTNA, RTZ: the three modes of the tilnote.io page "MoonMath AI HIP
 * attention kernel", section on the performance figures, and the snilld.dk
 * section "Numerik samlet et sted" / Numerics in one place).
 *
 * Every operation is IEEE-754 binary64, evaluated in the order written:
 *   1. decode each bf16 input exactly (bf16_decode);
 *   2. s_j = (sum_{c=0..127} q_c k_{j,c}) / sqrt(128), c ascending;
 *   3. m = max_j s_j, where any NaN makes m NaN (propagating maximum);
 *   4. w_j = exp(s_j - m);  l = sum_j w_j, j ascending;
 *   5. o_c = (sum_j w_j v_{j,c}) / l, j ascending;
 *   6. round o_c once, from binary64, to bf16 (round_bf16).
 * NaN and Inf follow from IEEE arithmetic on these steps; nothing is
 * special-cased beyond the propagating maximum of step 3.
 *
 * Causal mask.  The snilld.dk page lists the causal mask among what the
 * kernel it describes leaves out and what autoregressive serving needs
 * (sections "Hvad er udgivet" / What was released and "Autoregressiv serving,
 * de praktiske hager" / Autoregressive serving, the practical catches); it
 * gives no definition.  Read here as the usual one: query row i attends only
 * to the keys j <= i + off, where off = 0 aligns the diagonal at the top left
 * (row 0 sees key 0) and off = Sk - Sq at the bottom right (the last row sees
 * every key).  The masked keys do not take part at all: steps 2-5 run over
 * the visible keys j < n_i = min(max(i + off + 1, 0), Sk) only.  A row with no
 * visible key has an empty sum, l = 0 and o = 0/0 = NaN, the same result the
 * formula gives when every logit of a row is -Inf.
 *
 * Grouped K/V heads.  The same page lists GQA among what the kernel leaves
 * out (section "Hvad er udgivet" / What was released), again without a
 * definition.  Read as the usual one: K and V hold H_kv heads, H is a
 * multiple of H_kv, and query head h attends with K/V head h / (H / H_kv)
 * (consecutive query heads share one K/V head).  Everything else is as above.
 *
 * Log-sum-exp.  Per query row, lse = log(sum_j exp(s_j)) over the keys the
 * row sees (natural log, the logits of step 2), the per-row statistic the
 * FlashAttention family keeps for a backward pass or for merging key ranges;
 * the pages do not discuss it (an extension beside grouped heads and packed
 * batches).  Evaluated as m + log(l) from steps 3-4 when m is finite; -Inf
 * when the row sees no key or only -Inf logits (the log of an empty or zero
 * sum); NaN when m is NaN or +Inf (the rows whose output is NaN as well).
 *
 * Pins (tests/test_oracle_*.py): closed forms, invariants, brute force on
 * tiny inputs, a library softmax cross-check and exhaustive/definitional
 * checks of the rounding and decoding.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 *        -pthread attn_oracle.c -lm -o liboracle.so
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D 128

/* Oracle's own enum values (same order as the pages list the modes). */
enum { OR_RTNE = 0, OR_RTNA = 1, OR_RTZ = 2 };
/* Oracle's own layout codes. BSHD: [B, S, H, D]; BHSD: [B, H, S, D]. */
enum { OR_BSHD = 0, OR_BHSD = 1 };
/* Oracle's own mask codes: none, causal aligned top left, causal aligned bottom right. */
enum { OR_MASK_NONE = 0, OR_MASK_CAUSAL_TOP_LEFT = 1, OR_MASK_CAUSAL_BOTTOM_RIGHT = 2 };

/* ------------------------------------------------------------------------
 * bf16 <-> binary64, from the format definition
 *   bf16 = 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * ---------------------------------------------------------------------- */
double oracle_bf16_decode(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double mag;
    if (e == 0xFF) {
        mag = f ? NAN : INFINITY;
    } else if (e == 0) {
        mag = ldexp((double)f, -126 - 7); /* subnormal: f/128 * 2^-126 */
    } else {
        mag = ldexp((double)(128 + f), e - 127 - 7); /* (1 + f/128) * 2^(e-127) */
    }
    return sign ? -mag : mag;
}

/* Round a binary64 value to bf16 bits in one step.
 * NaN -> 0x7FC0 (sign and payload are not part of the contract);
 * +-Inf -> +-Inf; +-0 -> +-0.
 * Otherwise: e = max(floor(log2|x|), -126), ulp = 2^(e-7), t = |x|/ulp (exact),
 * f = floor(t), r = t - f (exact), n = f rounded up by the mode's rule:
 *   RTZ never, RTNE when r > 1/2 or (r == 1/2 and f odd), RTNA when r >= 1/2.
 * Result = n * ulp with n = 256 carrying into the next binade. Past the bf16
 * maximum the nearest modes give Inf and RTZ gives the maximum finite value.
 */
uint16_t oracle_round_bf16(double x, int mode)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int E;
    (void)frexp(a, &E); /* a = fr * 2^E, fr in [0.5, 1): floor(log2 a) = E - 1 */
    int e = E - 1;
    if (e < -126)
        e = -126;
    double t = ldexp(a, 7 - e); /* a / ulp, exact (power-of-two scaling) */
    double f = floor(t);
    double r = t - f;
    double n = f;
    if (mode == OR_RTNE) {
        if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) == 1.0))
            n = f + 1.0;
    } else if (mode == OR_RTNA) {
        if (r >= 0.5)
            n = f + 1.0;
    } /* OR_RTZ: n = f */
    if (n == 256.0) {
        n = 128.0;
        e += 1;
    }
    if (n < 128.0) /* only reachable in the subnormal binade (e == -126) */
        return sign | (uint16_t)n;
    int field = e + 127;
    if (field >= 0xFF) /* overflow */
        return mode == OR_RTZ ? (sign | 0x7F7F) : (sign | 0x7F80);
    return sign | (uint16_t)((field << 7) | ((int)n - 128));
}

void oracle_round_array(const double *x, int64_t n, int mode, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_round_bf16(x[i], mode);
}

void oracle_decode_array(const uint16_t *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_decode(b[i]);
}

/* ------------------------------------------------------------------------
 * layout addressing: element (b, h, s, c) of a tensor with S rows per head
 * ---------------------------------------------------------------------- */
static int64_t offset_of(int layout, int64_t H, int64_t S, int64_t b, int64_t h, int64_t s, int64_t c)
{
    if (layout == OR_BSHD)
        return ((b * S + s) * H + h) * D + c;
    return ((b * H + h) * S + s) * D + c;
}

/* propagating maximum: NaN if either argument is NaN */
static double max_nan(double a, double b)
{
    if (isnan(a) || isnan(b))
        return NAN;
    return a > b ? a : b;
}

/* Number of keys query row i attends to (the causal reading in the header). */
static int64_t visible_keys(int mask, int64_t i, int64_t Sq, int64_t Sk)
{
    if (mask == OR_MASK_NONE)
        return Sk;
    const int64_t off = mask == OR_MASK_CAUSAL_TOP_LEFT ? 0 : Sk - Sq;
    int64_t n = i + off + 1;
    if (n < 0)
        n = 0;
    return n < Sk ? n : Sk;
}

/* Steps 2-4 for one query row against the first Sk keys of a decoded head.
 * On return w[j] holds exp(s_j - m), *m_out the maximum m (-Inf when there
 * are no keys), and the function returns l = sum_j w_j (0 when there are no
 * keys). */
static double row_weights(const double *qrow, const double *Kd, int64_t Sk, double *w, double *m_out)
{
    *m_out = -INFINITY;
    if (Sk == 0)
        return 0.0;
    const double sqrt_d = sqrt((double)D);
    for (int64_t j = 0; j < Sk; ++j) {
        const double *kr = Kd + j * D;
        double acc = 0.0;
        for (int c = 0; c < D; ++c)
            acc += qrow[c] * kr[c];
        w[j] = acc / sqrt_d;
    }
    double m = w[0];
    for (int64_t j = 1; j < Sk; ++j)
        m = max_nan(m, w[j]);
    double l = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        w[j] = exp(w[j] - m);
        l += w[j];
    }
    *m_out = m;
    return l;
}

/* The log-sum-exp of a row from its maximum and shifted sum (see the header). */
static double row_lse(double m, double l)
{
    if (isfinite(m))
        return m + log(l);
    if (m == -INFINITY)
        return -INFINITY;
    return NAN;
}

/* Step 5 for one row. */
static void row_output(const double *w, double l, const double *Vd, int64_t Sk, double *o)
{
    double acc[D];
    for (int c = 0; c < D; ++c)
        acc[c] = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        const double *vr = Vd + j * D;
        for (int c = 0; c < D; ++c)
            acc[c] += w[j] * vr[c]; /* each acc[c] sums in ascending j */
    }
    for (int c = 0; c < D; ++c)
        o[c] = acc[c] / l;
}

typedef struct {
    const uint16_t *q;
    int64_t H, Sq, b, h;
    int layout;
    const double *Kd, *Vd;
    int64_t Sk;
    int mask;
    const int64_t *rows; /* triples */
    int64_t lo, hi;      /* row range within rows */
    double *o_exact;     /* nrows x D */
    uint16_t *o_round;   /* nrows x 3 x D */
    double *lse;         /* nrows, or NULL */
    int ok;
} job_t;

static void *run_job(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *w = (double *)malloc(sizeof(double) * (size_t)jb->Sk);
    if (!w) {
        jb->ok = 0;
        return NULL;
    }
    double qrow[D];
    for (int64_t r = jb->lo; r < jb->hi; ++r) {
        int64_t i = jb->rows[3 * r + 2];
        for (int c = 0; c < D; ++c)
            qrow[c] = oracle_bf16_decode(jb->q[offset_of(jb->layout, jb->H, jb->Sq, jb->b, jb->h, i, c)]);
        const int64_t n = visible_keys(jb->mask, i, jb->Sq, jb->Sk);
        double m;
        double l = row_weights(qrow, jb->Kd, n, w, &m);
        double *o = jb->o_exact + r * D;
        row_output(w, l, jb->Vd, n, o);
        if (jb->lse)
            jb->lse[r] = row_lse(m, l);
        for (int mode = 0; mode < 3; ++mode)
            for (int c = 0; c < D; ++c)
                jb->o_round[(r * 3 + mode) * D + c] = oracle_round_bf16(o[c], mode);
    }
    free(w);
    jb->ok = 1;
    return NULL;
}

/* Decode head (b, h) of a K or V tensor of H heads into a dense [S][D] binary64 array. */
static void decode_head(const uint16_t *t, int layout, int64_t H, int64_t S, int64_t b, int64_t h, double *out)
{
    for (int64_t s = 0; s < S; ++s)
        for (int c = 0; c < D; ++c)
            out[s * D + c] = oracle_bf16_decode(t[offset_of(layout, H, S, b, h, s, c)]);
}

/*
 * oracle_attn_rows_gqa: exact outputs and their three bf16 roundings for a
 * list of query rows.
 *   q: [B,Sq,H,128] (BSHD) or [B,H,Sq,128] (BHSD) bf16 bits; k, v likewise
 *   with Sk rows and H_kv heads (H a multiple of H_kv).
 *   mask: OR_MASK_NONE, OR_MASK_CAUSAL_TOP_LEFT or OR_MASK_CAUSAL_BOTTOM_RIGHT.
 *   rows: nrows triples (b, h, i); rows with equal (b, h) must be adjacent.
 *   lse: nrows binary64 log-sum-exp values, or NULL.
 *   o_exact: nrows x 128 binary64;  o_round: nrows x 3 x 128 bf16 bits
 *   (modes in the order RTNE, RTNA, RTZ).
 *   nthreads: worker threads (rows of one head are split among them).
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_attn_rows_gqa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int layout, int mask,
                         const int64_t *rows, int64_t nrows,
                         double *o_exact, uint16_t *o_round, double *lse, int nthreads)
{
    if (!q || !k || !v || !rows || !o_exact || !o_round)
        return -1;
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || Sq < 1 || Sk < 1 ||
        (layout != OR_BSHD && layout != OR_BHSD))
        return -1;
    const int64_t group = H / H_kv; /* query heads per K/V head */
    if (mask != OR_MASK_NONE && mask != OR_MASK_CAUSAL_TOP_LEFT && mask != OR_MASK_CAUSAL_BOTTOM_RIGHT)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Sq)
            return -1;
    }
    double *Kd = (double *)malloc(sizeof(double) * (size_t)(Sk * D));
    double *Vd = (double *)malloc(sizeof(double) * (size_t)(Sk * D));
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!Kd || !Vd || !jobs || !th) {
        free(Kd), free(Vd), free(jobs), free(th);
        return -2;
    }
    int status = 0;
    int64_t r0 = 0;
    while (r0 < nrows && status == 0) {
        int64_t b = rows[3 * r0], h = rows[3 * r0 + 1];
        int64_t r1 = r0;
        while (r1 < nrows && rows[3 * r1] == b && rows[3 * r1 + 1] == h)
            ++r1;
        decode_head(k, layout, H_kv, Sk, b, h / group, Kd);
        decode_head(v, layout, H_kv, Sk, b, h / group, Vd);
        int64_t n = r1 - r0;
        int nt = (int64_t)nthreads < n ? nthreads : (int)n;
        for (int t = 0; t < nt; ++t) {
            job_t *jb = &jobs[t];
            jb->q = q, jb->H = H, jb->Sq = Sq, jb->b = b, jb->h = h, jb->layout = layout;
            jb->Kd = Kd, jb->Vd = Vd, jb->Sk = Sk, jb->mask = mask, jb->rows = rows;
            jb->lo = r0 + n * t / nt, jb->hi = r0 + n * (t + 1) / nt;
            jb->o_exact = o_exact, jb->o_round = o_round, jb->lse = lse, jb->ok = 0;
        }
        int started = 0;
        for (int t = 1; t < nt; ++t) {
            if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0)
                break;
            started = t;
        }
        run_job(&jobs[0]);
        for (int t = 1; t <= started; ++t)
            pthread_join(th[t], NULL);
        for (int t = started + 1; t < nt; ++t) /* threads that could not start */
            run_job(&jobs[t]);
        for (int t = 0; t < nt; ++t)
            if (!jobs[t].ok)
                status = -2;
        r0 = r1;
    }
    free(Kd), free(Vd), free(jobs), free(th);
    return status;
}

/* oracle_attn_rows_masked: oracle_attn_rows_gqa with one K/V head per query head. */
int oracle_attn_rows_masked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int64_t B, int64_t H, int64_t Sq, int64_t Sk, int layout, int mask,
                            const int64_t *rows, int64_t nrows,
                            double *o_exact, uint16_t *o_round, int nthreads)
{
    return oracle_attn_rows_gqa(q, k, v, B, H, H, Sq, Sk, layout, mask, rows, nrows, o_exact, o_round, NULL,
                                nthreads);
}

/* oracle_attn_rows: the unmasked case of oracle_attn_rows_masked. */
int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int64_t B, int64_t H, int64_t Sq, int64_t Sk, int layout,
                     const int64_t *rows, int64_t nrows,
                     double *o_exact, uint16_t *o_round, int nthreads)
{
    return oracle_attn_rows_masked(q, k, v, B, H, Sq, Sk, layout, OR_MASK_NONE, rows, nrows, o_exact, o_round,
                                   nthreads);
}

/*
 * oracle_softmax_row: the normalised weights w_j / l of one query row
 * (steps 1-4), for the rows-sum-to-one pin. w: Sk binary64. Returns l.
 */
double oracle_softmax_row(const uint16_t *q, const uint16_t *k,
                          int64_t B, int64_t H, int64_t Sq, int64_t Sk, int layout,
                          int64_t b, int64_t h, int64_t i, double *w)
{
    (void)B;
    double *Kd = (double *)malloc(sizeof(double) * (size_t)(Sk * D));
    if (!Kd)
        return NAN;
    decode_head(k, layout, H, Sk, b, h, Kd);
    double qrow[D];
    for (int c = 0; c < D; ++c)
        qrow[c] = oracle_bf16_decode(q[offset_of(layout, H, Sq, b, h, i, c)]);
    double m;
    double l = row_weights(qrow, Kd, Sk, w, &m);
    for (int64_t j = 0; j < Sk; ++j)
        w[j] /= l;
    free(Kd);
    return l;
}
