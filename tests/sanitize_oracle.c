/*
 * The C oracle (oracle/attn_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Runs every exported oracle function on small inputs that reach its edge cases (empty rows and
 * columns, fully masked rows, causal masks with more queries than keys and the reverse, one and
 * several threads, block sizes of 1, uneven and larger than the problem, all 256 e4m3 codes), plus
 * arguments each function must refuse.  Besides the sanitizers' own checks, results are compared
 * across the oracle's independent routes (the definition, selected rows, the blockwise form, the
 * element-wise online normaliser) and against invariants of softmax:
 *   - each probability row sums to 1 ("digest_existing.txt", answer q02_flashattention, section 1);
 *   - the gradient rows satisfy sum_j dK_j = 0 and sum_j dV_j = sum of dO over the rows that see a
 *     key (P's rows sum to 1);
 *   - a row that sees no key has O = 0 and lse = -inf.
 * The inputs come from a fixed linear congruential generator.  Exit status 0 when all agree.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_softmax_rows(const double *x, long rows, long cols, double *p, double *lse);
int oracle_online_merge(const double *x, long n, const long *cuts, long ncuts, double *m, double *l);
int oracle_online_normalizer(const double *x, long n, double *m, double *d);
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse, double *p_out, long B,
                    long H, long nq, long nk, long d, int causal, double scale, int nthreads);
int oracle_attn_fwd_rows(const double *qrows, const long *row_idx, long R, const double *k, const double *v, long nq,
                         long nk, long d, int causal, double scale, double *o, double *lse);
int oracle_attn_fwd_blockwise(const double *q, const double *k, const double *v, long nq, long nk, long d, int causal,
                              double scale, long br, long bc, double *o, double *lse, double *m_out, double *l_out);
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout, double *dq, double *dk,
                    double *dv, double *dvec, long B, long H, long nq, long nk, long d, int causal, double scale,
                    int nthreads);
int oracle_fp8_e4m3_decode(const unsigned char *x, long n, double *out);

static int g_fail = 0, g_checks = 0;

static void check(int ok, const char *what, long a, long b)
{
    ++g_checks;
    if (!ok) {
        ++g_fail;
        fprintf(stderr, "FAILED %s (%ld, %ld)\n", what, a, b);
    }
}

static unsigned long long g_state = 0x9e3779b97f4a7c15ULL;

static double uniform(void) /* in [-1, 1) */
{
    g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(g_state >> 11) / 4503599627370496.0 - 1.0;
}

/* malloc of n doubles (at least one), filled with uniform values times amp */
static double *rnd(long n, double amp)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    long i;
    for (i = 0; i < n; ++i)
        x[i] = amp * uniform();
    return x;
}

static double *zeros(long n) { return (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

static int close_to(double a, double b, double tol)
{
    if (isinf(a) || isinf(b))
        return a == b;
    return fabs(a - b) <= tol * (1.0 + fabs(b));
}

static void softmax_cases(void)
{
    const long rows = 4, cols = 7;
    double *x = rnd(rows * cols, 3.0), *p = zeros(rows * cols), lse[4], m, l, dd;
    long r, j, cuts[3] = {1, 3, 6}, bad[2] = {3, 3};
    for (j = 0; j < cols; ++j)
        x[1 * cols + j] = -INFINITY; /* row 1: nothing but -inf */
    x[2 * cols + 0] = -INFINITY;     /* row 2: one -inf */
    check(oracle_softmax_rows(x, rows, cols, p, lse) == 0, "softmax_rows", 0, 0);
    for (r = 0; r < rows; ++r) {
        double s = 0.0;
        for (j = 0; j < cols; ++j)
            s += p[r * cols + j];
        if (r == 1)
            check(isinf(lse[r]) && lse[r] < 0 && s == 0.0, "all -inf row: lse = -inf, p = 0", r, 0);
        else
            check(fabs(s - 1.0) < 1e-13, "softmax row sums to 1", r, 0);
        check(oracle_online_normalizer(x + r * cols, cols, &m, &dd) == 0, "normalizer", r, 0);
        check(close_to(isinf(m) ? m : m + log(dd), lse[r], 1e-13), "normalizer lse = softmax lse", r, 0);
        check(oracle_online_merge(x + r * cols, cols, cuts, 3, &m, &l) == 0, "merge", r, 0);
        check(close_to(isinf(m) ? m : m + log(l), lse[r], 1e-13), "merge lse = softmax lse", r, 0);
        check(oracle_online_merge(x + r * cols, cols, NULL, 0, &m, &l) == 0, "merge, one block", r, 0);
        check(close_to(isinf(m) ? m : m + log(l), lse[r], 1e-13), "one-block merge lse", r, 0);
    }
    check(oracle_softmax_rows(x, 0, cols, p, lse) == 0, "no rows", 0, 0);
    check(oracle_online_normalizer(x, 0, &m, &dd) == 0 && isinf(m) && dd == 0.0, "empty normalizer", 0, 0);
    check(oracle_online_merge(x, cols, bad, 2, &m, &l) == -1, "merge refuses repeated cuts", 0, 0);
    check(oracle_online_merge(x, 0, NULL, 0, &m, &l) == -1, "merge refuses n = 0", 0, 0);
    check(oracle_softmax_rows(NULL, 1, 1, p, lse) == -1, "softmax refuses NULL", 0, 0);
    check(oracle_online_normalizer(x, -1, &m, &dd) == -1, "normalizer refuses n < 0", 0, 0);
    free(x);
    free(p);
}

/* one attention problem through every route */
static void attention_case(long B, long H, long nq, long nk, long d, int causal, int nthreads)
{
    const long nh = B * H, qn = nh * nq * d, kn = nh * nk * d;
    const double scale = 1.0 / sqrt((double)d);
    double *q = rnd(qn, 2.0), *k = rnd(kn, 2.0), *v = rnd(kn, 1.0), *dout = rnd(qn, 1.0);
    double *o = zeros(qn), *lse = zeros(nh * nq), *p = zeros(nh * nq * nk);
    double *dq = zeros(qn), *dk = zeros(kn), *dv = zeros(kn), *dvec = zeros(nh * nq);
    double *ob = zeros(nq * d), *lb = zeros(nq), *mb = zeros(nq), *lbl = zeros(nq), *orow = zeros(d);
    long *idx = (long *)malloc(sizeof(long) * (size_t)(nq > 0 ? nq : 1));
    long h, i, j, c, bi, bj;
    const long blocks[4] = {1, 3, 64, 1000};

    check(oracle_attn_fwd(q, k, v, o, lse, p, B, H, nq, nk, d, causal, scale, nthreads) == 0, "fwd", nq, nk);
    check(oracle_attn_bwd(q, k, v, dout, dq, dk, dv, dvec, B, H, nq, nk, d, causal, scale, nthreads) == 0, "bwd", nq,
          nk);
    for (h = 0; h < nh; ++h) {
        const double *qh = q + h * nq * d, *kh = k + h * nk * d, *vh = v + h * nk * d;
        for (i = 0; i < nq; ++i) {
            const double *oi = o + (h * nq + i) * d;
            double s = 0.0;
            int sees = 0;
            for (j = 0; j < nk; ++j) {
                s += p[(h * nq + i) * nk + j];
                if (!causal || j <= i + (nk - nq))
                    sees = 1;
            }
            if (sees) {
                check(fabs(s - 1.0) < 1e-12 && isfinite(lse[h * nq + i]), "P row sums to 1", h, i);
            } else {
                check(isinf(lse[h * nq + i]) && lse[h * nq + i] < 0 && s == 0.0, "unseen row: lse -inf", h, i);
                for (c = 0; c < d; ++c)
                    check(oi[c] == 0.0 && dq[(h * nq + i) * d + c] == 0.0, "unseen row: O = 0, dQ = 0", h, i);
            }
            /* the selected-rows route, one row at a time */
            idx[0] = i;
            check(oracle_attn_fwd_rows(qh + i * d, idx, 1, kh, vh, nq, nk, d, causal, scale, orow, lb) == 0, "rows",
                  h, i);
            for (c = 0; c < d; ++c)
                check(close_to(orow[c], oi[c], 1e-13), "rows = definition", h, i);
            check(close_to(lb[0], lse[h * nq + i], 1e-13), "rows lse = definition", h, i);
        }
        /* the blockwise route at several block shapes */
        for (bi = 0; bi < 4; ++bi)
            for (bj = 0; bj < 4; ++bj) {
                check(oracle_attn_fwd_blockwise(qh, kh, vh, nq, nk, d, causal, scale, blocks[bi], blocks[bj], ob, lb,
                                                mb, lbl) == 0,
                      "blockwise", blocks[bi], blocks[bj]);
                for (i = 0; i < nq; ++i) {
                    check(close_to(lb[i], lse[h * nq + i], 1e-12), "blockwise lse", blocks[bi], blocks[bj]);
                    for (c = 0; c < d; ++c)
                        check(close_to(ob[i * d + c], o[(h * nq + i) * d + c], 1e-12), "blockwise O", blocks[bi],
                              blocks[bj]);
                }
            }
        /* gradient invariants: sum_j dK_j = 0, sum_j dV_j = sum of dO over rows that see a key */
        for (c = 0; c < d; ++c) {
            double sk = 0.0, sv = 0.0, sd = 0.0, mag = 1.0;
            for (j = 0; j < nk; ++j) {
                sk += dk[(h * nk + j) * d + c];
                sv += dv[(h * nk + j) * d + c];
                mag += fabs(dk[(h * nk + j) * d + c]);
            }
            for (i = 0; i < nq; ++i)
                if (isfinite(lse[h * nq + i]))
                    sd += dout[(h * nq + i) * d + c];
            check(fabs(sk) <= 1e-11 * mag, "sum dK = 0", h, c);
            check(fabs(sv - sd) <= 1e-11 * (1.0 + fabs(sd)), "sum dV = sum dO", h, c);
        }
        /* D_i = <dO_i, O_i> */
        for (i = 0; i < nq; ++i) {
            double s = 0.0;
            for (c = 0; c < d; ++c)
                s += dout[(h * nq + i) * d + c] * o[(h * nq + i) * d + c];
            check(close_to(dvec[h * nq + i], s, 1e-12), "D = rowsum(dO * O)", h, i);
        }
    }
    free(q); free(k); free(v); free(dout); free(o); free(lse); free(p);
    free(dq); free(dk); free(dv); free(dvec); free(ob); free(lb); free(mb); free(lbl); free(orow); free(idx);
}

static void refusals(void)
{
    double x[64] = {0}, y[64] = {0};
    long bad_row = 5;
    check(oracle_attn_fwd(NULL, x, x, y, y, NULL, 1, 1, 2, 2, 4, 0, 1.0, 1) == -1, "fwd refuses NULL q", 0, 0);
    check(oracle_attn_fwd(x, x, x, y, y, NULL, -1, 1, 2, 2, 4, 0, 1.0, 1) == -1, "fwd refuses B < 0", 0, 0);
    check(oracle_attn_fwd(x, x, x, y, y, NULL, 1, 1, 2, 2, 0, 0, 1.0, 1) == -1, "fwd refuses d = 0", 0, 0);
    check(oracle_attn_bwd(x, x, x, x, y, y, NULL, NULL, 1, 1, 2, 2, 4, 0, 1.0, 1) == -1, "bwd refuses NULL dv", 0, 0);
    check(oracle_attn_fwd_rows(x, &bad_row, 1, x, x, 4, 4, 4, 0, 1.0, y, y) == -1, "rows refuses a row past nq", 0, 0);
    check(oracle_attn_fwd_blockwise(x, x, x, 2, 2, 4, 0, 1.0, 0, 1, y, NULL, NULL, NULL) == -1, "blockwise br = 0", 0,
          0);
    check(oracle_fp8_e4m3_decode(NULL, 3, y) == -1, "decode refuses NULL", 0, 0);
    /* empty problems are fine */
    check(oracle_attn_fwd(x, x, x, y, y, NULL, 0, 3, 2, 2, 4, 1, 1.0, 4) == 0, "fwd, B = 0", 0, 0);
    check(oracle_attn_bwd(x, x, x, x, y, y, y, NULL, 2, 0, 2, 2, 4, 1, 1.0, 4) == 0, "bwd, H = 0", 0, 0);
}

static void fp8_codes(void)
{
    unsigned char codes[256];
    double val[256];
    int i;
    for (i = 0; i < 256; ++i)
        codes[i] = (unsigned char)i;
    check(oracle_fp8_e4m3_decode(codes, 256, val) == 0, "decode", 0, 0);
    for (i = 0; i < 256; ++i) {
        if ((i & 0x7f) == 0x7f)
            check(isnan(val[i]), "e4m3 0x7f / 0xff is NaN", i, 0);
        else
            check(isfinite(val[i]) && fabs(val[i]) <= 448.0, "e4m3 finite and within 448", i, 0);
        if (i < 128 && (i & 0x7f) != 0x7f)
            check(val[i] == -val[i + 128], "sign bit negates", i, 0);
        if (i > 0 && i < 127)
            check(val[i] > val[i - 1], "codes 0..126 increase", i, 0);
    }
    check(val[0x7e] == 448.0 && val[1] == ldexp(1.0, -9), "largest 448, smallest subnormal 2^-9", 0, 0);
}

int main(void)
{
    softmax_cases();
    /* B, H, nq, nk, d, causal, threads */
    attention_case(1, 1, 5, 5, 4, 0, 1);
    attention_case(1, 2, 5, 5, 4, 1, 2);
    attention_case(2, 1, 7, 3, 8, 1, 3);  /* more queries than keys: rows 0..3 see nothing */
    attention_case(1, 1, 3, 9, 8, 1, 5);  /* more keys than queries: bottom-right alignment */
    attention_case(1, 3, 6, 11, 4, 0, 7); /* more threads than heads */
    attention_case(1, 1, 4, 0, 4, 0, 2);  /* no keys */
    attention_case(1, 1, 4, 0, 4, 1, 1);
    attention_case(1, 1, 0, 6, 4, 1, 2);  /* no queries */
    attention_case(1, 1, 1, 1, 1, 1, 1);
    refusals();
    fp8_codes();
    printf("oracle checks: %d, failed %d\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
