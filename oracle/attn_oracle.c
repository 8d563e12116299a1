/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of exact scaled-dot-product attention
 * (forward and backward).  It exists to check the GPU library: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the GPU path.
 *
 * What it follows (pages the method is described on):
 *   [digest]  "digest_existing.txt" of the xtrax package, answer
 *             q02_flashattention.  Section 1: standard attention materialises
 *             S = Q K^T and P = softmax(S) as N x N matrices.  Section 2: the
 *             running max m(x) and exp-sum l(x) of a partitioned vector merge as
 *             m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2, softmax = f(x)/l(x);
 *             FlashAttention's initialisation is l = 0, m = -inf, O = 0.
 *   [gpko]    "GPU Programming and Kernel Optimization" (ai.engineer), item 57
 *             (online normaliser m' = max(m, x), d' = d e^(m-m') + e^(x-m')),
 *             item 58 (FlashAttention: block statistics are rescaled to a common
 *             maximum and the output accumulators get the same rescaling; the
 *             backward regenerates scores from saved statistics), item 59 (causal
 *             masks aligned to the bottom-right corner when query and key lengths
 *             differ; fully masked rows have zero output), item 60 (a maximum of
 *             -inf is handled, no division by a zero denominator), item 51 (row
 *             softmax: subtract the row max, exponentiate, sum, divide).
 *
 * Layout: every tensor is a dense row-major fp64 array [B, H, N, d] (Q, dO, O,
 * dQ: N = nq; K, V, dK, dV: N = nk); lse and D are [B, H, nq].
 *
 * Readings where the pages say nothing (each also listed with the design notes):
 *   - lse is the natural log of sum_j exp(s_ij) over the scaled scores.
 *   - A fully masked row has O = 0 and lse = -inf (item 59 and item 60).
 *   - The backward pass is not printed on the pages (the digest answer is cut
 *     off); it is the chain rule of the forward definition, written out below.
 *
 * Every function returns 0 on success and -1 on a bad argument.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* Key j is visible to query i (both 0-based) when not causal, or when causal
 * and j <= i + (nk - nq): the mask is aligned to the bottom-right corner
 * ([gpko] item 59).  With nq == nk this is the usual j <= i. */
static int visible(long i, long j, long nq, long nk, int causal)
{
    return !causal || j <= i + (nk - nq);
}

/* Softmax of one row that may hold -inf entries ([gpko] item 51): subtract the
 * row maximum, exponentiate, sum, divide.  A row that is entirely -inf gives
 * all zeros and returns -inf ([gpko] items 59, 60: zero output, no division by
 * zero).  Returns the row's natural-log sum-exp. */
static double softmax_row(const double *s, long n, double *p)
{
    double m = -INFINITY, z = 0.0;
    long j;
    for (j = 0; j < n; ++j)
        if (s[j] > m)
            m = s[j];
    if (m == -INFINITY) {
        for (j = 0; j < n; ++j)
            p[j] = 0.0;
        return -INFINITY;
    }
    for (j = 0; j < n; ++j) {
        p[j] = exp(s[j] - m); /* exp(-inf) = 0 for masked entries */
        z += p[j];
    }
    for (j = 0; j < n; ++j)
        p[j] /= z;
    return m + log(z);
}

/* Row softmax of a rows x cols matrix; lse (may be NULL) gets each row's
 * natural-log sum-exp. */
int oracle_softmax_rows(const double *x, long rows, long cols, double *p, double *lse)
{
    long r;
    if (!x || !p || rows < 0 || cols < 0)
        return -1;
    for (r = 0; r < rows; ++r) {
        double l = softmax_row(x + r * cols, cols, p + r * cols);
        if (lse)
            lse[r] = l;
    }
    return 0;
}

/* The merge rule of [digest] section 2, applied left to right over the blocks
 * of x delimited by cuts[0..ncuts-1] (strictly increasing, inside (0, n)).
 * Each block's own statistics are computed directly (its max and the sum of
 * exponentials shifted by that max); blocks are then merged pairwise.
 * Returns the merged max in *m and exp-sum in *l. */
int oracle_online_merge(const double *x, long n, const long *cuts, long ncuts, double *m, double *l)
{
    double mm = -INFINITY, ll = 0.0; /* statistics of the empty prefix: m = -inf, l = 0 */
    long b, lo = 0;
    if (!x || !m || !l || n < 1 || ncuts < 0 || (ncuts > 0 && !cuts))
        return -1;
    for (b = 0; b <= ncuts; ++b) {
        long hi = (b < ncuts) ? cuts[b] : n, j;
        double mb = -INFINITY, lb = 0.0, mnew, lnew;
        if (hi <= lo || hi > n)
            return -1;
        for (j = lo; j < hi; ++j)
            if (x[j] > mb)
                mb = x[j];
        if (mb != -INFINITY)
            for (j = lo; j < hi; ++j)
                lb += exp(x[j] - mb);
        mnew = mm > mb ? mm : mb;
        if (mnew == -INFINITY) {
            lnew = 0.0;
        } else {
            lnew = (mm == -INFINITY ? 0.0 : exp(mm - mnew) * ll) + (mb == -INFINITY ? 0.0 : exp(mb - mnew) * lb);
        }
        mm = mnew;
        ll = lnew;
        lo = hi;
    }
    *m = mm;
    *l = ll;
    return 0;
}

/* The element-at-a-time online normaliser of [gpko] item 57:
 * m' = max(m, x), d' = d e^(m - m') + e^(x - m'), starting from m = -inf, d = 0. */
int oracle_online_normalizer(const double *x, long n, double *m, double *d)
{
    double mm = -INFINITY, dd = 0.0;
    long j;
    if (!x || !m || !d || n < 0)
        return -1;
    for (j = 0; j < n; ++j) {
        double mn = x[j] > mm ? x[j] : mm;
        if (mn == -INFINITY)
            continue; /* still nothing but -inf: m and d stay at -inf and 0 */
        dd = (mm == -INFINITY ? 0.0 : dd * exp(mm - mn)) + exp(x[j] - mn);
        mm = mn;
    }
    *m = mm;
    *d = dd;
    return 0;
}

/* One query row of one head, by the definition ([digest] section 1):
 * materialise the score row s_j = scale * <q_i, k_j> (-inf where masked),
 * take its softmax p, and form o_i = sum_j p_j v_j.  Returns lse_i. */
static double attend_row(const double *qi, long i, const double *K, const double *V, long nq, long nk, long d,
                         int causal, double scale, double *s, double *p, double *oi)
{
    long j, c;
    double lse;
    for (j = 0; j < nk; ++j) {
        if (visible(i, j, nq, nk, causal)) {
            double acc = 0.0;
            for (c = 0; c < d; ++c)
                acc += qi[c] * K[j * d + c];
            s[j] = scale * acc;
        } else {
            s[j] = -INFINITY;
        }
    }
    lse = softmax_row(s, nk, p);
    for (c = 0; c < d; ++c)
        oi[c] = 0.0;
    for (j = 0; j < nk; ++j) {
        if (p[j] == 0.0)
            continue;
        for (c = 0; c < d; ++c)
            oi[c] += p[j] * V[j * d + c];
    }
    return lse;
}

/* ---- threading over (batch, head) pairs ---------------------------------- */

typedef struct {
    const double *q, *k, *v, *dout;
    double *o, *lse, *pmat, *dq, *dk, *dv, *dvec;
    long nheads, nq, nk, d;
    int causal, nthreads, tid, status;
    double scale;
} job_t;

static void *fwd_worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    long h, i;
    double *s = (double *)malloc(sizeof(double) * (size_t)(jb->nk > 0 ? jb->nk : 1));
    double *p = (double *)malloc(sizeof(double) * (size_t)(jb->nk > 0 ? jb->nk : 1));
    if (!s || !p) {
        jb->status = -1;
        free(s);
        free(p);
        return NULL;
    }
    for (h = jb->tid; h < jb->nheads; h += jb->nthreads) {
        const double *Q = jb->q + h * jb->nq * jb->d;
        const double *K = jb->k + h * jb->nk * jb->d;
        const double *V = jb->v + h * jb->nk * jb->d;
        for (i = 0; i < jb->nq; ++i) {
            double l = attend_row(Q + i * jb->d, i, K, V, jb->nq, jb->nk, jb->d, jb->causal, jb->scale, s, p,
                                  jb->o + (h * jb->nq + i) * jb->d);
            if (jb->lse)
                jb->lse[h * jb->nq + i] = l;
            if (jb->pmat)
                memcpy(jb->pmat + (h * jb->nq + i) * jb->nk, p, sizeof(double) * (size_t)jb->nk);
        }
    }
    free(s);
    free(p);
    return NULL;
}

static int run_threads(job_t *proto, int nthreads, void *(*fn)(void *))
{
    pthread_t th[256];
    job_t jobs[256];
    int t, started = 0, status = 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > proto->nheads && proto->nheads > 0)
        nthreads = (int)proto->nheads;
    for (t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
        jobs[t].status = 0;
    }
    for (t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0)
            break;
        started = t;
    }
    /* threads that could not be started are run on this thread */
    for (t = started + 1; t < nthreads; ++t)
        fn(&jobs[t]);
    fn(&jobs[0]);
    for (t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    for (t = 0; t < nthreads; ++t)
        if (jobs[t].status)
            status = jobs[t].status;
    return status;
}

/* Forward pass by the definition, for all B*H heads.  o: [B,H,nq,d],
 * lse: [B,H,nq] (may be NULL), p_out: [B,H,nq,nk] or NULL (the probability
 * matrix P, materialised row by row). */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse, double *p_out, long B,
                    long H, long nq, long nk, long d, int causal, double scale, int nthreads)
{
    job_t jb;
    if (!q || !k || !v || !o || B < 0 || H < 0 || nq < 0 || nk < 0 || d < 1)
        return -1;
    memset(&jb, 0, sizeof jb);
    jb.q = q;
    jb.k = k;
    jb.v = v;
    jb.o = o;
    jb.lse = lse;
    jb.pmat = p_out;
    jb.nheads = B * H;
    jb.nq = nq;
    jb.nk = nk;
    jb.d = d;
    jb.causal = causal;
    jb.scale = scale;
    if (jb.nheads == 0 || nq == 0)
        return 0;
    return run_threads(&jb, nthreads, fwd_worker);
}

/* Forward pass for R selected query rows of ONE head: qrows [R,d] are the
 * rows' query vectors, row_idx[r] their 0-based positions (for the mask),
 * k, v: [nk, d] of that head.  Same definition as oracle_attn_fwd. */
int oracle_attn_fwd_rows(const double *qrows, const long *row_idx, long R, const double *k, const double *v, long nq,
                         long nk, long d, int causal, double scale, double *o, double *lse)
{
    long r;
    double *s, *p;
    if (!qrows || !row_idx || !k || !v || !o || R < 0 || nq < 0 || nk < 0 || d < 1)
        return -1;
    s = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    p = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    if (!s || !p) {
        free(s);
        free(p);
        return -1;
    }
    for (r = 0; r < R; ++r) {
        double l;
        if (row_idx[r] < 0 || row_idx[r] >= nq) {
            free(s);
            free(p);
            return -1;
        }
        l = attend_row(qrows + r * d, row_idx[r], k, v, nq, nk, d, causal, scale, s, p, o + r * d);
        if (lse)
            lse[r] = l;
    }
    free(s);
    free(p);
    return 0;
}

/* FlashAttention's blockwise forward for ONE head, in the order the pages give
 * it: statistics start at l = 0, m = -inf, O = 0 ([digest] section 2); the key
 * and value blocks of bc rows form the outer loop and the query blocks of br
 * rows the inner loop (T_c = ceil(nk/bc), T_r = ceil(nq/br)).  For each pair of
 * blocks the block's own row max and exp-sum are merged into the running ones
 * with the merge rule of [digest] section 2, and the output row is rescaled by
 * the same factors before the block's contribution is added ([gpko] item 58);
 * O is kept normalised after every block.  Outputs o [nq,d], lse [nq], and the
 * final statistics m [nq], l [nq] (each may be NULL except o). */
int oracle_attn_fwd_blockwise(const double *q, const double *k, const double *v, long nq, long nk, long d, int causal,
                              double scale, long br, long bc, double *o, double *lse, double *m_out, double *l_out)
{
    double *m, *l, *s, *pt, *pv;
    long jb, ib, i, j, c;
    if (!q || !k || !v || !o || nq < 0 || nk < 0 || d < 1 || br < 1 || bc < 1)
        return -1;
    m = (double *)malloc(sizeof(double) * (size_t)(nq + 1));
    l = (double *)malloc(sizeof(double) * (size_t)(nq + 1));
    s = (double *)malloc(sizeof(double) * (size_t)bc);
    pt = (double *)malloc(sizeof(double) * (size_t)bc);
    pv = (double *)malloc(sizeof(double) * (size_t)d);
    if (!m || !l || !s || !pt || !pv) {
        free(m);
        free(l);
        free(s);
        free(pt);
        free(pv);
        return -1;
    }
    for (i = 0; i < nq; ++i) { /* initialisation */
        m[i] = -INFINITY;
        l[i] = 0.0;
        for (c = 0; c < d; ++c)
            o[i * d + c] = 0.0;
    }
    for (jb = 0; jb < nk; jb += bc) { /* outer loop: key/value blocks */
        long jn = (jb + bc < nk) ? bc : nk - jb;
        for (ib = 0; ib < nq; ib += br) { /* inner loop: query blocks */
            long in = (ib + br < nq) ? br : nq - ib;
            for (i = ib; i < ib + in; ++i) {
                double mt = -INFINITY, lt = 0.0, mnew, lnew, a_old, a_blk;
                for (j = 0; j < jn; ++j) { /* the block's scores */
                    if (visible(i, jb + j, nq, nk, causal)) {
                        double acc = 0.0;
                        for (c = 0; c < d; ++c)
                            acc += q[i * d + c] * k[(jb + j) * d + c];
                        s[j] = scale * acc;
                    } else {
                        s[j] = -INFINITY;
                    }
                    if (s[j] > mt)
                        mt = s[j];
                }
                if (mt == -INFINITY)
                    continue; /* every key of this block is masked for row i: nothing to merge */
                for (j = 0; j < jn; ++j) { /* block's unnormalised probabilities and exp-sum */
                    pt[j] = exp(s[j] - mt);
                    lt += pt[j];
                }
                for (c = 0; c < d; ++c) { /* block's unnormalised output P~ V */
                    double acc = 0.0;
                    for (j = 0; j < jn; ++j)
                        acc += pt[j] * v[(jb + j) * d + c];
                    pv[c] = acc;
                }
                mnew = m[i] > mt ? m[i] : mt; /* merge rule */
                a_old = (m[i] == -INFINITY) ? 0.0 : exp(m[i] - mnew);
                a_blk = exp(mt - mnew);
                lnew = a_old * l[i] + a_blk * lt;
                for (c = 0; c < d; ++c)
                    o[i * d + c] = (l[i] * a_old * o[i * d + c] + a_blk * pv[c]) / lnew;
                m[i] = mnew;
                l[i] = lnew;
            }
        }
    }
    for (i = 0; i < nq; ++i) {
        if (lse)
            lse[i] = (l[i] > 0.0) ? m[i] + log(l[i]) : -INFINITY;
        if (m_out)
            m_out[i] = m[i];
        if (l_out)
            l_out[i] = l[i];
    }
    free(m);
    free(l);
    free(s);
    free(pt);
    free(pv);
    return 0;
}

/* Backward pass for one head, by the chain rule of the forward definition.
 * With P the probability matrix and dO the output gradient:
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = <dO_i, v_j>
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * P and dP (overwritten in place by dS) are materialised as nq x nk matrices. */
static void *bwd_worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    long nq = jb->nq, nk = jb->nk, d = jb->d, h, i, j, c;
    size_t nn = (size_t)(nq > 0 ? nq : 1) * (size_t)(nk > 0 ? nk : 1);
    double *P = (double *)malloc(sizeof(double) * nn);
    double *dS = (double *)malloc(sizeof(double) * nn);
    double *s = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    double *orow = (double *)malloc(sizeof(double) * (size_t)d);
    if (!P || !dS || !s || !orow) {
        jb->status = -1;
        free(P);
        free(dS);
        free(s);
        free(orow);
        return NULL;
    }
    for (h = jb->tid; h < jb->nheads; h += jb->nthreads) {
        const double *Q = jb->q + h * nq * d, *K = jb->k + h * nk * d, *V = jb->v + h * nk * d;
        const double *dO = jb->dout + h * nq * d;
        double *dQ = jb->dq + h * nq * d, *dK = jb->dk + h * nk * d, *dV = jb->dv + h * nk * d;
        for (i = 0; i < nq; ++i) /* P, row by row, by the forward definition */
            attend_row(Q + i * d, i, K, V, nq, nk, d, jb->causal, jb->scale, s, P + (size_t)i * nk, orow);
        for (i = 0; i < nq; ++i) { /* dP, then D, then dS in place */
            double Di = 0.0;
            double *row = dS + (size_t)i * nk;
            for (j = 0; j < nk; ++j) {
                double acc = 0.0;
                for (c = 0; c < d; ++c)
                    acc += dO[i * d + c] * V[j * d + c];
                row[j] = acc;
            }
            for (j = 0; j < nk; ++j)
                Di += P[(size_t)i * nk + j] * row[j];
            for (j = 0; j < nk; ++j)
                row[j] = P[(size_t)i * nk + j] * (row[j] - Di);
            if (jb->dvec)
                jb->dvec[h * nq + i] = Di;
        }
        for (j = 0; j < nk * d; ++j) {
            dK[j] = 0.0;
            dV[j] = 0.0;
        }
        for (i = 0; i < nq; ++i) {
            for (c = 0; c < d; ++c) { /* dQ_i = scale * sum_j dS_ij k_j */
                double acc = 0.0;
                for (j = 0; j < nk; ++j)
                    acc += dS[(size_t)i * nk + j] * K[j * d + c];
                dQ[i * d + c] = jb->scale * acc;
            }
            for (j = 0; j < nk; ++j) { /* dV_j += P_ij dO_i ; dK_j += dS_ij q_i */
                double pij = P[(size_t)i * nk + j], dsij = dS[(size_t)i * nk + j];
                for (c = 0; c < d; ++c) {
                    dV[j * d + c] += pij * dO[i * d + c];
                    dK[j * d + c] += dsij * Q[i * d + c];
                }
            }
        }
        for (j = 0; j < nk * d; ++j)
            dK[j] *= jb->scale;
    }
    free(P);
    free(dS);
    free(s);
    free(orow);
    return NULL;
}

/* Backward pass for all B*H heads.  dq [B,H,nq,d], dk and dv [B,H,nk,d],
 * dvec [B,H,nq] (the row sums D, may be NULL). */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout, double *dq, double *dk,
                    double *dv, double *dvec, long B, long H, long nq, long nk, long d, int causal, double scale,
                    int nthreads)
{
    job_t jb;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 0 || H < 0 || nq < 0 || nk < 0 || d < 1)
        return -1;
    memset(&jb, 0, sizeof jb);
    jb.q = q;
    jb.k = k;
    jb.v = v;
    jb.dout = dout;
    jb.dq = dq;
    jb.dk = dk;
    jb.dv = dv;
    jb.dvec = dvec;
    jb.nheads = B * H;
    jb.nq = nq;
    jb.nk = nk;
    jb.d = d;
    jb.causal = causal;
    jb.scale = scale;
    if (jb.nheads == 0)
        return 0;
    return run_threads(&jb, nthreads, bwd_worker);
}

/* ---------------------------------------------------------------------------
 * 8-bit floating-point inputs.
 *
 * FlashAttention v3 takes FP8 inputs ("FlashAttention v3 (Tri Dao et al.)",
 * section "What it is"); products of FP8 operands with fp32 results take the
 * e4m3 or e5m2 element type ("CUTLASS WGMMA Atom Skeleton", table "Atom
 * Family Names Seen In CUTLASS").  The codes here are e4m3 in the OCP 8-bit
 * floating-point definition (the form this GPU's matrix cores take): one sign
 * bit s, four exponent bits e with bias 7, three fraction bits f;
 *   e = 0:          (-1)^s * 2^-6 * f/8        (zero and subnormals)
 *   e = 1 .. 15:    (-1)^s * 2^(e-7) * (1 + f/8)
 * except e = 15, f = 7, which is NaN; there is no infinity (largest 448).
 * Each tensor of codes carries a per-head scale, and the real value is scale *
 * decoded code: the affine map r = S (q - Z) of "Quantization and Training of
 * Neural Networks for Efficient Integer-Arithmetic-Only Inference" ([gpko]
 * item 33) with zero point Z = 0.
 * ------------------------------------------------------------------------- */

/* Decode n e4m3 codes into doubles (exact). */
int oracle_fp8_e4m3_decode(const unsigned char *x, long n, double *out)
{
    long i;
    if ((!x || !out) && n > 0)
        return -1;
    for (i = 0; i < n; ++i) {
        const int s = x[i] >> 7, e = (x[i] >> 3) & 15, f = x[i] & 7;
        double mag;
        if (e == 15 && f == 7)
            mag = NAN;
        else if (e == 0)
            mag = ldexp((double)f / 8.0, -6);
        else
            mag = ldexp(1.0 + (double)f / 8.0, e - 7);
        out[i] = s ? -mag : mag;
    }
    return 0;
}
