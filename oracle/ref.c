/*
 * oracle/ref.c -- CPU reference for the exact attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the GPU library, and it never calls it.
 *
 * What it computes is the plain definition of attention for one head,
 * "[Attention优化] 从Online-Softmax到FlashAttention V1/V2/V3", section 0x01
 * (standard self-attention: S = Q K^T, P = softmax(S), O = P V), evaluated
 * with the 3-pass safe softmax of section 0x02 of the same page (pass 1: row
 * maximum; pass 2: sum of exp(x - max); pass 3: normalise), in double
 * precision.  The scale that the page leaves out of the formula is applied to
 * the scores before the mask, and masked keys are excluded from the row.
 * Multi-query / grouped-query attention follows section 0x09 of that page:
 * query head h reads key/value head h / (Hq / Hkv).
 *
 * The per-row log-sum-exp that the forward stores for the backward pass
 * ("FlashAttention：IO 感知的精确注意力", section 6: the forward keeps only the
 * row maximum m and the normaliser l) is returned as lse = m + ln(l), the
 * natural logarithm of the sum of exp over the visible scaled scores.
 *
 * Layout (all contiguous, C order): q [B][Nq][Hq][d], k and v
 * [B][Nk][Hkv][d], given as float (bf16 inputs are widened to float exactly
 * by the caller).  Arithmetic is entirely in double.
 *
 * Causal mask, aligned to the bottom-right corner of the score matrix (first
 * page, section 0x09): key j is visible to query i iff j <= i + (Nk - Nq).
 * With Nq == Nk this is j <= i.  A query that sees no key (possible when
 * Nq > Nk) gets an all-zero output row, as that section states, and
 * lse = -inf (the log of an empty sum).
 *
 * Block-sparse attention (first page, section 0x04: blocks that a sparsity
 * pattern marks are skipped entirely): with a block mask, key j is kept for
 * query i of head h only if mask[h][i / bq][j / bk] is nonzero, in addition
 * to the causal rule; the softmax runs over the kept keys alone.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v;
    int B, Hq, Hkv, Nq, Nk, d;
    double scale;
    int causal;
    const uint8_t *mask; /* optional block mask [Hq][ceil(Nq/bq)][ceil(Nk/bk)] */
    int bq, bk;
    const int32_t *rows; /* triples (b, h, i) */
    int64_t nrows;
    double *o;   /* [nrows][d] */
    double *lse; /* [nrows] */
    int64_t next;
    pthread_mutex_t lock;
} job_t;

/* Whether the block mask (if any) keeps key j for query i of head h. */
static int kept(const job_t *J, int h, int i, int j)
{
    if (!J->mask) return 1;
    const int64_t nqb = (J->Nq + J->bq - 1) / J->bq, nkb = (J->Nk + J->bk - 1) / J->bk;
    return J->mask[((int64_t)h * nqb + i / J->bq) * nkb + j / J->bk] != 0;
}

/* One query row, the three passes of the safe softmax, then P V. */
static void one_row(const job_t *J, int b, int h, int i, double *s,
                    double *o_out, double *lse_out)
{
    const int d = J->d;
    const int g = J->Hq / J->Hkv;
    const int hk = h / g;
    const float *qi = J->q + (((int64_t)b * J->Nq + i) * J->Hq + h) * d;
    int nvis = J->Nk;                       /* visible keys are 0 .. nvis-1 */
    if (J->causal) {
        const int64_t last = (int64_t)i + (J->Nk - J->Nq);
        nvis = last < 0 ? 0 : (last + 1 < J->Nk ? (int)(last + 1) : J->Nk);
    }
    int nkept = 0;
    for (int j = 0; j < nvis; ++j) nkept += kept(J, h, i, j);
    if (nkept == 0) {                       /* empty row: zero output */
        for (int x = 0; x < d; ++x) o_out[x] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* scores s_j = scale * <q_i, k_j> for the visible keys */
    for (int j = 0; j < nvis; ++j) {
        if (!kept(J, h, i, j)) continue;
        const float *kj = J->k + (((int64_t)b * J->Nk + j) * J->Hkv + hk) * d;
        double acc = 0.0;
        for (int x = 0; x < d; ++x)
            acc += (double)qi[x] * (double)kj[x];
        s[j] = J->scale * acc;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int j = 0; j < nvis; ++j)
        if (kept(J, h, i, j) && s[j] > m) m = s[j];
    /* pass 2: normaliser */
    double l = 0.0;
    for (int j = 0; j < nvis; ++j)
        if (kept(J, h, i, j)) l += exp(s[j] - m);
    /* pass 3: normalised weights a_j, then o = sum_j a_j v_j */
    for (int x = 0; x < d; ++x) o_out[x] = 0.0;
    for (int j = 0; j < nvis; ++j) {
        if (!kept(J, h, i, j)) continue;
        const double a = exp(s[j] - m) / l;
        const float *vj = J->v + (((int64_t)b * J->Nk + j) * J->Hkv + hk) * d;
        for (int x = 0; x < d; ++x)
            o_out[x] += a * (double)vj[x];
    }
    *lse_out = m + log(l);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)J->Nk);
    if (!s) return (void *)1;
    for (;;) {
        int64_t r;
        pthread_mutex_lock(&J->lock);
        r = J->next;
        J->next += 16;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->nrows) break;
        int64_t end = r + 16 < J->nrows ? r + 16 : J->nrows;
        for (; r < end; ++r) {
            const int32_t *t = J->rows + 3 * r;
            one_row(J, t[0], t[1], t[2], s, J->o + r * J->d, J->lse + r);
        }
    }
    free(s);
    return NULL;
}

/*
 * oracle_attention_masked: O and LSE for the listed query rows.
 *   q: [B][Nq][Hq][d]; k, v: [B][Nk][Hkv][d].
 *   mask: NULL, or a block mask [Hq][ceil(Nq/bq)][ceil(Nk/bk)] (bytes, nonzero
 *         = the block of bq query rows x bk keys is kept).
 *   rows: nrows triples (b, h, i), i < Nq; o: nrows*d doubles; lse: nrows doubles.
 *   scale: applied to q.k (the caller passes the same float the GPU gets).
 *   nthreads: worker threads (>= 1).
 * Returns 0 on success, -1 on a bad argument, -2 on allocation failure.
 */
int oracle_attention_masked(const float *q, const float *k, const float *v,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, double scale,
                            int causal, const uint8_t *mask, int bq, int bk,
                            const int32_t *rows, int64_t nrows,
                            double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !rows || !o || !lse) return -1;
    if (mask && (bq < 1 || bk < 1)) return -1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1 || Hq % Hkv) return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int32_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= Hq || t[2] < 0 || t[2] >= Nq)
            return -1;
    }
    if (nthreads < 1) nthreads = 1;
    job_t J;
    J.q = q; J.k = k; J.v = v;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.d = d;
    J.scale = scale; J.causal = causal;
    J.mask = mask; J.bq = bq; J.bk = bk;
    J.rows = rows; J.nrows = nrows; J.o = o; J.lse = lse;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) rc = (worker(&J) == NULL) ? 0 : -2;
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret != NULL) rc = -2;
    }
    free(th);
    pthread_mutex_destroy(&J.lock);
    return rc;
}

/* oracle_attention: oracle_attention_masked without a block mask. */
int oracle_attention(const float *q, const float *k, const float *v,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, double scale,
                     int causal, const int32_t *rows, int64_t nrows,
                     double *o, double *lse, int nthreads)
{
    return oracle_attention_masked(q, k, v, B, Hq, Hkv, Nq, Nk, d, scale, causal, NULL, 1, 1,
                                   rows, nrows, o, lse, nthreads);
}

/* ------------------------------------------------------------------------
 * Backward: gradients of the forward above with respect to q, k and v, for
 * an upstream gradient dout = dL/dO.
 *
 * This is the derivative of the definition, written out row by row in
 * double precision.  For query row i of head h (key/value head hk):
 *   P_ij  = softmax_j(s_i.) over the visible keys (0 elsewhere)
 *   dP_ij = <dout_i, v_j>
 *   dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)        (softmax Jacobian)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j += scale * dS_ij q_i,  dv_j += P_ij dout_i  (summed over the rows
 *                                                     and over the query
 *                                                     heads of the group)
 * The pages describe how FlashAttention organises this computation (the
 * first page, sections 0x04 and 0x05: S and P recomputed from the stored
 * row statistics, an outer loop over K/V blocks, dQ accumulated across
 * blocks; the second page, section 6); the gradients themselves are those
 * of the forward's definition.  A row without visible keys contributes
 * nothing.
 *
 * Work is done per key/value head group (b, hk): dq for the Hq/Hkv query
 * heads of the group and dk, dv of the shared head.  Threads split the query
 * rows of a group and keep private dk, dv sums that are added in thread
 * order at the end (the result does not depend on scheduling).
 * ------------------------------------------------------------------------ */
typedef struct {
    const float *q, *k, *v, *dout;
    int B, Hq, Hkv, Nq, Nk, d;
    double scale;
    int causal;
    int b, hk;              /* the group being processed */
    int nthreads;
    double *dq;             /* [g][Nq][d] */
    double *dk_part;        /* [nthreads][Nk][d] */
    double *dv_part;
    int fail;
} bwd_job_t;

typedef struct {
    bwd_job_t *J;
    int t;
} bwd_arg_t;

static void *bwd_worker(void *arg)
{
    bwd_arg_t *A = (bwd_arg_t *)arg;
    bwd_job_t *J = A->J;
    const int d = J->d, Nq = J->Nq, Nk = J->Nk;
    const int g = J->Hq / J->Hkv;
    double *p = (double *)malloc(sizeof(double) * (size_t)Nk);
    double *dp = (double *)malloc(sizeof(double) * (size_t)Nk);
    if (!p || !dp) {
        free(p);
        free(dp);
        J->fail = 1;
        return NULL;
    }
    double *dk = J->dk_part + (size_t)A->t * Nk * d;
    double *dv = J->dv_part + (size_t)A->t * Nk * d;
    const int64_t total = (int64_t)g * Nq;
    for (int64_t r = A->t; r < total; r += J->nthreads) {
        const int hh = (int)(r / Nq), i = (int)(r % Nq);
        const int h = J->hk * g + hh;
        const float *qi = J->q + (((int64_t)J->b * Nq + i) * J->Hq + h) * d;
        const float *doi = J->dout + (((int64_t)J->b * Nq + i) * J->Hq + h) * d;
        double *dqi = J->dq + ((int64_t)hh * Nq + i) * d;
        for (int x = 0; x < d; ++x) dqi[x] = 0.0;
        int nvis = Nk;
        if (J->causal) {
            const int64_t last = (int64_t)i + (Nk - Nq);
            nvis = last < 0 ? 0 : (last + 1 < Nk ? (int)(last + 1) : Nk);
        }
        if (nvis == 0) continue;
        /* P_i. by the three-pass softmax, and dP_i. */
        double m = -INFINITY;
        for (int j = 0; j < nvis; ++j) {
            const float *kj = J->k + (((int64_t)J->b * Nk + j) * J->Hkv + J->hk) * d;
            const float *vj = J->v + (((int64_t)J->b * Nk + j) * J->Hkv + J->hk) * d;
            double s = 0.0, t = 0.0;
            for (int x = 0; x < d; ++x) {
                s += (double)qi[x] * (double)kj[x];
                t += (double)doi[x] * (double)vj[x];
            }
            p[j] = J->scale * s;
            dp[j] = t;
            if (p[j] > m) m = p[j];
        }
        double l = 0.0;
        for (int j = 0; j < nvis; ++j) {
            p[j] = exp(p[j] - m);
            l += p[j];
        }
        double pdp = 0.0;
        for (int j = 0; j < nvis; ++j) {
            p[j] /= l;
            pdp += p[j] * dp[j];
        }
        for (int j = 0; j < nvis; ++j) {
            const double ds = p[j] * (dp[j] - pdp);
            const float *kj = J->k + (((int64_t)J->b * Nk + j) * J->Hkv + J->hk) * d;
            double *dkj = dk + (int64_t)j * d, *dvj = dv + (int64_t)j * d;
            for (int x = 0; x < d; ++x) {
                dqi[x] += J->scale * ds * (double)kj[x];
                dkj[x] += J->scale * ds * (double)qi[x];
                dvj[x] += p[j] * (double)doi[x];
            }
        }
    }
    free(p);
    free(dp);
    return NULL;
}

/*
 * oracle_attention_bwd: dq, dk, dv for the listed key/value head groups.
 *   q, dout: [B][Nq][Hq][d]; k, v: [B][Nk][Hkv][d] (float).
 *   groups: ngroups pairs (b, hk).
 *   dq: ngroups * (Hq/Hkv) * Nq * d doubles, [group][query head in group][i][x];
 *   dk, dv: ngroups * Nk * d doubles, [group][j][x].
 * Returns 0 on success, -1 on a bad argument, -2 on allocation failure.
 */
int oracle_attention_bwd(const float *q, const float *k, const float *v, const float *dout,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, double scale,
                         int causal, const int32_t *groups, int64_t ngroups,
                         double *dq, double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !dout || !groups || !dq || !dk || !dv) return -1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1 || Hq % Hkv) return -1;
    for (int64_t r = 0; r < ngroups; ++r)
        if (groups[2 * r] < 0 || groups[2 * r] >= B || groups[2 * r + 1] < 0 || groups[2 * r + 1] >= Hkv)
            return -1;
    if (nthreads < 1) nthreads = 1;
    const int g = Hq / Hkv;
    bwd_job_t J;
    J.q = q; J.k = k; J.v = v; J.dout = dout;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.d = d;
    J.scale = scale; J.causal = causal; J.nthreads = nthreads;
    J.dk_part = (double *)malloc(sizeof(double) * (size_t)nthreads * Nk * d);
    J.dv_part = (double *)malloc(sizeof(double) * (size_t)nthreads * Nk * d);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    bwd_arg_t *args = (bwd_arg_t *)malloc(sizeof(bwd_arg_t) * (size_t)nthreads);
    int rc = 0;
    if (!J.dk_part || !J.dv_part || !th || !args) rc = -2;
    for (int64_t r = 0; r < ngroups && rc == 0; ++r) {
        J.b = groups[2 * r];
        J.hk = groups[2 * r + 1];
        J.dq = dq + (size_t)r * g * Nq * d;
        J.fail = 0;
        memset(J.dk_part, 0, sizeof(double) * (size_t)nthreads * Nk * d);
        memset(J.dv_part, 0, sizeof(double) * (size_t)nthreads * Nk * d);
        int started = 0;
        for (int t = 0; t < nthreads; ++t) {
            args[t].J = &J;
            args[t].t = t;
        }
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&th[t], NULL, bwd_worker, &args[t]) != 0) break;
            ++started;
        }
        if (started < nthreads) {
            /* run the missing workers' rows here, in order */
            for (int t = started; t < nthreads; ++t) bwd_worker(&args[t]);
        }
        for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
        if (J.fail) {
            rc = -2;
            break;
        }
        double *dkg = dk + (size_t)r * Nk * d, *dvg = dv + (size_t)r * Nk * d;
        for (int64_t e = 0; e < (int64_t)Nk * d; ++e) {
            double sk = 0.0, sv = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                sk += J.dk_part[(size_t)t * Nk * d + e];
                sv += J.dv_part[(size_t)t * Nk * d + e];
            }
            dkg[e] = sk;
            dvg[e] = sv;
        }
    }
    free(J.dk_part);
    free(J.dv_part);
    free(th);
    free(args);
    return rc;
}
