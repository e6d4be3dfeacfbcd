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
    const int32_t *rows; /* triples (b, h, i) */
    int64_t nrows;
    double *o;   /* [nrows][d] */
    double *lse; /* [nrows] */
    int64_t next;
    pthread_mutex_t lock;
} job_t;

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
    if (nvis == 0) {                        /* empty row: zero output */
        for (int x = 0; x < d; ++x) o_out[x] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* scores s_j = scale * <q_i, k_j> for the visible keys */
    for (int j = 0; j < nvis; ++j) {
        const float *kj = J->k + (((int64_t)b * J->Nk + j) * J->Hkv + hk) * d;
        double acc = 0.0;
        for (int x = 0; x < d; ++x)
            acc += (double)qi[x] * (double)kj[x];
        s[j] = J->scale * acc;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int j = 0; j < nvis; ++j)
        if (s[j] > m) m = s[j];
    /* pass 2: normaliser */
    double l = 0.0;
    for (int j = 0; j < nvis; ++j)
        l += exp(s[j] - m);
    /* pass 3: normalised weights a_j, then o = sum_j a_j v_j */
    for (int x = 0; x < d; ++x) o_out[x] = 0.0;
    for (int j = 0; j < nvis; ++j) {
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
 * oracle_attention: O and LSE for the listed query rows.
 *   q: [B][Nq][Hq][d]; k, v: [B][Nk][Hkv][d].
 *   rows: nrows triples (b, h, i), i < Nq; o: nrows*d doubles; lse: nrows doubles.
 *   scale: applied to q.k (the caller passes the same float the GPU gets).
 *   nthreads: worker threads (>= 1).
 * Returns 0 on success, -1 on a bad argument, -2 on allocation failure.
 */
int oracle_attention(const float *q, const float *k, const float *v,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, double scale,
                     int causal, const int32_t *rows, int64_t nrows,
                     double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !rows || !o || !lse) return -1;
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
