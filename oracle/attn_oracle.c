/*
 * attn_oracle.c -- fp64 CPU oracle for the exact attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (the plain definition, no tiling, no online softmax):
 * for every batch b, head h and query row i,
 *
 *   valid(i,j) = not causal  or  j <= i                       (top-left causal mask)
 *   s[j]       = scale * sum_c q[b,h,i,c] * k[b,h,j,c]       if valid, else -inf
 *   m          = max_j s[j]
 *   p[j]       = exp(s[j] - m)                               (0 where s[j] = -inf)
 *   l          = sum_j p[j]
 *   O[b,h,i,c] = (sum_j p[j] * v[b,h,j,c]) / l
 *   L[b,h,i]   = m + ln(l)
 *
 * Sources on the pages:
 *  - page "flash_attention_2.cu" (leloykun/flash-hyperbolic-attention-minimal),
 *    forward kernel: the score is the dot product over the head dimension
 *    times the softmax scale; the causal guard drops key j for query i when
 *    i < j, so the diagonal is kept; the row max, exp(S - m) and row sum;
 *    the final division of O by l and L = m + log(l) (natural log).
 *  - page "Add Fused Multi-Head Attention example" (cuTile.jl PR #16), the
 *    masking snippet: keys past the key sequence length get an additive -Inf.
 *    Here the key range is exactly [0, Nk), so there is no padding to mask.
 *
 * Layout: q is [B,H,Nq,d], k and v are [B,H,Nk,d], all row-major fp64.
 * Every score row is materialised in full (Nk doubles per row). Rows are
 * independent, so they are spread over POSIX threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
    const double* q;
    const double* k;
    const double* v;
    int64_t B, H, Nq, Nk, d;
    double scale;
    int causal;
    const int64_t* rows; /* flat row ids ((b*H + h)*Nq + i), or NULL = all rows */
    int64_t nrows;
    double* o;   /* [nrows, d] */
    double* lse; /* [nrows]    */
    int nthreads;
    int tid;
    int status;
} job_t;

/* One query row: the definition above, written out. */
static void one_row(const job_t* J, int64_t row, double* s, double* o_row, double* lse_out)
{
    const int64_t d = J->d, Nk = J->Nk, Nq = J->Nq;
    const int64_t bh = row / Nq; /* b*H + h */
    const int64_t i = row % Nq;
    const double* qi = J->q + row * d;
    const double* kh = J->k + bh * Nk * d;
    const double* vh = J->v + bh * Nk * d;

    /* scores, with the mask */
    for (int64_t j = 0; j < Nk; ++j) {
        int valid = !J->causal || j <= i;
        if (!valid) {
            s[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qi[c] * kh[j * d + c];
        s[j] = J->scale * dot;
    }

    /* row max */
    double m = -INFINITY;
    for (int64_t j = 0; j < Nk; ++j)
        if (s[j] > m)
            m = s[j];

    /* exp and row sum; the weights overwrite the scores */
    double l = 0.0;
    for (int64_t j = 0; j < Nk; ++j) {
        double p = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        s[j] = p;
        l += p;
    }

    /* weighted sum of V rows, divided by the row sum */
    for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < Nk; ++j)
            acc += s[j] * vh[j * d + c];
        o_row[c] = acc / l;
    }
    *lse_out = m + log(l);
}

static void* worker(void* arg)
{
    job_t* J = (job_t*)arg;
    double* s = (double*)malloc((size_t)J->Nk * sizeof(double));
    if (!s) {
        J->status = 2;
        return NULL;
    }
    for (int64_t r = J->tid; r < J->nrows; r += J->nthreads) {
        int64_t row = J->rows ? J->rows[r] : r;
        one_row(J, row, s, J->o + r * J->d, J->lse + r);
    }
    free(s);
    J->status = 0;
    return NULL;
}

/*
 * Computes O and L for the requested rows.
 *   rows == NULL: every row, nrows must equal B*H*Nq; o is [B,H,Nq,d], lse [B,H,Nq].
 *   rows != NULL: rows[r] is a flat row id (b*H + h)*Nq + i; o is [nrows,d], lse [nrows].
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
int attn_oracle_fwd(const double* q, const double* k, const double* v,
                    int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                    double scale, int causal,
                    const int64_t* rows, int64_t nrows,
                    double* o, double* lse, int nthreads)
{
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1)
        return 1;
    if (!rows && nrows != B * H * Nq)
        return 1;
    if (rows) {
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= B * H * Nq)
                return 1;
    }
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;

    job_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) {
        job_t J = {q, k, v, B, H, Nq, Nk, d, scale, causal, rows, nrows, o, lse,
                   nthreads, t, 1};
        jobs[t] = J;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    /* threads that failed to start leave their rows to a serial sweep below */
    worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    int status = jobs[0].status;
    for (int t = started + 1; t < nthreads; ++t) {
        worker(&jobs[t]);
        if (jobs[t].status)
            status = jobs[t].status;
    }
    for (int t = 1; t <= started; ++t)
        if (jobs[t].status)
            status = jobs[t].status;
    return status;
}
