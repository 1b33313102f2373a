/*
 * eda_ref.c -- plain fp64 CPU oracle for the Erase-then-Delta Attention (EDA)
 * recurrence forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the numerical reference that the
 * GPU kernels are checked against.  It is compiled and called only by the
 * test suite, the package's smoke check and the benchmark's CPU-baseline
 * leg.  It shares no code, header or constant with the GPU library.
 *
 * What it computes (EDA paper, Sec. 3.3, Eqs. (8)-(13); reading slides,
 * frame "EDA preserves the delta write after cleanup"): for every head
 * (b, h) independently, with state S (d_k x d_v, rows = key channels) and
 * for t = 0 .. T-1, the three ordered stages
 *
 *   decay   (Eq. 9):  Sh[i][j] = alpha_t[i] * S[i][j]
 *   erase   (Eq. 11): re[j] = sum_i Sh[i][j] e_t[i]
 *                     St[i][j] = Sh[i][j] - gamma_t e_t[i] re[j]
 *   write   (Eq. 13): rk[j] = sum_i St[i][j] k_t[i]
 *                     S[i][j] = St[i][j] + beta_t k_t[i] (v_t[j] - rk[j])
 *
 * followed by the read o_t = S_t^T q_t from the post-update state (the
 * paper's notation section: memory is read through S_t^T q_t).  No query
 * scale is applied; q, k, e are used exactly as given.  All arithmetic is
 * IEEE fp64, sums over i run in ascending order.
 *
 * Value columns j never interact (every stage is column-wise), so a head's
 * columns may be split into blocks that run on different threads; the
 * result is bit-identical to the unsplit loop.
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *e, *v, *alpha, *beta, *gamma, *S0;
    double *o, *S_final;
    long B, T, H, dk, dv;
    long ncb;      /* value-column blocks per head */
    long ntasks;   /* B * H * ncb */
    int nthreads;
    int tid;
    int status;
} eda_ref_job;

/* One (b, h, column block [j0, j1)) task. */
static int run_task(const eda_ref_job *J, long task)
{
    const long dk = J->dk, dv = J->dv, H = J->H, T = J->T;
    const long unit = task / J->ncb, cb = task % J->ncb;
    const long b = unit / H, h = unit % H;
    const long bw = (dv + J->ncb - 1) / J->ncb;
    const long j0 = cb * bw, j1 = (j0 + bw < dv) ? j0 + bw : dv;
    const long w = j1 - j0;
    if (w <= 0) return 0;

    double *S = (double *)malloc(sizeof(double) * dk * w);
    double *re = (double *)malloc(sizeof(double) * w);
    double *rk = (double *)malloc(sizeof(double) * w);
    if (!S || !re || !rk) { free(S); free(re); free(rk); return 1; }

    /* S <- S0 (zeros when absent). */
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < w; ++j)
            S[i * w + j] = J->S0 ? J->S0[((b * H + h) * dk + i) * dv + j0 + j] : 0.0;

    for (long t = 0; t < T; ++t) {
        const long row = (b * T + t) * H + h;      /* [B, T, H] index */
        const double *q = J->q + row * dk, *k = J->k + row * dk, *e = J->e + row * dk;
        const double *a = J->alpha + row * dk, *v = J->v + row * dv;
        const double beta = J->beta[row], gamma = J->gamma[row];

        /* decay */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                S[i * w + j] = a[i] * S[i * w + j];

        /* erase: re = Sh^T e ; St = Sh - gamma e re^T */
        for (long j = 0; j < w; ++j) re[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                re[j] += S[i * w + j] * e[i];
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                S[i * w + j] = S[i * w + j] - gamma * e[i] * re[j];

        /* corrected write: rk = St^T k ; S = St + beta k (v - rk)^T */
        for (long j = 0; j < w; ++j) rk[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                rk[j] += S[i * w + j] * k[i];
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                S[i * w + j] = S[i * w + j] + beta * k[i] * (v[j0 + j] - rk[j]);

        /* read: o_t = S_t^T q_t (re is reused as the accumulator) */
        for (long j = 0; j < w; ++j) re[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                re[j] += S[i * w + j] * q[i];
        for (long j = 0; j < w; ++j)
            J->o[row * dv + j0 + j] = re[j];
    }

    if (J->S_final)
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                J->S_final[((b * H + h) * dk + i) * dv + j0 + j] = S[i * w + j];

    free(S); free(re); free(rk);
    return 0;
}

static void *worker(void *p)
{
    eda_ref_job *J = (eda_ref_job *)p;
    for (long task = J->tid; task < J->ntasks; task += J->nthreads)
        if (run_task(J, task)) J->status = 1;
    return NULL;
}

/*
 * eda_ref_fwd -- run the recurrence for all B*H heads.
 *   q, k, e, alpha : [B, T, H, dk]    v, o : [B, T, H, dv]
 *   beta, gamma    : [B, T, H]        S0, S_final : [B, H, dk, dv]
 * S0 may be NULL (zeros); S_final may be NULL (not written).  All arrays are
 * contiguous fp64.  nthreads >= 1.  Returns 0 on success, 1 on bad
 * arguments or allocation failure.
 */
int eda_ref_fwd(const double *q, const double *k, const double *e, const double *v,
                const double *alpha, const double *beta, const double *gamma,
                const double *S0, double *o, double *S_final,
                long B, long T, long H, long dk, long dv, int nthreads)
{
    if (!q || !k || !e || !v || !alpha || !beta || !gamma || !o) return 1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || nthreads < 1) return 1;

    eda_ref_job base;
    memset(&base, 0, sizeof(base));
    base.q = q; base.k = k; base.e = e; base.v = v; base.alpha = alpha;
    base.beta = beta; base.gamma = gamma; base.S0 = S0; base.o = o; base.S_final = S_final;
    base.B = B; base.T = T; base.H = H; base.dk = dk; base.dv = dv;

    const long units = B * H;
    if (units == 0) return 0;
    long ncb = (nthreads + units - 1) / units;   /* split columns only when units < threads */
    if (ncb > dv) ncb = dv;
    base.ncb = ncb;
    base.ntasks = units * ncb;
    if (nthreads > base.ntasks) nthreads = (int)base.ntasks;
    base.nthreads = nthreads;

    eda_ref_job *jobs = (eda_ref_job *)malloc(sizeof(eda_ref_job) * nthreads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    char *started = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !th || !started) { free(jobs); free(th); free(started); return 1; }
    int status = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = base;
        jobs[i].tid = i;
        if (i > 0) {
            if (pthread_create(&th[i], NULL, worker, &jobs[i]) == 0)
                started[i] = 1;
            else
                worker(&jobs[i]);   /* no thread available: run it here */
        }
    }
    worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i) status |= jobs[i].status;
    free(jobs); free(th); free(started);
    return status;
}
