/*
 * Test infrastructure only: the fp64 CPU oracle of the Kimi Delta Attention
 * (KDA) forward pass.  Only tests/, the smoke check and the benchmark's CPU
 * baseline leg load this file; the library never does.  It shares no code,
 * header or constant with the GPU path.
 *
 * What it computes (the plain token-by-token recurrence, nothing chunked):
 *
 *   Kimi-K3 深度解析 (d7kj.com blog), section 三 "KDA 的关键改进":
 *     the state is first decayed per channel by alpha_t, then corrected by an
 *     error term e_t = beta_t (v_t - vhat_t) written along k_t, where vhat_t
 *     is the value the (decayed) state currently predicts for k_t.
 *   深入 Kimi-K3 (xitter thread), the KDA paragraph: q and k are
 *     L2-normalised inside the kernel; the decay is per channel with a lower
 *     bound of -5 on its logarithm.
 *
 * Orientation.  The blog writes the state as d_v x d_k and decays its
 * columns; here the state is stored as its transpose, S[i][j] with i the key
 * channel (d_k rows) and j the value channel (d_v columns), so the decay
 * scales key rows.  Both describe the same map.
 *
 * Per sequence (one batch entry and head), with S = h0 (or 0):
 *   for t = 0 .. T-1
 *     qh = q_t / sqrt(|q_t|^2 + eps),  kh = k_t / sqrt(|k_t|^2 + eps)
 *     S[i][:] *= exp(g_t[i])                 decay on key rows
 *     p[j]     = sum_i kh[i] S[i][j]         prediction from the decayed state
 *     u[j]     = beta_t (v_t[j] - p[j])      beta is one scalar per token
 *     S[i][j] += kh[i] u[j]                  delta-rule write
 *     o_t[j]   = scale sum_i qh[i] S[i][j]   read-out includes token t
 *   hT = S
 *
 * All arithmetic is double precision.  Sequences are independent and are
 * spread over POSIX threads; the work inside one sequence is sequential.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int n_seq, T, dk, dv;
    const double *q, *k, *v, *g, *beta, *h0;
    double scale, eps;
    double *o, *hT;
    int first, stride; /* this worker handles sequences first, first+stride, ... */
    int status;
} job_t;

static void run_sequence(const job_t *jb, int s, double *S, double *qh, double *kh,
                         double *p, double *u) {
    const int T = jb->T, dk = jb->dk, dv = jb->dv;
    const double *q = jb->q + (size_t)s * T * dk;
    const double *k = jb->k + (size_t)s * T * dk;
    const double *v = jb->v + (size_t)s * T * dv;
    const double *g = jb->g + (size_t)s * T * dk;
    const double *beta = jb->beta + (size_t)s * T;
    double *o = jb->o + (size_t)s * T * dv;

    if (jb->h0)
        memcpy(S, jb->h0 + (size_t)s * dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk;
        const double *vt = v + (size_t)t * dv, *gt = g + (size_t)t * dk;
        double *ot = o + (size_t)t * dv;

        /* L2 normalisation of q and k */
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; ++i) {
            sq += qt[i] * qt[i];
            sk += kt[i] * kt[i];
        }
        const double nq = sqrt(sq + jb->eps), nk = sqrt(sk + jb->eps);
        for (int i = 0; i < dk; ++i) {
            qh[i] = nq > 0.0 ? qt[i] / nq : 0.0;
            kh[i] = nk > 0.0 ? kt[i] / nk : 0.0;
        }

        /* decay: every key row i is scaled by exp(g_t[i]) */
        for (int i = 0; i < dk; ++i) {
            const double a = exp(gt[i]);
            double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) row[j] *= a;
        }

        /* prediction p = S^T kh from the decayed state */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) p[j] += kh[i] * row[j];
        }

        /* error term u = beta (v - p) */
        for (int j = 0; j < dv; ++j) u[j] = beta[t] * (vt[j] - p[j]);

        /* delta-rule write S += kh u^T */
        for (int i = 0; i < dk; ++i) {
            double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) row[j] += kh[i] * u[j];
        }

        /* read-out o = scale S^T qh, after the write */
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) ot[j] += qh[i] * row[j];
        }
        for (int j = 0; j < dv; ++j) ot[j] *= jb->scale;
    }

    if (jb->hT) memcpy(jb->hT + (size_t)s * dk * dv, S, sizeof(double) * dk * dv);
}

static void *worker(void *arg) {
    job_t *jb = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)jb->dk * jb->dv);
    double *qh = (double *)malloc(sizeof(double) * (size_t)jb->dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)jb->dk);
    double *p = (double *)malloc(sizeof(double) * (size_t)jb->dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)jb->dv);
    if (!S || !qh || !kh || !p || !u) {
        jb->status = -2;
    } else {
        for (int s = jb->first; s < jb->n_seq; s += jb->stride)
            run_sequence(jb, s, S, qh, kh, p, u);
        jb->status = 0;
    }
    free(S); free(qh); free(kh); free(p); free(u);
    return NULL;
}

/*
 * Runs n_seq independent sequences.  Layouts (all contiguous, double):
 *   q, k, g : [n_seq][T][dk]     v, o : [n_seq][T][dv]     beta : [n_seq][T]
 *   h0, hT  : [n_seq][dk][dv]    (h0 may be NULL = zero state; hT may be NULL)
 * Returns 0 on success, -1 on a bad argument, -2 when memory or threads fail.
 */
int kda_oracle_run(int n_seq, int T, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta,
                   double scale, double eps, const double *h0,
                   double *o, double *hT, int n_threads) {
    if (n_seq < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (n_seq == 0) return 0;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > n_seq) n_threads = n_seq;

    job_t *jobs = (job_t *)calloc((size_t)n_threads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    char *live = (char *)calloc((size_t)n_threads, 1);
    if (!jobs || !tids || !live) { free(jobs); free(tids); free(live); return -2; }

    int rc = 0;
    for (int w = 0; w < n_threads; ++w) {
        job_t *jb = &jobs[w];
        jb->n_seq = n_seq; jb->T = T; jb->dk = dk; jb->dv = dv;
        jb->q = q; jb->k = k; jb->v = v; jb->g = g; jb->beta = beta; jb->h0 = h0;
        jb->scale = scale; jb->eps = eps; jb->o = o; jb->hT = hT;
        jb->first = w; jb->stride = n_threads; jb->status = -2;
        if (n_threads == 1) {
            worker(jb);
        } else if (pthread_create(&tids[w], NULL, worker, jb) == 0) {
            live[w] = 1;
        } else {
            /* run what could not get a thread on this one */
            worker(jb);
        }
    }
    if (n_threads > 1)
        for (int w = 0; w < n_threads; ++w)
            if (live[w]) pthread_join(tids[w], NULL);
    for (int w = 0; w < n_threads; ++w)
        if (jobs[w].status != 0) rc = jobs[w].status;
    free(jobs); free(tids); free(live);
    return rc;
}
