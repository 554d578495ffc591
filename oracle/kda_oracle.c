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

/*
 * Backward of the whole recurrence, token by token (backpropagation through
 * the sequence).  The pages give no backward; the ai-pulse-lab summary of the
 * technical report (KDA paragraph) says only that the log-decay bound serves
 * training speed.  What is computed is the plain definition: the gradient of
 *
 *   L = sum_t <d_o_t, o_t> + <d_hT, hT>,   (o, hT) = the recurrence above,
 *
 * obtained by running the recurrence forward while keeping the state before
 * every token, then taking the tokens in reverse order and differentiating
 * each one's assignments in reverse (the L2 norms included).  For one token,
 * with St = Diag(exp g) S_prev, p = St^T kh, u = beta (v - p),
 * Sn = St + kh u^T, o = scale Sn^T qh, and G = dL/dSn (the gradient carried
 * from the later tokens) plus scale qh d_o^T:
 *
 *   dqh = scale Sn d_o,   du = G^T kh,   dkh = G u + St dp,
 *   dv = beta du,   dbeta = du . (v - p),   dp = -beta du,
 *   dSt = G + kh dp^T,   dS_prev = Diag(exp g) dSt,   dg_i = sum_j St_ij dSt_ij,
 *   dq = (dqh - qh (qh . dqh)) / sqrt(|q|^2 + eps)   (likewise dk),
 *
 * and dS_prev is the G of the token before.  dh0 is the last dS_prev.
 * Every state is kept: T * dk * dv doubles per sequence in flight.
 */
typedef struct {
    int n_seq, T, dk, dv;
    const double *q, *k, *v, *g, *beta, *h0, *d_o, *d_hT;
    double scale, eps;
    double *dq, *dkk, *dvv, *dg, *dbeta, *dh0;
    int first, stride;
    int status;
} bjob_t;

static void backward_sequence(const bjob_t *jb, int s, double *states, double *G, double *St,
                              double *w) {
    const int T = jb->T, dk = jb->dk, dv = jb->dv;
    const size_t nS = (size_t)dk * dv;
    const double *q = jb->q + (size_t)s * T * dk, *k = jb->k + (size_t)s * T * dk;
    const double *v = jb->v + (size_t)s * T * dv, *g = jb->g + (size_t)s * T * dk;
    const double *beta = jb->beta + (size_t)s * T, *d_o = jb->d_o + (size_t)s * T * dv;
    double *qh = w, *kh = w + dk, *p = w + 2 * dk, *u = p + dv, *du = u + dv;
    double *dqh = du + dv, *dkh = dqh + dk, *dp = dkh + dk, *a = dp + dv;

    /* forward: states[t] is the state before token t, states[T] the last */
    double *S = states;
    if (jb->h0)
        memcpy(S, jb->h0 + (size_t)s * nS, sizeof(double) * nS);
    else
        memset(S, 0, sizeof(double) * nS);
    for (int t = 0; t < T; ++t) {
        const double *kt = k + (size_t)t * dk, *gt = g + (size_t)t * dk;
        const double *vt = v + (size_t)t * dv;
        double *Sn = states + (size_t)(t + 1) * nS;
        double sk = 0.0;
        for (int i = 0; i < dk; ++i) sk += kt[i] * kt[i];
        const double nk = sqrt(sk + jb->eps);
        for (int i = 0; i < dk; ++i) kh[i] = nk > 0.0 ? kt[i] / nk : 0.0;
        for (int i = 0; i < dk; ++i) {
            const double ai = exp(gt[i]);
            for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] = ai * S[(size_t)i * dv + j];
        }
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += kh[i] * Sn[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) u[j] = beta[t] * (vt[j] - p[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] += kh[i] * u[j];
        S = Sn;
    }

    /* reverse */
    if (jb->d_hT)
        memcpy(G, jb->d_hT + (size_t)s * nS, sizeof(double) * nS);
    else
        memset(G, 0, sizeof(double) * nS);
    for (int t = T - 1; t >= 0; --t) {
        const double *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk;
        const double *gt = g + (size_t)t * dk, *vt = v + (size_t)t * dv;
        const double *dot = d_o + (size_t)t * dv;
        const double *Sp = states + (size_t)t * nS, *Sn = states + (size_t)(t + 1) * nS;
        const double bt = beta[t];
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; ++i) {
            sq += qt[i] * qt[i];
            sk += kt[i] * kt[i];
        }
        const double nq = sqrt(sq + jb->eps), nk = sqrt(sk + jb->eps);
        for (int i = 0; i < dk; ++i) {
            qh[i] = nq > 0.0 ? qt[i] / nq : 0.0;
            kh[i] = nk > 0.0 ? kt[i] / nk : 0.0;
            a[i] = exp(gt[i]);
        }
        /* the token's forward quantities again: St, p, u */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) St[(size_t)i * dv + j] = a[i] * Sp[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += kh[i] * St[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - p[j]);
        /* o = scale Sn^T qh: into G and dqh */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                G[(size_t)i * dv + j] += jb->scale * qh[i] * dot[j];
                acc += Sn[(size_t)i * dv + j] * dot[j];
            }
            dqh[i] = jb->scale * acc;
        }
        /* Sn = St + kh u^T */
        for (int j = 0; j < dv; ++j) du[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += G[(size_t)i * dv + j] * u[j];
                du[j] += G[(size_t)i * dv + j] * kh[i];
            }
            dkh[i] = acc;
        }
        /* u = beta (v - p) */
        double db = 0.0;
        for (int j = 0; j < dv; ++j) {
            jb->dvv[((size_t)s * T + t) * dv + j] = bt * du[j];
            db += du[j] * (vt[j] - p[j]);
            dp[j] = -bt * du[j];
        }
        jb->dbeta[(size_t)s * T + t] = db;
        /* p = St^T kh; St = Diag(a) S_prev.  G becomes dL/dS_prev */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0, dgi = 0.0;
            for (int j = 0; j < dv; ++j) {
                const double dst = G[(size_t)i * dv + j] + kh[i] * dp[j];
                acc += St[(size_t)i * dv + j] * dp[j];
                dgi += St[(size_t)i * dv + j] * dst;
                G[(size_t)i * dv + j] = a[i] * dst;
            }
            dkh[i] += acc;
            jb->dg[((size_t)s * T + t) * dk + i] = dgi;
        }
        /* qh = q / sqrt(|q|^2 + eps), likewise k */
        double qd = 0.0, kd = 0.0;
        for (int i = 0; i < dk; ++i) {
            qd += qh[i] * dqh[i];
            kd += kh[i] * dkh[i];
        }
        for (int i = 0; i < dk; ++i) {
            jb->dq[((size_t)s * T + t) * dk + i] = nq > 0.0 ? (dqh[i] - qh[i] * qd) / nq : 0.0;
            jb->dkk[((size_t)s * T + t) * dk + i] = nk > 0.0 ? (dkh[i] - kh[i] * kd) / nk : 0.0;
        }
    }
    if (jb->dh0) memcpy(jb->dh0 + (size_t)s * nS, G, sizeof(double) * nS);
}

static void *bworker(void *arg) {
    bjob_t *jb = (bjob_t *)arg;
    const size_t nS = (size_t)jb->dk * jb->dv;
    double *states = (double *)malloc(sizeof(double) * nS * ((size_t)jb->T + 1));
    double *G = (double *)malloc(sizeof(double) * nS);
    double *St = (double *)malloc(sizeof(double) * nS);
    double *w = (double *)malloc(sizeof(double) * (5 * (size_t)jb->dk + 4 * (size_t)jb->dv));
    if (!states || !G || !St || !w) {
        jb->status = -2;
    } else {
        for (int s = jb->first; s < jb->n_seq; s += jb->stride)
            backward_sequence(jb, s, states, G, St, w);
        jb->status = 0;
    }
    free(states); free(G); free(St); free(w);
    return NULL;
}

/*
 * Gradients of L = <d_o, o> + <d_hT, hT> for n_seq independent sequences.
 * Layouts as kda_oracle_run; d_o [n_seq][T][dv]; d_hT, dh0 [n_seq][dk][dv]
 * (d_hT NULL = zero, dh0 NULL = not stored; h0 NULL = zero state).  Outputs
 * dq, dk, dg [n_seq][T][dk], dv [n_seq][T][dv], dbeta [n_seq][T].  Each
 * worker thread holds (T + 1) * dk * dv doubles of states.  Returns 0, -1 on
 * a bad argument, -2 when memory or threads fail.
 */
int kda_oracle_seq_backward(int n_seq, int T, int dk, int dv,
                            const double *q, const double *k, const double *v,
                            const double *g, const double *beta, double scale, double eps,
                            const double *h0, const double *d_o, const double *d_hT,
                            double *dq, double *dkk, double *dvv, double *dg, double *dbeta,
                            double *dh0, int n_threads) {
    if (n_seq < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (n_seq == 0) return 0;
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dkk || !dvv || !dg ||
                  !dbeta))
        return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > n_seq) n_threads = n_seq;

    bjob_t *jobs = (bjob_t *)calloc((size_t)n_threads, sizeof(bjob_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    char *live = (char *)calloc((size_t)n_threads, 1);
    if (!jobs || !tids || !live) { free(jobs); free(tids); free(live); return -2; }

    int rc = 0;
    for (int w = 0; w < n_threads; ++w) {
        bjob_t *jb = &jobs[w];
        jb->n_seq = n_seq; jb->T = T; jb->dk = dk; jb->dv = dv;
        jb->q = q; jb->k = k; jb->v = v; jb->g = g; jb->beta = beta; jb->h0 = h0;
        jb->d_o = d_o; jb->d_hT = d_hT; jb->scale = scale; jb->eps = eps;
        jb->dq = dq; jb->dkk = dkk; jb->dvv = dvv; jb->dg = dg; jb->dbeta = dbeta;
        jb->dh0 = dh0;
        jb->first = w; jb->stride = n_threads; jb->status = -2;
        if (n_threads == 1) {
            bworker(jb);
        } else if (pthread_create(&tids[w], NULL, bworker, jb) == 0) {
            live[w] = 1;
        } else {
            bworker(jb);
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
