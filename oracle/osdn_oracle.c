/*
 * CPU float64 oracle for the Online Scaled DeltaNet (OSDN) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path includes, links or calls this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares
 * no code, header or constant with the HIP library.
 *
 * What it computes is the plain token-by-token recurrence, written out as defined:
 *
 *   OSDN write (OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
 *   Attention, technical summary, section 2.1): one gradient step on the per-token loss
 *   f_t(S) = 1/2 ||S k_t - v_t||^2 (same summary, section 1), right-preconditioned by
 *   D_t = diag(d_t).  It equals a write with the scaled key  k~_t = d_t (.) k_t  while the
 *   residual keeps the plain key:
 *        S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k~_t^T .
 *   Gated form (Erase-then-Delta Attention, section 2.2, eq. 4): a per-head scalar
 *   alpha_t in (0,1] decays the old state before the delta step.
 *   Channel-wise form (Erase-then-Delta Attention, section 2.2, eq. 5, the Kimi Delta
 *   Attention gate; section 3.2, eq. 7): a per-token diagonal Diag(a_t), one retention
 *   factor per key feature, decays the old state (its key-indexed rows) before the delta
 *   step, in place of (or on top of) the scalar gate.
 *   Read-out (Erase-then-Delta Attention, section 2.1, eq. 1): o_t = S_t^T q_t in that
 *   page's dk x dv convention, i.e. after the write.
 *
 * Storage convention: M = S^T in R^{dk x dv}, row-major [dk][dv] per (b,h).  One token is
 *        M <- alpha_t M                     (scalar gate), then
 *        M[i][:] <- a_t[i] M[i][:]          (channel-wise gate), then
 *        r <- v_t - M^T k_t
 *        M <- M + beta_t (d_t (.) k_t) r^T
 *        o_t <- M^T q_t
 * Inputs are float64 (exact upcasts of the stored values).  Sequences (b,h) are independent
 * and are spread over POSIX threads; each thread runs the plain loops above.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *beta, *d, *alpha, *alpha_ch, *S0;
    double *o, *S_T;
    int64_t BH, T, dk, dv;
    int64_t first, stride;
    int status;
} oracle_job;

/* One (b,h) sequence of T tokens. */
static int run_sequence(const oracle_job *J, int64_t bh) {
    const int64_t T = J->T, dk = J->dk, dv = J->dv;
    const double *q = J->q + bh * T * dk;
    const double *k = J->k + bh * T * dk;
    const double *v = J->v + bh * T * dv;
    const double *beta = J->beta + bh * T;
    const double *d = J->d + bh * T * dk;
    const double *alpha = J->alpha ? J->alpha + bh * T : NULL;
    const double *alpha_ch = J->alpha_ch ? J->alpha_ch + bh * T * dk : NULL;
    double *o = J->o ? J->o + bh * T * dv : NULL;

    double *M = (double *)malloc((size_t)(dk * dv) * sizeof(double));
    double *r = (double *)malloc((size_t)dv * sizeof(double));
    if (!M || !r) {
        free(M);
        free(r);
        return -1;
    }
    if (J->S0)
        memcpy(M, J->S0 + bh * dk * dv, (size_t)(dk * dv) * sizeof(double));
    else
        memset(M, 0, (size_t)(dk * dv) * sizeof(double));

    for (int64_t t = 0; t < T; ++t) {
        const double *qt = q + t * dk, *kt = k + t * dk, *vt = v + t * dv, *dt = d + t * dk;
        const double a = alpha ? alpha[t] : 1.0;
        const double b = beta[t];

        /* decay of the old state: scalar gate, then one factor per key feature (row) */
        for (int64_t i = 0; i < dk * dv; ++i) M[i] *= a;
        if (alpha_ch)
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) M[i * dv + j] *= alpha_ch[t * dk + i];

        /* residual against the plain key: r = v - M^T k */
        for (int64_t j = 0; j < dv; ++j) r[j] = vt[j];
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) r[j] -= M[i * dv + j] * kt[i];

        /* write along the preconditioned key k~ = d (.) k, scaled by beta */
        for (int64_t i = 0; i < dk; ++i) {
            const double w = b * (dt[i] * kt[i]);
            for (int64_t j = 0; j < dv; ++j) M[i * dv + j] += w * r[j];
        }

        /* read-out after the write: o = M^T q */
        if (o) {
            double *ot = o + t * dv;
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) ot[j] += M[i * dv + j] * qt[i];
        }
    }
    if (J->S_T) memcpy(J->S_T + bh * dk * dv, M, (size_t)(dk * dv) * sizeof(double));
    free(M);
    free(r);
    return 0;
}

static void *worker(void *arg) {
    oracle_job *J = (oracle_job *)arg;
    J->status = 0;
    for (int64_t bh = J->first; bh < J->BH; bh += J->stride)
        if (run_sequence(J, bh) != 0) J->status = -1;
    return NULL;
}

/*
 * q, k, d: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T]; alpha: [B,H,T] or NULL (no scalar
 * decay); alpha_ch: [B,H,T,dk] or NULL (no channel-wise decay); S0: [B,H,dk,dv] or NULL
 * (zero state); o: [B,H,T,dv] or NULL; S_T: [B,H,dk,dv] or NULL.
 * S_T may equal S0 (each sequence copies its S0 slice before writing S_T).
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int osdn_oracle_fwd2(const double *q, const double *k, const double *v, const double *beta,
                     const double *d, const double *alpha, const double *alpha_ch,
                     const double *S0, double *o, double *S_T, int64_t B, int64_t H, int64_t T,
                     int64_t dk, int64_t dv, int nthreads) {
    if (!q || !k || !v || !beta || !d) return -1;
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    const int64_t BH = B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > BH) nthreads = BH > 0 ? (int)BH : 1;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -1;
    }
    for (int w = 0; w < nthreads; ++w) {
        oracle_job J = {q, k, v, beta, d, alpha, alpha_ch, S0, o, S_T, BH, T, dk, dv,
                        w, nthreads, 0};
        jobs[w] = J;
    }
    int status = 0;
    if (nthreads == 1) {
        worker(&jobs[0]);
        status = jobs[0].status;
    } else {
        int started = 0;
        for (int w = 0; w < nthreads; ++w) {
            if (pthread_create(&tid[w], NULL, worker, &jobs[w]) != 0) break;
            ++started;
        }
        for (int w = 0; w < started; ++w) pthread_join(tid[w], NULL);
        /* sequences of threads that failed to start run here */
        for (int w = started; w < nthreads; ++w) worker(&jobs[w]);
        for (int w = 0; w < nthreads; ++w) status |= jobs[w].status;
    }
    free(jobs);
    free(tid);
    return status;
}

/* The same without the channel-wise gate. */
int osdn_oracle_fwd(const double *q, const double *k, const double *v, const double *beta,
                    const double *d, const double *alpha, const double *S0, double *o,
                    double *S_T, int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                    int nthreads) {
    return osdn_oracle_fwd2(q, k, v, beta, d, alpha, NULL, S0, o, S_T, B, H, T, dk, dv,
                            nthreads);
}
