/*
 * kda_oracle.c -- fp64 token-by-token recurrence of the Kimi Delta Attention forward.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py. It shares nothing with the HIP library.
 *
 * Definition (read off the chunked listing of "手撕KDA" ("KDA by hand"), section 1, with a
 * one-token chunk; the recurrent form is named there in section 5 as the cross-check): for
 * each sequence s and value head j, with q/k head h = j / (HV / H) and state S[K][V]:
 *     S        <- diag(exp(g_t)) S
 *     r        <- v_t - S^T k_t
 *     S        <- S + beta_t k_t r^T
 *     o_t      <- scale * S^T q_t          (read after the write)
 *     final[s,j] = S
 *
 * Layouts (row-major, packed token axis of T_total = sum of sequence lengths):
 *     q, k  [T_total][H][K]   v [T_total][HV][V]   g [T_total][HV][K]   beta [T_total][HV]
 *     h0, ht [N][HV][K][V]    o [T_total][HV][V]
 * Inputs are fp32 (exact carriers of the bf16 or fp32 values the GPU reads); all arithmetic
 * and outputs are fp64. Sequence s spans tokens [bounds[s], bounds[s+1]).
 *
 * Independent (s, j) units run on a pool of POSIX threads. `units` (pairs s, j) restricts the
 * work to a sample; o and ht are then written only for those units.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int N, H, HV, K, V;
    double scale;
    const int64_t *bounds;
    const float *q, *k, *v, *g, *beta, *h0;
    double *o, *ht;
    const int32_t *units;
    int n_units;
    int next;               /* shared work counter */
} job_t;

static void run_unit(const job_t *J, int s, int j, double *S)
{
    const int H = J->H, HV = J->HV, K = J->K, V = J->V;
    const int h = j / (HV / H);
    if (J->h0) {
        const float *src = J->h0 + ((size_t)s * HV + j) * (size_t)K * V;
        for (size_t i = 0; i < (size_t)K * V; ++i) S[i] = (double)src[i];
    } else {
        memset(S, 0, sizeof(double) * (size_t)K * V);
    }
    double r[1024];
    for (int64_t t = J->bounds[s]; t < J->bounds[s + 1]; ++t) {
        const float *qt = J->q + ((size_t)t * H + h) * K;
        const float *kt = J->k + ((size_t)t * H + h) * K;
        const float *vt = J->v + ((size_t)t * HV + j) * V;
        const float *gt = J->g + ((size_t)t * HV + j) * K;
        const double bt = (double)J->beta[(size_t)t * HV + j];
        /* decay */
        for (int d = 0; d < K; ++d) {
            const double a = exp((double)gt[d]);
            double *row = S + (size_t)d * V;
            for (int n = 0; n < V; ++n) row[n] *= a;
        }
        /* residual r = v - S^T k */
        for (int n = 0; n < V; ++n) r[n] = (double)vt[n];
        for (int d = 0; d < K; ++d) {
            const double kd = (double)kt[d];
            const double *row = S + (size_t)d * V;
            for (int n = 0; n < V; ++n) r[n] -= row[n] * kd;
        }
        /* rank-1 write S += beta k r^T */
        for (int d = 0; d < K; ++d) {
            const double c = bt * (double)kt[d];
            double *row = S + (size_t)d * V;
            for (int n = 0; n < V; ++n) row[n] += c * r[n];
        }
        /* read o = scale S^T q */
        if (J->o) {
            double *ot = J->o + ((size_t)t * HV + j) * V;
            for (int n = 0; n < V; ++n) ot[n] = 0.0;
            for (int d = 0; d < K; ++d) {
                const double qd = (double)qt[d];
                const double *row = S + (size_t)d * V;
                for (int n = 0; n < V; ++n) ot[n] += row[n] * qd;
            }
            for (int n = 0; n < V; ++n) ot[n] *= J->scale;
        }
    }
    if (J->ht) {
        double *dst = J->ht + ((size_t)s * HV + j) * (size_t)K * V;
        memcpy(dst, S, sizeof(double) * (size_t)K * V);
    }
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->K * J->V);
    if (!S) return (void *)1;
    const int total = J->units ? J->n_units : J->N * J->HV;
    for (;;) {
        const int u = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (u >= total) break;
        int s, j;
        if (J->units) { s = J->units[2 * u]; j = J->units[2 * u + 1]; }
        else { s = u / J->HV; j = u % J->HV; }
        run_unit(J, s, j, S);
    }
    free(S);
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on a thread or allocation failure. */
int kda_oracle_fwd(int N, const int64_t *bounds, int H, int HV, int K, int V, double scale,
                   const float *q, const float *k, const float *v, const float *g,
                   const float *beta, const float *h0, double *o, double *ht,
                   const int32_t *units, int n_units, int n_threads)
{
    if (N < 0 || !bounds || H <= 0 || HV <= 0 || HV % H || K <= 0 || V <= 0 || V > 1024)
        return -1;
    if (!q || !k || !v || !g || !beta) return -1;
    job_t J = {N, H, HV, K, V, scale, bounds, q, k, v, g, beta, h0, o, ht, units, n_units, 0};
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) { rc = -2; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret) rc = -2;
    }
    return rc;
}
