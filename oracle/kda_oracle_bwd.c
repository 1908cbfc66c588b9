/*
 * kda_oracle_bwd.c -- fp64 gradients of the Kimi Delta Attention forward, token by token.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/ (the full-size backward parity). It shares
 * nothing with the HIP library.
 *
 * The forward is the token recurrence of kda_oracle.c (read off the chunked listing of
 * "手撕KDA" ("KDA by hand"), section 1, with a one-token chunk; section 5 names the recurrent
 * form as the cross-check): per token t, value head j, q/k head h = j / (HV / H),
 *     S' = diag(exp g_t) S;  r = v_t - S'^T k_t;  S_t = S' + beta_t k_t r^T;
 *     o_t = scale S_t^T q_t
 * and final_state = S_T. The loss is L = sum(o * do) + sum(final_state * dht). Section 2.1 of
 * the same page walks the chunks in reverse, carrying the state gradient from the final state
 * backwards; here the carried quantity is dS = dL/dS_t, token by token, newest first:
 *     dS     += scale q_t do_t^T            (o_t reads S_t)
 *     dq_t   += scale S_t do_t
 *     u       = dS^T k_t;  dr = beta_t u    (S_t = S' + beta k r^T)
 *     dbeta_t = r . u
 *     dk_t   += beta_t dS r - S' dr         (r = v - S'^T k contributes -S' dr)
 *     dv_t    = dr
 *     dS'     = dS - k_t dr^T
 *     dg_t    = rowsum(dS' * S')            (S' = diag(e^g) S: d/dg_d = S'_d. dS'_d.)
 *     dS      = diag(exp g_t) dS'           (now dL/dS_{t-1})
 * and dh0 = dS after the sequence's first token. dq and dk of a q/k head sum over the G value
 * heads of its group. Each line is the chain rule of one forward line, in reverse order.
 *
 * The states S' of a sequence are rebuilt by re-running the forward: a first pass keeps S at
 * every CK-th token, and each CK-token segment is then recomputed from its checkpoint (keeping
 * S' and r of its tokens) and walked backwards. The arithmetic is the same fp64 forward, so
 * the recomputed states equal the first pass's bit for bit.
 *
 * Layouts as in kda_oracle.c (packed token axis, row-major):
 *     q, k, dq, dk [T_total][H][K]   v, do, dv [T_total][HV][V]   g, dg [T_total][HV][K]
 *     beta, dbeta [T_total][HV]      h0, dht, dh0 [N][HV][K][V]
 * Inputs are fp32 (exact carriers of the bf16 or fp32 values the GPU reads); h0, dht and do
 * may be NULL (zero). Outputs are fp64 and fully written (tokens outside every sequence
 * stay as the caller initialised them). Work is split over (sequence, q/k head) tasks on a
 * pool of POSIX threads, so each task owns its rows of dq and dk.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CK 256

typedef struct {
    int N, H, HV, K, V;
    double scale;
    const int64_t *bounds;
    const float *q, *k, *v, *g, *beta, *h0, *dout, *dht;
    double *dq, *dk, *dv, *dg, *dbeta, *dh0;
    int next;               /* shared task counter */
} bjob_t;

typedef struct {
    double *ckpt;   /* [n_ck][K][V]: S before token bos + CK c */
    double *sp;     /* [CK][K][V]: S' of the segment's tokens */
    double *st;     /* [K][V]: S_t of the token being walked */
    double *rr;     /* [CK][V]: r of the segment's tokens */
    double *dS;     /* [K][V] */
    double *tmp;    /* [V] + [V] */
} bwork_t;

static inline size_t kv(const bjob_t *J) { return (size_t)J->K * J->V; }

/* One forward token on S (in place): S <- diag(e^g) S, r = v - S^T k, S += beta k r^T. When
 * sp_out is not NULL it receives S' (after the decay, before the write); r_out receives r. */
static void fwd_token(const bjob_t *J, int64_t t, int h, int j, double *S, double *sp_out,
                      double *r_out)
{
    const int H = J->H, HV = J->HV, K = J->K, V = J->V;
    const float *kt = J->k + ((size_t)t * H + h) * K;
    const float *vt = J->v + ((size_t)t * HV + j) * V;
    const float *gt = J->g + ((size_t)t * HV + j) * K;
    const double bt = (double)J->beta[(size_t)t * HV + j];
    for (int d = 0; d < K; ++d) {
        const double a = exp((double)gt[d]);
        double *row = S + (size_t)d * V;
        for (int n = 0; n < V; ++n) row[n] *= a;
    }
    if (sp_out) memcpy(sp_out, S, sizeof(double) * kv(J));
    for (int n = 0; n < V; ++n) r_out[n] = (double)vt[n];
    for (int d = 0; d < K; ++d) {
        const double kd = (double)kt[d];
        const double *row = S + (size_t)d * V;
        for (int n = 0; n < V; ++n) r_out[n] -= row[n] * kd;
    }
    for (int d = 0; d < K; ++d) {
        const double c = bt * (double)kt[d];
        double *row = S + (size_t)d * V;
        for (int n = 0; n < V; ++n) row[n] += c * r_out[n];
    }
}

/* The reverse walk over one (sequence s, value head j); dq, dk of q/k head h accumulate. */
static void bwd_unit(const bjob_t *J, bwork_t *W, int s, int j)
{
    const int H = J->H, HV = J->HV, K = J->K, V = J->V;
    const int h = j / (HV / H);
    const int64_t bos = J->bounds[s], eos = J->bounds[s + 1];
    const int64_t len = eos - bos;
    const size_t KV = kv(J);
    double *S = W->dS;                   /* forward pass state (dS is free until the walk) */
    if (J->h0) {
        const float *src = J->h0 + ((size_t)s * HV + j) * KV;
        for (size_t i = 0; i < KV; ++i) S[i] = (double)src[i];
    } else {
        memset(S, 0, sizeof(double) * KV);
    }
    /* pass 1: checkpoints every CK tokens */
    const int64_t n_ck = len > 0 ? (len + CK - 1) / CK : 0;
    double *r = W->tmp;
    for (int64_t c = 0; c < n_ck; ++c) {
        memcpy(W->ckpt + (size_t)c * KV, S, sizeof(double) * KV);
        const int64_t t1 = bos + (c + 1) * CK < eos ? bos + (c + 1) * CK : eos;
        for (int64_t t = bos + c * CK; t < t1; ++t) fwd_token(J, t, h, j, S, NULL, r);
    }
    /* the walk, newest segment first */
    double *dS = W->dS;
    if (J->dht) {
        const float *src = J->dht + ((size_t)s * HV + j) * KV;
        for (size_t i = 0; i < KV; ++i) dS[i] = (double)src[i];
    } else {
        memset(dS, 0, sizeof(double) * KV);
    }
    double *u = W->tmp, *dr = W->tmp + V;
    for (int64_t c = n_ck - 1; c >= 0; --c) {
        const int64_t t0 = bos + c * CK;
        const int64_t t1 = t0 + CK < eos ? t0 + CK : eos;
        /* recompute the segment: S' and r of each token; st carries S */
        memcpy(W->st, W->ckpt + (size_t)c * KV, sizeof(double) * KV);
        for (int64_t t = t0; t < t1; ++t)
            fwd_token(J, t, h, j, W->st, W->sp + (size_t)(t - t0) * KV,
                      W->rr + (size_t)(t - t0) * V);
        /* W->st is now S after token t1 - 1 */
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double *sp = W->sp + (size_t)(t - t0) * KV;
            const double *rt = W->rr + (size_t)(t - t0) * V;
            const float *qt = J->q + ((size_t)t * H + h) * K;
            const float *kt = J->k + ((size_t)t * H + h) * K;
            const float *gt = J->g + ((size_t)t * HV + j) * K;
            const double bt = (double)J->beta[(size_t)t * HV + j];
            double *dqt = J->dq + ((size_t)t * H + h) * K;
            double *dkt = J->dk + ((size_t)t * H + h) * K;
            double *dvt = J->dv + ((size_t)t * HV + j) * V;
            double *dgt = J->dg + ((size_t)t * HV + j) * K;
            const double *St = W->st;     /* S_t, the state o_t reads */
            if (J->dout) {
                const float *dot = J->dout + ((size_t)t * HV + j) * V;
                /* dq_t += scale S_t do_t */
                for (int d = 0; d < K; ++d) {
                    const double *row = St + (size_t)d * V;
                    double acc = 0.0;
                    for (int n = 0; n < V; ++n) acc += row[n] * (double)dot[n];
                    dqt[d] += J->scale * acc;
                }
                /* dS += scale q_t do_t^T */
                for (int d = 0; d < K; ++d) {
                    const double c0 = J->scale * (double)qt[d];
                    double *row = dS + (size_t)d * V;
                    for (int n = 0; n < V; ++n) row[n] += c0 * (double)dot[n];
                }
            }
            /* u = dS^T k, dr = beta u, dbeta = r . u */
            for (int n = 0; n < V; ++n) u[n] = 0.0;
            for (int d = 0; d < K; ++d) {
                const double kd = (double)kt[d];
                const double *row = dS + (size_t)d * V;
                for (int n = 0; n < V; ++n) u[n] += row[n] * kd;
            }
            double db = 0.0;
            for (int n = 0; n < V; ++n) {
                dr[n] = bt * u[n];
                db += rt[n] * u[n];
                dvt[n] = dr[n];
            }
            J->dbeta[(size_t)t * HV + j] = db;
            /* dk_t += beta dS r - S' dr */
            for (int d = 0; d < K; ++d) {
                const double *row = dS + (size_t)d * V;
                const double *prow = sp + (size_t)d * V;
                double a = 0.0, b = 0.0;
                for (int n = 0; n < V; ++n) {
                    a += row[n] * rt[n];
                    b += prow[n] * dr[n];
                }
                dkt[d] += bt * a - b;
            }
            /* dS' = dS - k dr^T; dg = rowsum(dS' * S'); dS = diag(e^g) dS' */
            for (int d = 0; d < K; ++d) {
                const double kd = (double)kt[d];
                const double e = exp((double)gt[d]);
                double *row = dS + (size_t)d * V;
                const double *prow = sp + (size_t)d * V;
                double acc = 0.0;
                for (int n = 0; n < V; ++n) {
                    row[n] -= kd * dr[n];
                    acc += row[n] * prow[n];
                    row[n] *= e;
                }
                dgt[d] = acc;
            }
            /* the next (older) token reads its own S_t, i.e. S_{t-1} = S'_{t-1} + beta_{t-1}
             * k_{t-1} r_{t-1}^T: formed from the stored S' and r of token t - 1 with the
             * forward's own operations, so it equals the forward's value bit for bit */
            if (t > t0) {
                const double *spp = W->sp + (size_t)(t - 1 - t0) * KV;
                const double *rp = W->rr + (size_t)(t - 1 - t0) * V;
                const float *kp = J->k + ((size_t)(t - 1) * H + h) * K;
                const double bp = (double)J->beta[(size_t)(t - 1) * HV + j];
                for (int d = 0; d < K; ++d) {
                    const double c0 = bp * (double)kp[d];
                    const double *prow = spp + (size_t)d * V;
                    double *row = W->st + (size_t)d * V;
                    for (int n = 0; n < V; ++n) row[n] = prow[n] + c0 * rp[n];
                }
            } else if (c > 0) {
                /* token t0 - 1 is the previous segment's newest: its S_t is checkpoint c */
                memcpy(W->st, W->ckpt + (size_t)c * KV, sizeof(double) * KV);
            }
        }
    }
    if (J->dh0) memcpy(J->dh0 + ((size_t)s * HV + j) * KV, dS, sizeof(double) * KV);
}

static void *bworker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    const size_t KV = kv(J);
    int64_t max_len = 0;
    for (int s = 0; s < J->N; ++s) {
        const int64_t l = J->bounds[s + 1] - J->bounds[s];
        if (l > max_len) max_len = l;
    }
    bwork_t W;
    const size_t n_ck_max = (size_t)((max_len + CK - 1) / CK);
    W.ckpt = (double *)malloc(sizeof(double) * KV * (n_ck_max ? n_ck_max : 1));
    W.sp = (double *)malloc(sizeof(double) * KV * CK);
    W.st = (double *)malloc(sizeof(double) * KV);
    W.rr = (double *)malloc(sizeof(double) * (size_t)J->V * CK);
    W.dS = (double *)malloc(sizeof(double) * KV);
    W.tmp = (double *)malloc(sizeof(double) * 2 * (size_t)J->V);
    void *ret = NULL;
    if (!W.ckpt || !W.sp || !W.st || !W.rr || !W.dS || !W.tmp) {
        ret = (void *)1;
    } else {
        const int G = J->HV / J->H;
        const int total = J->N * J->H;
        for (;;) {
            const int task = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
            if (task >= total) break;
            const int s = task / J->H, h = task % J->H;
            const int64_t bos = J->bounds[s], eos = J->bounds[s + 1];
            for (int64_t t = bos; t < eos; ++t) {
                memset(J->dq + ((size_t)t * J->H + h) * J->K, 0, sizeof(double) * J->K);
                memset(J->dk + ((size_t)t * J->H + h) * J->K, 0, sizeof(double) * J->K);
            }
            for (int jj = 0; jj < G; ++jj) bwd_unit(J, &W, s, h * G + jj);
        }
    }
    free(W.ckpt); free(W.sp); free(W.st); free(W.rr); free(W.dS); free(W.tmp);
    return ret;
}

/* Returns 0 on success, -1 on bad arguments, -2 on a thread or allocation failure. Sequence
 * s spans tokens [bounds[s], bounds[s+1]) (nondecreasing). dh0 may be NULL. */
int kda_oracle_bwd(int N, const int64_t *bounds, int H, int HV, int K, int V, double scale,
                   const float *q, const float *k, const float *v, const float *g,
                   const float *beta, const float *h0, const float *dout, const float *dht,
                   double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0,
                   int n_threads)
{
    if (N < 0 || !bounds || H <= 0 || HV <= 0 || HV % H || K <= 0 || V <= 0) return -1;
    if (!q || !k || !v || !g || !beta || !dq || !dk || !dv || !dg || !dbeta) return -1;
    for (int s = 0; s < N; ++s)
        if (bounds[s + 1] < bounds[s] || bounds[s] < 0) return -1;
    bjob_t J = {N, H, HV, K, V, scale, bounds, q, k, v, g, beta, h0, dout, dht,
                dq, dk, dv, dg, dbeta, dh0, 0};
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, bworker, &J) != 0) { rc = -2; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret) rc = -2;
    }
    return rc;
}
