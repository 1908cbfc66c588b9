// kda_backward.hip -- gradients of the chunked KDA forward: dq, dk, dv, dg, dbeta and dh0 from
// the gradients of o and of the final state. fp32 arithmetic throughout, 16-token chunks.
//
// The chunked form of the forward ("手撕KDA" section 1), per chunk c of a (sequence, value
// head), with S the state at the chunk start:
//     delta = U - W S,   O = QD S + Mqk delta,   S_next = diag(E) S + KR^T delta
// with U = A v, W = A KD, A = (I + L)^{-1} diag(beta), L = diag(beta) strict_tril(G),
// G_ij = sum_d k_id k_jd e^{Gam_id - Gam_jd}, Mqk_ij = scale sum_d q_id k_jd e^{Gam_id - Gam_jd}
// (i >= j), KD = k e^{Gam}, QD = scale q e^{Gam}, KR = k e^{gam - Gam}, E = e^{gam}.
// The backward follows the reverse sweep of the C++ chunk backward of "手撕KDA" section 2.1:
// the states at every chunk start are recorded by a forward pass, the gradient of the state
// (Lam = d loss / d S) is carried across chunks newest first,
//     dDelta = Mqk^T dO + KR Lam_next,   Lam = diag(E) Lam_next + QD^T dO - W^T dDelta,
// and every chunk then back-propagates its own quantities to its tokens independently. Launches:
//   prepare_f32 (kda_prepare.hip)  the chunk records (W, QD, KR, U, Mqk, E) in fp32
//   bwd_states_kernel              S at the start of every chunk
//   bwd_chain_kernel               Lam at the end of every chunk, and dh0
//   bwd_local_kernel               per (chunk, value head): dv, dg, dbeta and dq, dk
//   bwd_group_sum_kernel           dq, dk summed over the value heads of a q/k head (G > 1)
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ float ldx(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldx(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

// State at the start of every chunk: one block per (sequence, value head), thread n owns
// column n of S (the fp32 state pass of kda_state.hip without the output).
template <int K, int V>
__global__ __launch_bounds__(V) void bwd_states_kernel(BwdParams b)
{
    const FwdParams &p = b.f;
    using WS = WsF32<K, V>;
    __shared__ float sw[16][K], skr[16][K], seg[K];
    const int n = threadIdx.x;
    const int j = blockIdx.x % p.HV, s = blockIdx.x / p.HV;
    const int64_t bos = seq_bos(p.seq, s), eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CHUNK - 1) / CHUNK);
    const size_t slot0 = (size_t)j * p.seq.n_slots + (size_t)(bos / CHUNK + s);
    float S[K];
    if (p.h0) {
        const float *h0 = p.h0 + ((size_t)s * p.HV + j) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) S[d] = h0[(size_t)d * V];
    } else {
#pragma unroll
        for (int d = 0; d < K; ++d) S[d] = 0.f;
    }
    for (int c = 0; c < nc; ++c) {
        float *ck = b.ck_S + (slot0 + c) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) ck[(size_t)d * V] = S[d];
        const float *ch = (const float *)(p.ws + (slot0 + c) * (size_t)WS::BYTES);
        for (int idx = n; idx < 16 * K; idx += V) {
            sw[idx / K][idx % K] = ch[WS::W / 4 + idx];
            skr[idx / K][idx % K] = ch[WS::KR / 4 + idx];
        }
        for (int idx = n; idx < K; idx += V) seg[idx] = ch[WS::EG / 4 + idx];
        __syncthreads();
        float dl[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = ch[WS::U / 4 + t * V + n];
#pragma unroll
            for (int kk = 0; kk < K; ++kk) acc -= sw[t][kk] * S[kk];
            dl[t] = acc;
        }
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            float acc = seg[kk] * S[kk];
#pragma unroll
            for (int t = 0; t < 16; ++t) acc += skr[t][kk] * dl[t];
            S[kk] = acc;
        }
        __syncthreads();
    }
}

// Gradient of the state, newest chunk first: Lam (thread n: column n) starts as dht; before
// chunk c is processed Lam is the gradient at its end and is recorded; after the first chunk
// it is dh0.
template <int K, int V, typename T>
__global__ __launch_bounds__(V) void bwd_chain_kernel(BwdParams b)
{
    const FwdParams &p = b.f;
    using WS = WsF32<K, V>;
    __shared__ float sw[16][K], sqd[16][K], skr[16][K], smq[16][16], seg[K];
    const int n = threadIdx.x;
    const int j = blockIdx.x % p.HV, s = blockIdx.x / p.HV;
    const int64_t bos = seq_bos(p.seq, s), eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CHUNK - 1) / CHUNK);
    const size_t slot0 = (size_t)j * p.seq.n_slots + (size_t)(bos / CHUNK + s);
    const T *dout = (const T *)b.d_o;
    float L[K];
    if (b.dht) {
        const float *dh = b.dht + ((size_t)s * p.HV + j) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) L[d] = dh[(size_t)d * V];
    } else {
#pragma unroll
        for (int d = 0; d < K; ++d) L[d] = 0.f;
    }
    for (int c = nc - 1; c >= 0; --c) {
        float *ck = b.ck_L + (slot0 + c) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) ck[(size_t)d * V] = L[d];
        const float *ch = (const float *)(p.ws + (slot0 + c) * (size_t)WS::BYTES);
        for (int idx = n; idx < 16 * K; idx += V) {
            sw[idx / K][idx % K] = ch[WS::W / 4 + idx];
            sqd[idx / K][idx % K] = ch[WS::QD / 4 + idx];
            skr[idx / K][idx % K] = ch[WS::KR / 4 + idx];
        }
        for (int idx = n; idx < 256; idx += V) smq[idx / 16][idx % 16] = ch[WS::MQK / 4 + idx];
        for (int idx = n; idx < K; idx += V) seg[idx] = ch[WS::EG / 4 + idx];
        __syncthreads();
        float dO[16], dd[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int64_t tok = bos + 16 * c + t;
            dO[t] = tok < eos ? ldx(dout, (tok * p.HV + j) * V + n) : 0.f;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {            // dDelta = Mqk^T dO + KR Lam
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc += smq[m][t] * dO[m];
#pragma unroll
            for (int kk = 0; kk < K; ++kk) acc += skr[t][kk] * L[kk];
            dd[t] = acc;
        }
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {           // Lam = E Lam + QD^T dO - W^T dDelta
            float acc = seg[kk] * L[kk];
#pragma unroll
            for (int t = 0; t < 16; ++t) acc += sqd[t][kk] * dO[t] - sw[t][kk] * dd[t];
            L[kk] = acc;
        }
        __syncthreads();
    }
    if (b.dh0) {
        float *dh = b.dh0 + ((size_t)s * p.HV + j) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) dh[(size_t)d * V] = L[d];
    }
}

// One block (256 threads) per (chunk slot, value head): recompute the chunk in fp32 and
// back-propagate O, S_next (through delta, U, W, A, the inverse, L, Mqk and the decay factors)
// to the chunk's tokens. Products are formed from exponent differences (every factor
// e^{Gam_i - Gam_j}, i >= j, and e^{gam - Gam} is at most 1). V is visited in blocks of 16
// columns so that only a K x 16 block of S and of Lam sits in LDS (about 105 KB in all at
// K = V = 128, within the 160 KB of one CU).
template <int K, int V>
struct LocalShare {
    static constexpr int VB = 16;
    float q[16][K + 1], k[16][K + 1], gm[16][K + 1];   // q, k, Gam (cumsum of g)
    float v[16][V + 1];
    float w[16][K + 1], kr[16][K + 1];                 // W = A KD, KR
    float dqd[16][K + 1], dkr[16][K + 1], dw[16][K + 1];
    float S[K][VB + 1], L[K][VB + 1];                  // blocks of S and Lam_next
    float dO[16][VB + 1], dl[16][VB + 1], dd[16][VB + 1];
    float G[16][17], Mq[16][17], X[16][17], A[16][17], P[16][17], T1[16][17];
    float dA[16][17], dMq[16][17], dL[16][17];
    float beta[16], dbeta[16], E[K], dE[K];
};

template <int K, int V, typename T>
__global__ __launch_bounds__(256) void bwd_local_kernel(BwdParams b)
{
    const FwdParams &p = b.f;
    constexpr int VB = LocalShare<K, V>::VB;
    __shared__ LocalShare<K, V> sh;
    const int tid = threadIdx.x;
    const int slot = blockIdx.x, j = blockIdx.y, h = j / p.G;
    int s;
    int64_t bos;
    int nvalid;
    if (!locate_slot(p.seq, slot, &s, &bos, &nvalid)) return;
    const size_t gslot = (size_t)j * p.seq.n_slots + slot;
    const float sc = p.scale;
    const T *q = (const T *)p.q, *k = (const T *)p.k, *v = (const T *)p.v;
    const T *g = (const T *)p.g, *bt = (const T *)p.beta, *dout = (const T *)b.d_o;

    // ---- inputs of the chunk (rows past the end are zero) and the cumsum of g
    for (int idx = tid; idx < 16 * K; idx += 256) {
        const int r = idx / K, d = idx % K;
        const bool ok = r < nvalid;
        const int64_t t = bos + r;
        sh.q[r][d] = ok ? ldx(q, (t * p.H + h) * K + d) : 0.f;
        sh.k[r][d] = ok ? ldx(k, (t * p.H + h) * K + d) : 0.f;
        sh.gm[r][d] = ok ? ldx(g, (t * p.HV + j) * K + d) : 0.f;
    }
    for (int idx = tid; idx < 16 * V; idx += 256) {
        const int r = idx / V, d = idx % V;
        sh.v[r][d] = r < nvalid ? ldx(v, ((bos + r) * p.HV + j) * V + d) : 0.f;
    }
    if (tid < 16) {
        sh.beta[tid] = tid < nvalid ? ldx(bt, (bos + tid) * p.HV + j) : 0.f;
        sh.dbeta[tid] = 0.f;
    }
    __syncthreads();
    for (int d = tid; d < K; d += 256) {
        float acc = 0.f;
        for (int r = 0; r < 16; ++r) { acc += sh.gm[r][d]; sh.gm[r][d] = acc; }
        sh.E[d] = __expf(acc);
        sh.dE[d] = 0.f;
    }
    __syncthreads();

    // ---- G (strict lower), Mqk (lower with diagonal), L = diag(beta) G, P = L, INV = I - L
    const int i16 = tid >> 4, j16 = tid & 15;
    {
        float Gv = 0.f, Mv = 0.f;
        if (i16 >= j16) {
            for (int d = 0; d < K; ++d) {
                const float e = __expf(sh.gm[i16][d] - sh.gm[j16][d]);
                Gv += sh.k[i16][d] * sh.k[j16][d] * e;
                Mv += sh.q[i16][d] * sh.k[j16][d] * e;
            }
        }
        sh.G[i16][j16] = i16 > j16 ? Gv : 0.f;
        sh.Mq[i16][j16] = i16 >= j16 ? sc * Mv : 0.f;
        const float Lv = i16 > j16 ? sh.beta[i16] * Gv : 0.f;
        sh.P[i16][j16] = Lv;
        sh.X[i16][j16] = (i16 == j16 ? 1.f : 0.f) - Lv;
    }
    __syncthreads();
    for (int it = 0; it < 3; ++it) {     // Neumann doubling: P <- P^2, X <- X + X P
        float acc = 0.f;
        for (int m = 0; m < 16; ++m) acc += sh.P[i16][m] * sh.P[m][j16];
        __syncthreads();
        sh.P[i16][j16] = acc;
        __syncthreads();
        float add = 0.f;
        for (int m = 0; m < 16; ++m) add += sh.X[i16][m] * sh.P[m][j16];
        sh.T1[i16][j16] = sh.X[i16][j16] + add;
        __syncthreads();
        sh.X[i16][j16] = sh.T1[i16][j16];
        __syncthreads();
    }
    sh.A[i16][j16] = sh.X[i16][j16] * sh.beta[j16];
    sh.dA[i16][j16] = 0.f;
    sh.dMq[i16][j16] = 0.f;
    __syncthreads();

    // ---- W = A KD and KR; zero the K-wide accumulators
    for (int idx = tid; idx < 16 * K; idx += 256) {
        const int t = idx / K, d = idx % K;
        float acc = 0.f;
        for (int m = 0; m < 16; ++m) acc += sh.A[t][m] * sh.k[m][d] * __expf(sh.gm[m][d]);
        sh.w[t][d] = acc;
        sh.kr[t][d] = sh.k[t][d] * __expf(sh.gm[15][d] - sh.gm[t][d]);
        sh.dqd[t][d] = 0.f;
        sh.dkr[t][d] = 0.f;
        sh.dw[t][d] = 0.f;
    }
    __syncthreads();

    // ---- V in blocks of VB columns
    const float *cS = b.ck_S + gslot * (size_t)K * V;
    const float *cL = b.ck_L + gslot * (size_t)K * V;
    for (int vb = 0; vb < V; vb += VB) {
        for (int idx = tid; idx < K * VB; idx += 256) {
            const int d = idx / VB, n = idx % VB;
            sh.S[d][n] = cS[(size_t)d * V + vb + n];
            sh.L[d][n] = cL[(size_t)d * V + vb + n];
        }
        {
            const int t = i16, n = j16;
            const int64_t tok = bos + t;
            sh.dO[t][n] = t < nvalid ? ldx(dout, (tok * p.HV + j) * V + vb + n) : 0.f;
        }
        __syncthreads();
        {   // delta = A v - W S, dDelta = Mqk^T dO + KR Lam (one entry per thread)
            const int t = i16, n = j16;
            float u = 0.f, dd = 0.f;
            for (int m = 0; m < 16; ++m) {
                u += sh.A[t][m] * sh.v[m][vb + n];
                dd += sh.Mq[m][t] * sh.dO[m][n];
            }
            for (int d = 0; d < K; ++d) {
                u -= sh.w[t][d] * sh.S[d][n];
                dd += sh.kr[t][d] * sh.L[d][n];
            }
            sh.dl[t][n] = u;
            sh.dd[t][n] = dd;
        }
        __syncthreads();
        for (int idx = tid; idx < 16 * K; idx += 256) {   // K-wide accumulations over the block
            const int t = idx / K, d = idx % K;
            float aq = 0.f, ar = 0.f, aw = 0.f;
#pragma unroll
            for (int n = 0; n < VB; ++n) {
                aq += sh.dO[t][n] * sh.S[d][n];
                ar += sh.dl[t][n] * sh.L[d][n];
                aw += sh.dd[t][n] * sh.S[d][n];
            }
            sh.dqd[t][d] += aq;
            sh.dkr[t][d] += ar;
            sh.dw[t][d] -= aw;
        }
        for (int d = tid; d < K; d += 256) {
            float acc = 0.f;
#pragma unroll
            for (int n = 0; n < VB; ++n) acc += sh.L[d][n] * sh.S[d][n];
            sh.dE[d] += acc;
        }
        {   // dMqk += dO delta^T, dA += dDelta v^T (dU = dDelta); dv = A^T dDelta
            const int r = i16, c = j16;
            float am = 0.f, aa = 0.f, dv = 0.f;
#pragma unroll
            for (int n = 0; n < VB; ++n) {
                am += sh.dO[r][n] * sh.dl[c][n];
                aa += sh.dd[r][n] * sh.v[c][vb + n];
            }
            sh.dMq[r][c] += am;
            sh.dA[r][c] += aa;
            for (int m = 0; m < 16; ++m) dv += sh.A[m][r] * sh.dd[m][c];
            if (r < nvalid) b.dv[((bos + r) * p.HV + j) * V + vb + c] = dv;
        }
        __syncthreads();
    }

    // ---- dA += dW KD^T; dbeta (columns of A); dX = dA diag(beta)
    {
        const int r = i16, c = j16;
        float acc = 0.f;
        for (int d = 0; d < K; ++d) acc += sh.dw[r][d] * sh.k[c][d] * __expf(sh.gm[c][d]);
        sh.dA[r][c] += acc;
    }
    __syncthreads();
    if (tid < 16) {
        float acc = 0.f;
        for (int r = 0; r < 16; ++r) acc += sh.dA[r][tid] * sh.X[r][tid];
        sh.dbeta[tid] += acc;
    }
    {
        const int r = i16, c = j16;
        sh.T1[r][c] = sh.dA[r][c] * sh.beta[c];                     // dX
        sh.dMq[r][c] = r >= c ? sh.dMq[r][c] : 0.f;
    }
    __syncthreads();
    {   // dL = -X^T dX X^T, strictly lower part: first P = X^T dX
        const int r = i16, c = j16;
        float acc = 0.f;
        for (int m = 0; m < 16; ++m) acc += sh.X[m][r] * sh.T1[m][c];
        sh.P[r][c] = acc;
    }
    __syncthreads();
    {
        const int r = i16, c = j16;
        float acc = 0.f;
        for (int m = 0; m < 16; ++m) acc += sh.P[r][m] * sh.X[c][m];
        sh.dL[r][c] = r > c ? -acc : 0.f;
    }
    __syncthreads();
    if (tid < 16) {            // dbeta (rows of L) and dG = diag(beta) dL into T1
        float acc = 0.f;
        for (int c = 0; c < 16; ++c) acc += sh.dL[tid][c] * sh.G[tid][c];
        sh.dbeta[tid] += acc;
    }
    {
        const int r = i16, c = j16;
        sh.T1[r][c] = sh.beta[r] * sh.dL[r][c];
    }
    __syncthreads();

    // ---- per (token, key dim): dk, dq and dGam; dKD = A^T dW
    // dGam is written over dQD: entry (t, d) of dQD is read only by the thread that owns (t, d)
    float *dq_out = p.G > 1 ? b.part_q : b.dq;
    float *dk_out = p.G > 1 ? b.part_k : b.dk;
    const int qk_heads = p.G > 1 ? p.HV : p.H, qk_head = p.G > 1 ? j : h;
    for (int idx = tid; idx < 16 * K; idx += 256) {
        const int t = idx / K, d = idx % K;
        float dkd = 0.f;
        for (int m = 0; m < 16; ++m) dkd += sh.A[m][t] * sh.dw[m][d];
        const float gt = sh.gm[t][d], et = __expf(gt);
        const float kt = sh.k[t][d], qt = sh.q[t][d];
        const float ert = __expf(sh.gm[15][d] - gt);
        float dk = dkd * et + sh.dkr[t][d] * ert;
        float dq = sc * sh.dqd[t][d] * et;
        float dgam = dkd * kt * et + sh.dqd[t][d] * sc * qt * et - sh.dkr[t][d] * kt * ert;
        for (int m = 0; m < 16; ++m) {
            const float km = sh.k[m][d], qm = sh.q[m][d], gmm = sh.gm[m][d];
            if (m < t) {        // t is the row i of G, Mqk: e^{Gam_t - Gam_m}
                const float e = __expf(gt - gmm);
                const float wg = sh.T1[t][m] * km * e, wq = sh.dMq[t][m] * sc * km * e;
                dk += wg;
                dq += wq;
                dgam += kt * wg + qt * wq;
            }
            if (m > t) {        // t is the column j: e^{Gam_m - Gam_t}
                const float e = __expf(gmm - gt);
                const float wg = sh.T1[m][t] * km * e, wq = sh.dMq[m][t] * sc * qm * e;
                dk += wg + wq;
                dgam -= kt * (wg + wq);
            }
            if (m == t) {       // diagonal of Mqk: q_t k_t, no decay
                const float wq = sh.dMq[t][t] * sc;
                dq += wq * kt;
                dk += wq * qt;
            }
        }
        if (t < nvalid) {
            const int64_t tok = bos + t;
            dq_out[(tok * qk_heads + qk_head) * K + d] = dq;
            dk_out[(tok * qk_heads + qk_head) * K + d] = dk;
        }
        sh.dqd[t][d] = dgam;
    }
    __syncthreads();
    // ---- dgam = dE E + sum_t dKR KR; dg_tau = sum_{t >= tau} dGam_t + dgam; dbeta out
    for (int d = tid; d < K; d += 256) {
        float dgam = sh.dE[d] * sh.E[d];
        for (int t = 0; t < 16; ++t) dgam += sh.dkr[t][d] * sh.kr[t][d];
        float acc = dgam;
        for (int t = 15; t >= 0; --t) {
            acc += sh.dqd[t][d];
            if (t < nvalid) b.dg[((bos + t) * p.HV + j) * K + d] = acc;
        }
    }
    if (tid < nvalid) b.dbeta[(bos + tid) * p.HV + j] = sh.dbeta[tid];
}

// dq, dk of q/k head h = sum of the partials of its G value heads (fixed order: deterministic)
template <int K>
__global__ void bwd_group_sum_kernel(BwdParams b)
{
    const int64_t n = b.f.seq.T_total * b.f.H * K;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tok = i / ((int64_t)b.f.H * K);
        const int h = (int)((i / K) % b.f.H), d = (int)(i % K);
        float aq = 0.f, ak = 0.f;
        for (int jj = 0; jj < b.f.G; ++jj) {
            const int64_t o = (tok * b.f.HV + h * b.f.G + jj) * K + d;
            aq += b.part_q[o];
            ak += b.part_k[o];
        }
        b.dq[i] = aq;
        b.dk[i] = ak;
    }
}

}  // namespace

template <int K, int V>
hipError_t launch_backward(const BwdParams &b, bool in_bf16, hipStream_t st)
{
    const FwdParams &p = b.f;
    hipError_t e;
    if (p.seq.T_total > 0 && (e = launch_prepare_f32<K, V>(p, st, in_bf16)) != hipSuccess)
        return e;
    const unsigned units = (unsigned)(p.seq.N * p.HV);
    if (units == 0) return hipSuccess;
    bwd_states_kernel<K, V><<<dim3(units), dim3(V), 0, st>>>(b);
    if (in_bf16)
        bwd_chain_kernel<K, V, uint16_t><<<dim3(units), dim3(V), 0, st>>>(b);
    else
        bwd_chain_kernel<K, V, float><<<dim3(units), dim3(V), 0, st>>>(b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.seq.T_total == 0) return hipSuccess;
    dim3 grid(p.seq.n_slots, p.HV);
    if (in_bf16)
        bwd_local_kernel<K, V, uint16_t><<<grid, dim3(256), 0, st>>>(b);
    else
        bwd_local_kernel<K, V, float><<<grid, dim3(256), 0, st>>>(b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.G > 1) bwd_group_sum_kernel<K><<<dim3(1024), dim3(256), 0, st>>>(b);
    return hipGetLastError();
}

#define KDA_INST(K, V) \
    template hipError_t launch_backward<K, V>(const BwdParams &, bool, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
