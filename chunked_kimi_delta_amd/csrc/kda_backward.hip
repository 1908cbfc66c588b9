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
//   prepare_f32 (kda_prepare.hip)  the chunk records in fp32: W, QD, KR, U, Mqk, E and, for the
//                                  local gradients, the inverse X and the Gram G (WsF32B)
//   bwd_chains_kernel              S at the start and Lam at the end of every chunk, and dh0
//   bwd_local_kernel               per (chunk, value head): dv, dg, dbeta and dq, dk
//   bwd_qk_finalize_kernel         dq, dk summed over the value heads of a q/k head (G > 1)
//                                  and carried through the q/k L2 norm (when it is on)
//   bwd_param_kernel               dA_log, dt_bias: per-chunk partials summed (gate on)
// With the pre-stage on, the kernels read raw inputs and apply it on load (prepare_f32 and the
// local kernel), and the gradients leave through its reverse mode: dbeta times
// sigma (1 - sigma), dg times the gate's slope (with dA_log and dt_bias summed over all tokens),
// dq and dk through the L2 norm, dx = r dy - r^3 x (x . dy) (the backward of the pre-stage in
// the C++ reference of "手撕KDA" section 2.1).
#include "kda_chain_f32.h"

namespace kda {

namespace {

// Both chains of the backward in one launch (they are independent): per unit, sub-slices
// 2i (states, recorded at every chunk start) and 2i + 1 (the state gradient, recorded at every
// chunk end, then dh0) of the 16-column slice i, all on one XCD (kda_chain_f32.h).
template <int K, int V>
__global__ __launch_bounds__(64 * CHAIN_WAVES) void bwd_chains_kernel(BwdParams b)
{
    constexpr int NSL = V / 16;
    int unit, sub;
    if (!state_unit(blockIdx.x, 2 * NSL, b.f.seq.N * b.f.HV, &unit, &sub)) return;
    unit = longest_first(b.f.seq, b.f.HV, unit);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n0 = (sub >> 1) * 16;
    constexpr int RB = WsF32B<K, V>::BYTES;
    if (sub & 1)
        chain_run<K, V, CHAIN_GRADS>(b.f, unit, n0, wave, lane, b.dht, b.ck_L, b.dh0, nullptr,
                                     RB);
    else
        chain_run<K, V, CHAIN_STATES>(b.f, unit, n0, wave, lane, b.f.h0, b.ck_S, nullptr,
                                      nullptr, RB);
}

// One block (4 waves) per (chunk slot, value head): back-propagate O and S_next (through
// delta, U, W, A, the inverse, L, Mqk and the decay factors) to the chunk's tokens, reading X, G,
// Mqk, W and KR from the chunk's record. Products are formed from exponent differences (every
// factor e^{Gam_i - Gam_j}, i >= j, and e^{gam - Gam} is at most 1).
// The contractions over V run on the fp32 matrix cores, one 16-column block of V at a time,
// with the K rows split over the waves as in the chains (wave w owns the row tiles
// w * K/64 ...): per block
//     delta = A v - W S,  dDelta = Mqk^T dO + KR Lam           (partials summed through LDS)
//     dQD += dO S^T,  dKR += delta Lam^T,  dW -= dDelta S^T     (the wave's own K tiles)
//     dE += rowsum(Lam . S),  dMqk += dO delta^T,  dA += dDelta v^T,  dv = A^T dDelta
// S and Lam are read as the chains recorded them (C-layout tiles, one non-temporal 16-byte
// load per tile and lane) and are needed in two register layouts: C-layout (the B operand of a
// product over K) and its transpose (the B operand of a product over V), made through a
// wave-private LDS tile. dKD = A^T dW is one product per tile of the V loop's accumulators;
// the rest of the chunk's algebra (16 x 16 and 16 x K) is scalar, the pairs of G and Mqk in
// one pass per key dim.
template <int K, int V>
struct alignas(16) LocalShare {
    float q[16][K + 1], k[16][K + 1], gm[16][K + 1];   // q, k, Gam (cumsum of g)
    float kd[16][K + 1];                               // KD = k e^Gam
    union alignas(16) {                                // two phases, one region
        struct {                                       // the V loop
            float part[2][2][CHAIN_WAVES][16][20];     // V-block partials of delta, dDelta
            float tr[CHAIN_WAVES][16][17];             // per-wave tile transposes
        };
        struct {                                       // after it
            float dqd[16][K + 1], dkr[16][K + 1];
            union {
                struct { float dw[16][K + 1], dkd[16][K + 1]; };
                float red[256 / K][16][K];             // per-key-dim pass: partial sums
            };
        };
    };
    float G[16][17], Mq[16][17], X[16][17], A[16][17], P[16][17], T1[16][17];
    float dA[16][17], dMq[16][17], dL[16][17];
    float beta[16], dbeta[16], E[K], dE[K];
};

// A 16 x 16 fp32 tile held in C-layout (lane: rows 4g + i, column r) returned in the transposed
// arrangement (lane: row r, columns 4g + i), through a wave-private LDS tile. LDS operations of
// one wave complete in order, so no barrier is needed; the scheduling barriers keep the
// compiler from moving the accesses of one use across those of the next.
__device__ __forceinline__ f32x4 tile_transpose(float (&t)[16][17], f32x4 c, int r, int g)
{
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) t[4 * g + i][r] = c[i];
    __builtin_amdgcn_wave_barrier();
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = t[r][4 * g + i];
    __builtin_amdgcn_wave_barrier();
    return o;
}

// four consecutive values of an io-dtype row as fp32
__device__ __forceinline__ f32x4 ld4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ f32x4 ld4(const uint16_t *p) {
    const uint2 raw = *(const uint2 *)p;
    float o[4];
    unpack_bf16x4(raw, o);
    return f32x4{o[0], o[1], o[2], o[3]};
}

// Operands of one V block for one wave (loaded one block ahead; used as loaded, rows past the
// chunk's end are zeroed at use).
template <int K>
struct BlockOps {
    static constexpr int TPW = K / 16 / CHAIN_WAVES;
    f32x4 sc[TPW], lc[TPW];                     // S, Lam tiles (C-layout)
    f32x4 doc, doa, vc, va;                     // dO, v: C-layout (rows 4g+i) and row r
};

template <int K, int V, typename T>
__global__ __launch_bounds__(256) void bwd_local_kernel(BwdParams b)
{
    const FwdParams &p = b.f;
    constexpr int TPW = BlockOps<K>::TPW, NB = V / 16;
    __shared__ LocalShare<K, V> sh;
    const int tid = threadIdx.x;
    const int slot = blockIdx.x, j = blockIdx.y, h = j / p.G;
    int s;
    int64_t bos;
    int nvalid;
    const bool gated = p.pre.gate != 0;
    if (!locate_slot(p.seq, slot, &s, &bos, &nvalid)) {
        if (gated) {               // slots without a chunk contribute nothing to the sums
            const size_t ps = (size_t)j * p.seq.n_slots + slot;
            for (int d = tid; d < K; d += 256) b.part_dt[ps * K + d] = 0.f;
            if (tid == 0) b.part_A[ps] = 0.f;
        }
        return;
    }
    const size_t gslot = (size_t)j * p.seq.n_slots + slot;
    const float sc = p.scale;
    const T *q = (const T *)p.q, *k = (const T *)p.k, *v = (const T *)p.v;
    const T *g = (const T *)p.g, *bt = (const T *)p.beta, *dout = (const T *)b.d_o;
    const float aexp = gated ? __builtin_amdgcn_exp2f(p.pre.A_log[j] * LOG2E) : 0.f;
    auto dtb = [&](int d) { return gated && p.pre.dt_bias ? p.pre.dt_bias[j * K + d] : 0.f; };

    // ---- inputs of the chunk (rows past the end are zero), pre-stage, the cumsum of g
    // Every load is issued before any value is used: rows past the sequence end read its last
    // row (nvalid >= 1) and are zeroed on the way to LDS (a load under a branch, or used next
    // to it, made the compiler wait for each load in turn).
    {
        constexpr int NE = 16 * K / 256;
        T rq[NE], rk[NE], rg[NE], rb;
        float rdt[NE];
        const float *dtp = gated && p.pre.dt_bias ? p.pre.dt_bias + (size_t)j * K : nullptr;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int idx = tid + 256 * e, r = idx / K, d = idx % K;
            const int64_t t = bos + (r < nvalid ? r : nvalid - 1);
            rq[e] = q[(t * p.H + h) * K + d];
            rk[e] = k[(t * p.H + h) * K + d];
            rg[e] = g[(t * p.HV + j) * K + d];
            rdt[e] = dtp ? dtp[d] : 0.f;
        }
        rb = bt[(bos + ((tid & 15) < nvalid ? (tid & 15) : nvalid - 1)) * p.HV + j];
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int idx = tid + 256 * e, r = idx / K, d = idx % K;
            const bool ok = r < nvalid;
            sh.q[r][d] = ok ? to_f32(rq[e]) : 0.f;
            sh.k[r][d] = ok ? to_f32(rk[e]) : 0.f;
            float gv = ok ? to_f32(rg[e]) : 0.f;
            if (gated && ok) gv = gate_activation(p.pre, gv + rdt[e], aexp);
            sh.gm[r][d] = gv;
        }
        if (tid < 16) {
            float bv = tid < nvalid ? to_f32(rb) : 0.f;
            if (p.pre.beta_sigmoid && tid < nvalid) bv = sigmoid_f(bv);
            sh.beta[tid] = bv;
            sh.dbeta[tid] = 0.f;
        }
    }
    __syncthreads();
    if (p.pre.qk_l2norm) {         // 16 threads per token row: partial sums, xor reduction
        const int rr = tid >> 4, l = tid & 15;
        float a = 0.f, c = 0.f;
        for (int d = l; d < K; d += 16) {
            a += sh.q[rr][d] * sh.q[rr][d];
            c += sh.k[rr][d] * sh.k[rr][d];
        }
        for (int m = 1; m < 16; m <<= 1) {
            a += __shfl_xor(a, m);
            c += __shfl_xor(c, m);
        }
        const float fq = l2norm_factor(a), fk = l2norm_factor(c);
        for (int d = l; d < K; d += 16) {
            sh.q[rr][d] *= fq;
            sh.k[rr][d] *= fk;
        }
        __syncthreads();
    }
    for (int d = tid; d < K; d += 256) {
        float acc = 0.f;
        for (int r = 0; r < 16; ++r) { acc += sh.gm[r][d]; sh.gm[r][d] = acc; }
        sh.E[d] = __expf(acc);
    }
    // ---- the chunk's inverse X, Gram G and Mqk from its record (the prepare kernel's)
    using WSB = WsF32B<K, V>;
    const float *rec = (const float *)(p.ws + gslot * (size_t)WSB::BYTES);
    const int i16 = tid >> 4, j16 = tid & 15;
    sh.X[i16][j16] = rec[WSB::XM / 4 + tid];
    sh.G[i16][j16] = rec[WSB::GM / 4 + tid];
    sh.Mq[i16][j16] = rec[WSB::MQK / 4 + tid];
    __syncthreads();
    sh.A[i16][j16] = sh.X[i16][j16] * sh.beta[j16];
    for (int idx = tid; idx < 16 * K; idx += 256) {
        const int t = idx / K, d = idx % K;
        sh.kd[t][d] = sh.k[t][d] * __expf(sh.gm[t][d]);
    }
    __syncthreads();

    // ---- the V blocks on the matrix cores
    const int wave = tid >> 6, lane = tid & 63, r = lane & 15, gq = lane >> 4;
    f32x4 Wa[TPW], KRa[TPW], Aa, At, Mqt;        // loop-invariant A operands
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int k0 = (wave * TPW + x) * 16;
        Wa[x] = *(const f32x4 *)(rec + WSB::W / 4 + r * K + k0 + 4 * gq);
        KRa[x] = *(const f32x4 *)(rec + WSB::KR / 4 + r * K + k0 + 4 * gq);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        Aa[i] = sh.A[r][4 * gq + i];
        At[i] = sh.A[4 * gq + i][r];
        Mqt[i] = sh.Mq[4 * gq + i][r];
    }
    const float *cS = b.ck_S + gslot * (size_t)K * V + wave * TPW * 256 + lane * 4;
    const float *cL = b.ck_L + gslot * (size_t)K * V + wave * TPW * 256 + lane * 4;
    const int rc = r < nvalid ? r : nvalid - 1;               // clamped rows: loads stay inside
    int rq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rq[i] = 4 * gq + i < nvalid ? 4 * gq + i : nvalid - 1;
    auto load = [&](BlockOps<K> &o, int nb) {
        const int n0 = nb * 16;
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            // read once: non-temporal, so they do not evict the chunk records from L2
            const size_t to = ((size_t)nb * (K / 16) + x) * 256;
            o.sc[x] = __builtin_nontemporal_load((const f32x4 *)(cS + to));
            o.lc[x] = __builtin_nontemporal_load((const f32x4 *)(cL + to));
        }
        o.doc = *(const f32x4 *)(rec + WSB::DO / 4 + (nb * 64 + lane) * 4);   // dO, C-layout
#pragma unroll
        for (int i = 0; i < 4; ++i) o.vc[i] = ldx(v, ((bos + rq[i]) * p.HV + j) * V + n0 + r);
        o.doa = ld4(dout + ((bos + rc) * p.HV + j) * V + n0 + 4 * gq);
        o.va = ld4(v + ((bos + rc) * p.HV + j) * V + n0 + 4 * gq);
    };
    f32x4 aq[TPW], ar[TPW], aw[TPW], aMq = zero4(), aA = zero4();
    float aE[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) { aq[x] = ar[x] = aw[x] = zero4(); aE[x] = 0.f; }
    auto step = [&](const BlockOps<K> &o, int nb) {
        const int n0 = nb * 16;
        f32x4 doc = o.doc, doa = o.doa, vc = o.vc, va = o.va;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool okq = 4 * gq + i < nvalid;
            doc[i] = okq ? doc[i] : 0.f;
            vc[i] = okq ? vc[i] : 0.f;
            doa[i] = r < nvalid ? doa[i] : 0.f;
            va[i] = r < nvalid ? va[i] : 0.f;
        }
        // transposed layouts of the S and Lam tiles: element (r, 4g + i) of the tile
        f32x4 sa[TPW], la[TPW];
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            sa[x] = tile_transpose(sh.tr[wave], o.sc[x], r, gq);
            la[x] = tile_transpose(sh.tr[wave], o.lc[x], r, gq);
        }
        f32x4 pd = zero4(), pk = zero4();
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            pd = mm16_f32(Wa[x], o.sc[x], pd);
            pk = mm16_f32(KRa[x], o.lc[x], pk);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) pd[i] = -pd[i];
        if (wave == 0) {
            pd = mm16_f32(Aa, vc, pd);                     // + A v
            pk = mm16_f32(Mqt, doc, pk);                   // + Mqk^T dO
        }
        const int par = nb & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sh.part[par][0][wave][4 * gq + i][r] = pd[i];
            sh.part[par][1][wave][4 * gq + i][r] = pk[i];
        }
        lds_barrier();
        f32x4 ddc = zero4(), dtr = zero4(), ddtr = zero4();
#pragma unroll
        for (int w = 0; w < CHAIN_WAVES; ++w) {
            const f32x4 t0 = *(const f32x4 *)&sh.part[par][0][w][r][4 * gq];
            const f32x4 t1 = *(const f32x4 *)&sh.part[par][1][w][r][4 * gq];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ddc[i] += sh.part[par][1][w][4 * gq + i][r];
                dtr[i] += t0[i];
                ddtr[i] += t1[i];
            }
        }
        // dtr, ddtr: delta, dDelta in the transposed layout (row r); ddc: dDelta in C-layout
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            aq[x] = mm16_f32(doa, sa[x], aq[x]);            // dQD += dO S^T
            ar[x] = mm16_f32(dtr, la[x], ar[x]);            // dKR += delta Lam^T
            aw[x] = mm16_f32(ddtr, sa[x], aw[x]);           // dW  -= dDelta S^T (sign later)
#pragma unroll
            for (int i = 0; i < 4; ++i) aE[x] += sa[x][i] * la[x][i];
        }
        if (wave == 0) aMq = mm16_f32(doa, dtr, aMq);       // dMqk += dO delta^T
        if (wave == 1) aA = mm16_f32(ddtr, va, aA);         // dA += dDelta v^T
        if (wave == 2) {                                    // dv = A^T dDelta
            const f32x4 dv = mm16_f32(At, ddc, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * gq + i < nvalid)
                    b.dv[((bos + 4 * gq + i) * p.HV + j) * V + n0 + r] = dv[i];
        }
    };
    {
        BlockOps<K> o0, o1;
        load(o0, 0);
        for (int nb = 0; nb < NB; nb += 2) {
            load(o1, nb + 1 < NB ? nb + 1 : nb);
            step(o0, nb);
            if (nb + 1 >= NB) break;
            load(o0, nb + 2 < NB ? nb + 2 : nb + 1);
            step(o1, nb + 1);
        }
    }
    __syncthreads();                                        // partials done: reuse as dQD...
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int k0 = (wave * TPW + x) * 16;
        f32x4 nw;
#pragma unroll
        for (int i = 0; i < 4; ++i) nw[i] = -aw[x][i];
        const f32x4 dkd = mm16_f32(At, nw, zero4());          // dKD = A^T dW
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sh.dqd[4 * gq + i][k0 + r] = aq[x][i];
            sh.dkr[4 * gq + i][k0 + r] = ar[x][i];
            sh.dw[4 * gq + i][k0 + r] = nw[i];
            sh.dkd[4 * gq + i][k0 + r] = dkd[i];
        }
        const float e = sum_lane_groups(aE[x]);
        if (gq == 0) sh.dE[k0 + r] = e;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (wave == 0) sh.dMq[4 * gq + i][r] = aMq[i];
        if (wave == 1) sh.dA[4 * gq + i][r] = aA[i];
    }
    __syncthreads();

    // ---- dA += dW KD^T; dbeta (columns of A); dX = dA diag(beta)
    {
        const int r = i16, c = j16;
        float acc = 0.f;
        for (int d = 0; d < K; ++d) acc += sh.dw[r][d] * sh.kd[c][d];
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

    // ---- per key dim d: dk, dq and dGam of the 16 tokens, from the chunk-level gradients
    // (dQD, dKR, dKD) and the pairs (i > j) of G and Mqk, each pair's e^{Gam_i - Gam_j}
    // evaluated once. The P = 256 / K waves-groups of a key dim share the rows i between them
    // (a wave-uniform split balanced to 120 / P pairs each) and their partial sums are added
    // through LDS afterwards; dGam is then written over dQD.
    {
        constexpr int P = 256 / K;
        const int d = tid % K, pp = tid / K;              // pp is uniform within a wave
        float kk[16], qq[16], gg[16], ak[16], aqv[16], ag[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            kk[t] = sh.k[t][d];
            qq[t] = sh.q[t][d];
            gg[t] = sh.gm[t][d];
            ak[t] = aqv[t] = ag[t] = 0.f;
        }
        // rows {15,14,1,0}, {13,12,3,2}, {11,10,5,4}, {9,8,7,6}: 30 pairs each (P = 4);
        // P = 2 joins the first two and the last two
        constexpr int own4[16] = {0, 0, 1, 1, 2, 2, 3, 3, 3, 3, 2, 2, 1, 1, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (own4[i] * P / 4 != pp) continue;
            const float ei = __expf(gg[i]), eri = __expf(gg[15] - gg[i]);
            const float dkd = sh.dkd[i][d], dkr = sh.dkr[i][d], dqd = sh.dqd[i][d];
            const float wd = sh.dMq[i][i] * sc;            // diagonal of Mqk: q_i k_i
            ak[i] += dkd * ei + dkr * eri + wd * qq[i];
            aqv[i] += sc * dqd * ei + wd * kk[i];
            ag[i] += (dkd * kk[i] + sc * dqd * qq[i]) * ei - dkr * kk[i] * eri;
#pragma unroll
            for (int jx = 0; jx < i; ++jx) {
                const float e = __expf(gg[i] - gg[jx]);
                const float w1 = sh.T1[i][jx] * e, w2 = sh.dMq[i][jx] * sc * e;
                ak[i] += w1 * kk[jx];
                aqv[i] += w2 * kk[jx];
                const float c = w1 * kk[i] + w2 * qq[i];
                ak[jx] += c;
                const float gx = c * kk[jx];
                ag[i] += gx;
                ag[jx] -= gx;
            }
        }
        const bool via_part = p.G > 1 || p.pre.qk_l2norm;
        float *dq_out = via_part ? b.part_q : b.dq;
        float *dk_out = via_part ? b.part_k : b.dk;
        const int qk_heads = via_part ? p.HV : p.H, qk_head = via_part ? j : h;
#pragma unroll
        for (int which = 0; which < 3; ++which) {         // dk, dq, dGam in turn
            __syncthreads();
#pragma unroll
            for (int t = 0; t < 16; ++t)
                sh.red[pp][t][d] = which == 0 ? ak[t] : which == 1 ? aqv[t] : ag[t];
            __syncthreads();
            for (int idx = tid; idx < 16 * K; idx += 256) {
                const int t = idx / K, dd = idx % K;
                float v2 = 0.f;
#pragma unroll
                for (int q2 = 0; q2 < P; ++q2) v2 += sh.red[q2][t][dd];
                if (which == 2) {
                    sh.dqd[t][dd] = v2;
                } else if (t < nvalid) {
                    float *out = which == 0 ? dk_out : dq_out;
                    out[((bos + t) * qk_heads + qk_head) * K + dd] = v2;
                }
            }
        }
    }
    __syncthreads();
    // ---- dgam = dE E + sum_t dKR KR; dg_tau = sum_{t >= tau} dGam_t + dgam; through the
    // gate (raw g reloaded): dg_raw = dg * slope, and this chunk's share of dA_log, ddt_bias
    float gA = 0.f;
    for (int d = tid; d < K; d += 256) {
        float dgam = sh.dE[d] * sh.E[d];
        for (int t = 0; t < 16; ++t) dgam += sh.dkr[t][d] * rec[WSB::KR / 4 + t * K + d];
        float acc = dgam, adt = 0.f;
        for (int t = 15; t >= 0; --t) {
            acc += sh.dqd[t][d];
            if (t < nvalid) {
                const int64_t o = ((bos + t) * p.HV + j) * K + d;
                float dgo = acc;
                if (gated) {
                    const float x = ldx(g, o) + dtb(d);
                    float slope, dfa;                  // dg/dx and dg/dA_log
                    if (p.pre.gate == 1) {
                        slope = -aexp * sigmoid_f(x);
                        dfa = -aexp * softplus_f(x);
                    } else {
                        const float sg = sigmoid_f(aexp * x);
                        slope = p.pre.lower_bound * sg * (1.f - sg) * aexp;
                        dfa = slope * x;
                    }
                    dgo = acc * slope;
                    adt += dgo;
                    gA += acc * dfa;
                }
                b.dg[o] = dgo;
            }
        }
        if (gated) b.part_dt[gslot * K + d] = adt;
    }
    if (gated) {                   // block sum of gA (the threads d < K carry a share)
        gA = wave_sum(gA);
        __syncthreads();
        if ((tid & 63) == 0) sh.dA[0][tid >> 6] = gA;
        __syncthreads();
        if (tid == 0) b.part_A[gslot] = sh.dA[0][0] + sh.dA[0][1] + sh.dA[0][2] + sh.dA[0][3];
    }
    if (tid < nvalid) {
        float db = sh.dbeta[tid];
        if (p.pre.beta_sigmoid) {
            const float sg = sigmoid_f(ldx(bt, (bos + tid) * p.HV + j));
            db *= sg * (1.f - sg);
        }
        b.dbeta[(bos + tid) * p.HV + j] = db;
    }
}

// dq, dk of q/k head h: the partials of its G value heads summed in a fixed order
// (deterministic), then, with the L2 norm on, carried through it: with r = (|x|^2 + eps)^-1/2
// and y = x r for the raw row x, dx = r (dy - y (y . dy)). One wave per (token, q/k head) row.
template <int K, typename T>
__global__ __launch_bounds__(256) void bwd_qk_finalize_kernel(BwdParams b)
{
    const FwdParams &p = b.f;
    constexpr int PL = K / 64;                      // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t rows = p.seq.T_total * p.H;
    const int64_t wid = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t row = wid; row < rows; row += nw) {
        const int64_t tok = row / p.H;
        const int h = (int)(row % p.H);
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const float *part = which ? b.part_k : b.part_q;
            float dy[PL];
#pragma unroll
            for (int e = 0; e < PL; ++e) {
                float acc = 0.f;
#pragma unroll 4
                for (int jj = 0; jj < p.G; ++jj)
                    acc += part[(tok * p.HV + h * p.G + jj) * K + lane + 64 * e];
                dy[e] = acc;
            }
            if (p.pre.qk_l2norm) {
                const T *x = (const T *)(which ? p.k : p.q) + (tok * p.H + h) * K;
                float xv[PL], ss = 0.f;
#pragma unroll
                for (int e = 0; e < PL; ++e) {
                    xv[e] = ldx(x, lane + 64 * e);
                    ss += xv[e] * xv[e];
                }
                const float r = l2norm_factor(wave_sum(ss));
                float yd = 0.f;
#pragma unroll
                for (int e = 0; e < PL; ++e) yd += xv[e] * r * dy[e];
                yd = wave_sum(yd);
#pragma unroll
                for (int e = 0; e < PL; ++e) dy[e] = r * (dy[e] - xv[e] * r * yd);
            }
            float *out = (which ? b.dk : b.dq) + (tok * p.H + h) * K;
#pragma unroll
            for (int e = 0; e < PL; ++e) out[lane + 64 * e] = dy[e];
        }
    }
}

// dA_log[j] and ddt_bias[j][:]: per-chunk partials summed over the slots in a fixed order.
template <int K>
__global__ __launch_bounds__(256) void bwd_param_kernel(BwdParams b)
{
    const FwdParams &p = b.f;
    __shared__ float red[256];
    const int j = blockIdx.x, tid = threadIdx.x;
    const size_t s0 = (size_t)j * p.seq.n_slots;
    if (p.seq.T_total == 0) {      // no tokens: no chunk partials were written
        for (int d = tid; d < K; d += 256)
            if (b.ddt_bias) b.ddt_bias[j * K + d] = 0.f;
        if (tid == 0) b.dA_log[j] = 0.f;
        return;
    }
    if (b.ddt_bias) {
        for (int d = tid; d < K; d += 256) {
            float acc = 0.f;
            for (int sl = 0; sl < p.seq.n_slots; ++sl) acc += b.part_dt[(s0 + sl) * K + d];
            b.ddt_bias[j * K + d] = acc;
        }
    }
    float acc = 0.f;
    for (int sl = tid; sl < p.seq.n_slots; sl += 256) acc += b.part_A[s0 + sl];
    red[tid] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) b.dA_log[j] = red[0];
}

}  // namespace

template <int K, int V>
hipError_t launch_backward(const BwdParams &b, bool in_bf16, hipStream_t st)
{
    const FwdParams &p = b.f;
    hipError_t e;
    if (p.seq.T_total > 0 &&
        (e = launch_prepare_f32<K, V>(p, st, in_bf16, true)) != hipSuccess)
        return e;
    const int64_t units = (int64_t)p.seq.N * p.HV;
    if (units == 0) return hipSuccess;
    const dim3 cgrid((unsigned)((units + 7) / 8 * 8 * 2 * (V / 16)));
    bwd_chains_kernel<K, V><<<cgrid, dim3(64 * CHAIN_WAVES), 0, st>>>(b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.seq.T_total > 0) {
        dim3 grid(p.seq.n_slots, p.HV);
        if (in_bf16)
            bwd_local_kernel<K, V, uint16_t><<<grid, dim3(256), 0, st>>>(b);
        else
            bwd_local_kernel<K, V, float><<<grid, dim3(256), 0, st>>>(b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (p.G > 1 || p.pre.qk_l2norm) {
            // one wave per (token, q/k head) row up to 2^20 waves (the loads of a row are
            // waited for where they are used, so the latency is covered by other waves)
            const int64_t rows = p.seq.T_total * p.H;
            const unsigned fg = (unsigned)((rows + 3) / 4 < (1 << 18) ? (rows + 3) / 4 : (1 << 18));
            if (in_bf16)
                bwd_qk_finalize_kernel<K, uint16_t><<<dim3(fg), dim3(256), 0, st>>>(b);
            else
                bwd_qk_finalize_kernel<K, float><<<dim3(fg), dim3(256), 0, st>>>(b);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (p.pre.gate) bwd_param_kernel<K><<<dim3(p.HV), dim3(256), 0, st>>>(b);
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
