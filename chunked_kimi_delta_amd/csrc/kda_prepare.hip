// kda_prepare.hip -- stage 1 of the chunked KDA forward: everything that depends only on one
// 16-token chunk of one value head, computed independently for every (chunk, value head).
//
// For a chunk with in-chunk token index i (rows past the end of the sequence are zero with
// g = 0, "KDA源码剖析之FlashKDA（上）" part 7) the kernel forms
//     Gam_i = sum_{tau <= i} g_tau      gam = Gam_15                     (part 7: cumsum)
//     L     = beta_row * strict_tril(kd . ki^T),  Mqk = tril(qd' . ki^T) (parts 9-11)
//     A     = (I + L)^{-1} diag(beta)  by the Neumann doubling product   (part 12)
//     w = A (k exp(Gam)),  u = A v,  qd = scale q exp(Gam),  kr = k exp(gam - Gam), exp(gam)
// which is the per-chunk half of naive_chunk_kda ("手撕KDA" section 1) and of the v8 prepare
// kernel of "手撕KDA" section 5 (w and u formed in stage 1).
//
// gfx950 design (bf16 io). One wave64 per (chunk, value head); no LDS at all:
//  * q, k, g, v are loaded in TPL (8-byte loads, lane = token row) and upcast to fp32.
//  * The cumsum over the 16 tokens is a DPP row scan (the 16 lanes of a DPP row are the 16
//    tokens), in log2 units so every exponential is one v_exp_f32.
//  * The decayed Gram matrices use factors centred on token 7 (kd' = k 2^(G - G7), ki' = k
//    2^(G7 - G)): products keep the exact exponent difference while each factor spans only
//    half the chunk's decay range. The factors are split hi + lo in bf16 and multiplied in
//    three 16x16x32 MFMA passes (hi.hi + hi.lo + lo.hi), about 16 mantissa bits.
//  * The Neumann product runs on the fp32 matrix core entirely in registers, using C(X) ==
//    A-layout of X^T so that every power is formed in both orientations directly (no
//    transposes through memory); the "+ INV" of each doubling step is the accumulator.
//  * k exp(Gam), v and kr are moved from TPL to the column-per-lane layout the token-axis
//    products need by an MFMA against the identity (exact for bf16/fp16 inputs).
//  * Outputs go to the workspace as fp16 in the state kernel's lane order (kda_internal.h).
#include "kda_internal.h"

namespace kda {

template <int K, int V>
__global__ __launch_bounds__(64) void prepare_bf16_kernel(FwdParams p)
{
    constexpr int NK = K / 16;     // 16-wide key-dim tiles
    constexpr int NV = V / 16;     // 16-wide value-dim tiles
    constexpr int NS = K / 32;     // 16x16x32 steps over the key dims
    using WS = WsBf16<K, V>;

    const int lane = threadIdx.x;
    const int grp = lane >> 4;
    const int r = lane & 15;       // TPL: token row. C-layout: column index.
    const int slot = blockIdx.x;
    const int j = blockIdx.y;
    const int h = j / p.G;

    int s;
    int64_t bos;
    int nvalid;
    if (!locate_slot(p.seq, slot, &s, &bos, &nvalid)) return;
    const bool live = r < nvalid;
    const int64_t tok = bos + r;

    // ---------------------------------------------------------------- loads (TPL)
    const bool gated = p.pre.gate != 0;             // pre-stage gate parameters
    float aexp = 0.f;
    f32x4 dtv[NK];
#pragma unroll
    for (int c = 0; c < NK; ++c) dtv[c] = zero4();
    if (gated) {
        aexp = __builtin_amdgcn_exp2f(p.pre.A_log[j] * LOG2E);
        if (p.pre.dt_bias) {
#pragma unroll
            for (int c = 0; c < NK; ++c)
                dtv[c] = *(const f32x4 *)(p.pre.dt_bias + (size_t)j * K + 16 * c + 4 * grp);
        }
    }
    float qf[NK][4], kf[NK][4], gl[NK][4];
    uint2 vraw[NV];
    float beta_r = 0.f;
#pragma unroll
    for (int c = 0; c < NK; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) { qf[c][i] = 0.f; kf[c][i] = 0.f; gl[c][i] = 0.f; }
#pragma unroll
    for (int c = 0; c < NV; ++c) vraw[c] = make_uint2(0u, 0u);
    if (live) {
        const uint16_t *qp = (const uint16_t *)p.q + ((tok * p.H + h) * K + 4 * grp);
        const uint16_t *kp = (const uint16_t *)p.k + ((tok * p.H + h) * K + 4 * grp);
        const uint16_t *gp = (const uint16_t *)p.g + ((tok * p.HV + j) * K + 4 * grp);
        const uint16_t *vp = (const uint16_t *)p.v + ((tok * p.HV + j) * V + 4 * grp);
        uint2 qr[NK], kr[NK], gr[NK];
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            qr[c] = *(const uint2 *)(qp + 16 * c);
            kr[c] = *(const uint2 *)(kp + 16 * c);
            gr[c] = *(const uint2 *)(gp + 16 * c);
        }
#pragma unroll
        for (int c = 0; c < NV; ++c) vraw[c] = *(const uint2 *)(vp + 16 * c);
        beta_r = bf16_bits_to_f32(((const uint16_t *)p.beta)[tok * p.HV + j]);
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            unpack_bf16x4(qr[c], qf[c]);
            unpack_bf16x4(kr[c], kf[c]);
            unpack_bf16x4(gr[c], gl[c]);
        }
        // pre-stage on the valid rows (padding rows keep q = k = g = beta = 0)
        if (p.pre.beta_sigmoid) beta_r = sigmoid_f(beta_r);
        if (gated) {
#pragma unroll
            for (int c = 0; c < NK; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    gl[c][i] = gate_activation(p.pre, gl[c][i] + dtv[c][i], aexp);
        }
    }
    float rq = 1.f, rk = 1.f;                       // L2-norm factors of this lane's row
    if (p.pre.qk_l2norm) {
        // L2 norm of each token's q and k row: this lane holds a quarter of row r, the three
        // other lane groups the rest
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < NK; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sq += qf[c][i] * qf[c][i];
                sk += kf[c][i] * kf[c][i];
            }
        rq = l2norm_factor(sum_lane_groups(sq));
        rk = l2norm_factor(sum_lane_groups(sk));
#pragma unroll
        for (int c = 0; c < NK; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qf[c][i] *= rq;
                kf[c][i] *= rk;
            }
    }

    // ---------------------------------------------------------------- cumsum (log2 units)
    float G2[NK][4], ref[NK][4], gam[NK][4];
#pragma unroll
    for (int c = 0; c < NK; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) G2[c][i] = row_inclusive_scan(gl[c][i] * LOG2E);
    const int lane7 = (lane & 48) | 7, lane15 = lane | 15;
#pragma unroll
    for (int c = 0; c < NK; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ref[c][i] = lane_read(G2[c][i], lane7);
            gam[c][i] = lane_read(G2[c][i], lane15);
        }

    // ---------------------------------------------------------------- decay factors
    const float sc = p.scale;
    float KD[NK][4], QD[NK][4], KRv[NK][4];
    bf16x8 kdh[NS], kdl[NS], kih[NS], kil[NS], qdh[NS], qdl[NS];
    float span = 0.f;                               // largest |exponent| of a Gram factor
#pragma unroll
    for (int c = 0; c < NK; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d1 = G2[c][i] - ref[c][i];
            span = fmaxf(span, fabsf(d1));
            const float e1 = __builtin_amdgcn_exp2f(d1);
            const float e2 = __builtin_amdgcn_exp2f(-d1);
            const float eA = __builtin_amdgcn_exp2f(G2[c][i]);
            const float eR = __builtin_amdgcn_exp2f(gam[c][i] - G2[c][i]);
            const float kk = kf[c][i], qq = sc * qf[c][i];
            KD[c][i] = kk * eA;
            QD[c][i] = qq * eA;
            KRv[c][i] = kk * eR;
            const float xd = kk * e1, xi = kk * e2, xq = qq * e1;
            const int st = c >> 1, e = (c & 1) * 4 + i;
            const __bf16 hd = (__bf16)xd, hi_ = (__bf16)xi, hq = (__bf16)xq;
            kdh[st][e] = hd; kdl[st][e] = (__bf16)(xd - (float)hd);
            kih[st][e] = hi_; kil[st][e] = (__bf16)(xi - (float)hi_);
            qdh[st][e] = hq; qdl[st][e] = (__bf16)(xq - (float)hq);
        }

    // ---------------------------------------------------------------- L and Mqk (C-layout)
    f32x4 Lacc = zero4(), Macc = zero4();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        Lacc = mfma32(kdh[st], kih[st], Lacc);
        Macc = mfma32(qdh[st], kih[st], Macc);
        Lacc = mfma32(kdh[st], kil[st], Lacc);
        Macc = mfma32(qdh[st], kil[st], Macc);
        Lacc = mfma32(kdl[st], kih[st], Lacc);
        Macc = mfma32(qdl[st], kih[st], Macc);
    }
    // Decays too strong for the centred factors (their exponents span more than
    // FACTOR_SPAN_MAX): the chunk's Gram products are formed from exact per-token decay
    // products instead (wave-uniform branch).
    if (__builtin_amdgcn_ballot_w64(span > FACTOR_SPAN_MAX) != 0) {
        const BlockRows br{(const uint16_t *)p.q + (bos * p.H + h) * K,
                           (const uint16_t *)p.k + (bos * p.H + h) * K,
                           (const uint16_t *)p.g + (bos * p.HV + j) * K,
                           (int64_t)p.H * K, (int64_t)p.HV * K, nvalid};
        exact_block_gram<K>(br, p.pre, j, aexp, rk, sc * rq, lane, Lacc, Macc);
    }
    float b4[4], Mq[4];
    f32x4 L, eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * grp + i;
        b4[i] = lane_read(beta_r, row);                 // beta of token `row` (lanes 0..15)
        L[i] = row > r ? b4[i] * Lacc[i] : 0.f;         // beta_i (kd_i . ki_j), i > j
        Mq[i] = row >= r ? Macc[i] : 0.f;               // qd_i . ki_j, i >= j
        eye[i] = row == r ? 1.f : 0.f;
    }
    const bf16x4 Ib = to_bf16x4(eye);
    const f16x4 Ih = to_f16x4(eye);

    // ---------------------------------------------------------------- Neumann inverse
    // M = L^T. INV accumulates (I + M)^{-1} = (I - M)(I + M^2)(I + M^4)(I + M^8), which is
    // C(((I + L)^{-1})^T); X^T of every power comes from the swapped product. The powers of L
    // can be far larger than the inverse (keys that are nearly parallel make L^m grow like
    // binomial coefficients, up to C(14, 7) for m = 8, while (I + L)^{-1} stays O(1)), so the
    // product is evaluated on the fp32 matrix core: 16-bit operands would lose the inverse to
    // cancellation.
    const f32x4 Mf = mm16_f32(L, eye, zero4());         // C(M): transpose on the matrix core
    const f32x4 P2 = mm16_f32(L, Mf, zero4());          // C(M M)       (A16 of M == C(L))
    const f32x4 Q2 = mm16_f32(Mf, L, zero4());          // C((M^2)^T)   (A16 of L == C(M))
    const f32x4 P4 = mm16_f32(Q2, P2, zero4());         // C(M^4)
    const f32x4 Q4 = mm16_f32(P2, Q2, zero4());         // C((M^4)^T)
    const f32x4 Q8 = mm16_f32(P4, Q4, zero4());         // C((M^8)^T) == A16 of M^8
    f32x4 INV = eye - Mf;
    INV = mm16_f32(Q2, INV, INV);                       // (I + M^2)(I - M)
    INV = mm16_f32(Q4, INV, INV);                       // (I + M^4) ...
    INV = mm16_f32(Q8, INV, INV);                       // (I + M^8) ...
    float AT[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) AT[i] = INV[i] * b4[i];  // A^T = diag(beta) (I + L)^{-T}
    const bf16x4 ATb = to_bf16x4(AT);                    // B-layout of A^T == A-layout of A

    // the record, through a buffer resource: every store below is at most 8 bytes wide
    const __amdgpu_buffer_rsrc_t wr =
        buffer_rsrc(p.ws + ((size_t)j * p.seq.n_slots + slot) * (size_t)WS::BYTES, WS::BYTES);

    // ---------------------------------------------------------------- w = A KD  (TPL out)
    f16x4 wT[NK];
#pragma unroll
    for (int c = 0; c < NK; ++c) {
        const f32x4 kdC = mfma16(to_bf16x4(KD[c]), Ib, zero4());     // C(KD_c)
        wT[c] = to_f16x4(mfma16(to_bf16x4(kdC), ATb, zero4()));      // C((A KD_c)^T)
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
        bstore16<0>(wr, lane * 16, WS::W + st * 1024, cat(wT[2 * st], wT[2 * st + 1]));

    // ---------------------------------------------------------------- u = A V  (C-layout)
#pragma unroll
    for (int c = 0; c < NV; ++c) {
        const bf16x4 vA = __builtin_bit_cast(bf16x4, vraw[c]);
        const f32x4 vC = mfma16(vA, Ib, zero4());                    // C(V_c)
        bstore8<0>(wr, lane * 8, WS::U + c * 512,
                   to_f16x4(mfma16(ATb, to_bf16x4(vC), zero4())));   // C(A V_c)
    }

    // ---------------------------------------------------------------- qd (TPL), kr (C)
#pragma unroll
    for (int st = 0; st < NS; ++st)
        bstore16<0>(wr, lane * 16, WS::QD + st * 1024,
                    cat(to_f16x4(QD[2 * st]), to_f16x4(QD[2 * st + 1])));
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const f32x4 a = mfma16(to_f16x4(KRv[2 * st]), Ih, zero4());
        const f32x4 b = mfma16(to_f16x4(KRv[2 * st + 1]), Ih, zero4());
        bstore16<0>(wr, lane * 16, WS::KR + st * 1024, cat(to_f16x4(a), to_f16x4(b)));
    }

    // ---------------------------------------------------------------- Mqk (A-layout)
    bstore8<0>(wr, lane * 8, WS::MQK, to_f16x4(mfma16(to_f16x4(Mq), Ih, zero4())));

    // ---------------------------------------------------------------- exp(gam)
    if (r == 15) {
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            f32x4 e;
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(G2[c][i]);
            bstore16<0>(wr, grp * 16, WS::EG + 64 * c, e);
        }
    }
}

// =============================================================================== fp32 io
// Plain fp32 evaluation of the same chunk quantities (a correctness mode: no MFMA, the
// decayed Gram entries use exp of the exact exponent difference, the inverse is the same
// Neumann doubling product). One 256-thread block per (chunk, value head). T is the storage
// type of the inputs (float for fp32 io; uint16_t bf16 bits for the backward of bf16 io, which
// evaluates the chunks in fp32 from the same inputs).

// out = A X for A 16 x 16 (rows 16-byte aligned) and X 16 x N in LDS, out row-major 16 x N:
// each of the 256 threads takes one column and 16 N / 256 rows, so it reads its column of X
// once and A's rows as broadcast 16-byte reads (the sum over m in ascending order).
template <int N, int LD>
__device__ __forceinline__ void rows_times_a(const float (*A)[20], const float (*X)[LD],
                                             float *out, int tid)
{
    constexpr int RPT = 16 * N / 256;
    const int d = tid % N, t0 = (tid / N) * RPT;
    float x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) x[m] = X[m][d];
#pragma unroll 2
    for (int r = 0; r < RPT; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const float4 a = *(const float4 *)&A[t0 + r][4 * m4];
            acc += a.x * x[4 * m4];
            acc += a.y * x[4 * m4 + 1];
            acc += a.z * x[4 * m4 + 2];
            acc += a.w * x[4 * m4 + 3];
        }
        out[(t0 + r) * N + d] = acc;
    }
}

template <int K, int V, typename T, bool BWD>
__global__ __launch_bounds__(256) void prepare_f32_kernel(FwdParams p)
{
    using WS = WsF32<K, V>;
    constexpr int STRIDE = BWD ? WsF32B<K, V>::BYTES : WS::BYTES;
    // rows padded to a multiple of 16 bytes (4 dims at a time in the Gram loop); a padding of
    // 4 floats also puts the 16 rows of one dim in distinct banks
    __shared__ __attribute__((aligned(16))) float sq[16][K + 4], sk[16][K + 4], sG[16][K + 4];
    __shared__ float sv[16][V + 1];
    __shared__ float sb[16], sL[16][17], sI[16][17], sT[16][17];
    __shared__ __attribute__((aligned(16))) float sP[16][20];    // 16-byte rows
    const int tid = threadIdx.x;
    const int slot = blockIdx.x, j = blockIdx.y, h = j / p.G;
    int s;
    int64_t bos;
    int nvalid;
    if (!locate_slot(p.seq, slot, &s, &bos, &nvalid)) return;

    const bool gated = p.pre.gate != 0;              // pre-stage gate (valid rows only)
    const float aexp = gated ? __builtin_amdgcn_exp2f(p.pre.A_log[j] * LOG2E) : 0.f;
    // Every load is issued before any value is used, through buffer resources that end with
    // the chunk's last valid row (later rows read as zero, with no branch: a load under a
    // branch, or arithmetic next to it, made the compiler wait for each load in turn; scalar
    // bases keep one 32-bit offset register per load).
    constexpr int NE = 16 * K / 256, NEV = 16 * V / 256;   // elements per thread
    constexpr int SZ = (int)sizeof(T);
    const int64_t sqk = (int64_t)p.H * K, sgk = (int64_t)p.HV * K, svv = (int64_t)p.HV * V;
    const auto rs_q = rows_in((const T *)p.q + (bos * p.H + h) * K, nvalid, sqk, K);
    const auto rs_k = rows_in((const T *)p.k + (bos * p.H + h) * K, nvalid, sqk, K);
    const auto rs_g = rows_in((const T *)p.g + (bos * p.HV + j) * K, nvalid, sgk, K);
    const auto rs_v = rows_in((const T *)p.v + (bos * p.HV + j) * V, nvalid, svv, V);
    const auto rs_b = rows_in((const T *)p.beta + bos * p.HV + j, nvalid, p.HV, 1);
    T rq[NE], rk[NE], rg[NE], rv[NEV], rb;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int idx = tid + 256 * e, rr = idx / K, d = idx % K;
        bload_elem(rs_q, (int)(rr * sqk + d) * SZ, rq[e]);
        bload_elem(rs_k, (int)(rr * sqk + d) * SZ, rk[e]);
        bload_elem(rs_g, (int)(rr * sgk + d) * SZ, rg[e]);
    }
#pragma unroll
    for (int e = 0; e < NEV; ++e) {
        const int idx = tid + 256 * e, rr = idx / V, d = idx % V;
        bload_elem(rs_v, (int)(rr * svv + d) * SZ, rv[e]);
    }
    bload_elem(rs_b, (tid & 15) * p.HV * SZ, rb);
    // the gate's dt_bias of this thread's key dim (K divides 256: the same dim for every e)
    const float rdt = gated && p.pre.dt_bias ? p.pre.dt_bias[j * K + tid % K] : 0.f;
    // dO (backward): column tid % V, rows do0 .. do0 + NEV - 1 of the chunk
    const int do0 = (tid / V) * NEV;
    T rdo[BWD ? NEV : 1];
    if (BWD) {
        const auto rs_o = rows_in((const T *)p.d_o + (bos * p.HV + j) * V, nvalid, svv, V);
#pragma unroll
        for (int e = 0; e < NEV; ++e)
            bload_elem(rs_o, (int)((do0 + e) * svv + tid % V) * SZ, rdo[e]);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int idx = tid + 256 * e, rr = idx / K, d = idx % K;
        const bool ok = rr < nvalid;
        sq[rr][d] = ok ? to_f32(rq[e]) : 0.f;
        sk[rr][d] = ok ? to_f32(rk[e]) : 0.f;
        float gv = ok ? to_f32(rg[e]) : 0.f;
        if (gated && ok)
            gv = gate_activation(p.pre, gv + rdt, aexp);
        sG[rr][d] = gv;
    }
#pragma unroll
    for (int e = 0; e < NEV; ++e) {
        const int idx = tid + 256 * e, rr = idx / V, d = idx % V;
        sv[rr][d] = rr < nvalid ? to_f32(rv[e]) : 0.f;
    }
    if (tid < 16) {
        float b = tid < nvalid ? to_f32(rb) : 0.f;
        if (p.pre.beta_sigmoid && tid < nvalid) b = sigmoid_f(b);
        sb[tid] = b;
    }
    __syncthreads();
    if (p.pre.qk_l2norm) {
        // 16 threads per token row (one DPP row of lanes): partial sums, xor reduction, scale
        const int rr = tid >> 4, l = tid & 15;
        float a = 0.f, b = 0.f;
        for (int d = l; d < K; d += 16) {
            a += sq[rr][d] * sq[rr][d];
            b += sk[rr][d] * sk[rr][d];
        }
        for (int m = 1; m < 16; m <<= 1) {
            a += __shfl_xor(a, m);
            b += __shfl_xor(b, m);
        }
        const float fq = l2norm_factor(a), fk = l2norm_factor(b);
        for (int d = l; d < K; d += 16) {
            sq[rr][d] *= fq;
            sk[rr][d] *= fk;
        }
        __syncthreads();
    }
    for (int d = tid; d < K; d += 256) {               // inclusive cumsum per key dim
        float acc = 0.f;
        for (int rr = 0; rr < 16; ++rr) { acc += sG[rr][d]; sG[rr][d] = acc; }
    }
    __syncthreads();

    const int i = tid >> 4, jj = tid & 15;
    // Gram and Mqk entries of the pairs row > col, with the exponent difference exact per pair
    // and dim: pair (a, b) is split over two threads, (a, b) summing the first half of the key
    // dims and (b, a) the second, which hands its part over through sT / sP. The diagonal of
    // Mqk (no decay) is a plain dot product, reduced over the 16 threads of its row.
    const int pa = i > jj ? i : jj, pb = i > jj ? jj : i;
    const int dlo = i >= jj ? 0 : K / 2;
    float Lij = 0.f, Mij = 0.f;
#pragma unroll 2
    for (int d = dlo; d < dlo + K / 2; d += 4) {
        const float4 ga = *(const float4 *)&sG[pa][d], gb = *(const float4 *)&sG[pb][d];
        const float4 ka = *(const float4 *)&sk[pa][d], kb = *(const float4 *)&sk[pb][d];
        const float4 qa = *(const float4 *)&sq[pa][d];
        const float e[4] = {__expf(ga.x - gb.x), __expf(ga.y - gb.y), __expf(ga.z - gb.z),
                            __expf(ga.w - gb.w)};
        const float kd[4] = {kb.x * e[0], kb.y * e[1], kb.z * e[2], kb.w * e[3]};
        Lij += ka.x * kd[0]; Lij += ka.y * kd[1]; Lij += ka.z * kd[2]; Lij += ka.w * kd[3];
        Mij += qa.x * kd[0]; Mij += qa.y * kd[1]; Mij += qa.z * kd[2]; Mij += qa.w * kd[3];
    }
    float Mdiag = 0.f;
    for (int d = jj; d < K; d += 16) Mdiag += sq[i][d] * sk[i][d];
    for (int m = 1; m < 16; m <<= 1) Mdiag += __shfl_xor(Mdiag, m);
    if (i < jj) {
        sT[i][jj] = Lij;
        sP[i][jj] = Mij;
    }
    __syncthreads();
    if (i > jj) {
        Lij += sT[jj][i];
        Mij += sP[jj][i];
    } else if (i == jj) {
        Lij = 0.f;
        Mij = Mdiag;
    }
    const float Lv = i > jj ? sb[i] * Lij : 0.f;
    const float Mv = i >= jj ? p.scale * Mij : 0.f;
    sL[i][jj] = Lv;                   // P = L
    sI[i][jj] = (i == jj ? 1.f : 0.f) - Lv;
    __syncthreads();
    for (int it = 0; it < 3; ++it) {  // P <- P^2 ; INV <- INV + INV P
        float acc = 0.f;
        for (int m = 0; m < 16; ++m) acc += sL[i][m] * sL[m][jj];
        __syncthreads();
        sL[i][jj] = acc;
        __syncthreads();
        float add = 0.f;
        for (int m = 0; m < 16; ++m) add += sI[i][m] * sL[m][jj];
        sT[i][jj] = sI[i][jj] + add;
        __syncthreads();
        sI[i][jj] = sT[i][jj];
        __syncthreads();
    }
    sP[i][jj] = sI[i][jj] * sb[jj];   // A = INV diag(beta)
    __syncthreads();

    float *ws = (float *)(p.ws + ((size_t)j * p.seq.n_slots + slot) * (size_t)STRIDE);
    for (int idx = tid; idx < 16 * K; idx += 256) {   // qd, kr; KD = k e^Gam over q's slot
        const int t = idx / K, d = idx % K;
        const float e = __expf(sG[t][d]);
        ws[WS::QD / 4 + t * K + d] = p.scale * sq[t][d] * e;
        ws[WS::KR / 4 + t * K + d] = sk[t][d] * __expf(sG[15][d] - sG[t][d]);
        sq[t][d] = sk[t][d] * e;
    }
    __syncthreads();
    rows_times_a<K>(sP, sq, ws + WS::W / 4, tid);        // w = A KD
    rows_times_a<V>(sP, sv, ws + WS::U / 4, tid);        // u = A v
    ws[WS::MQK / 4 + i * 16 + jj] = Mv;
    for (int d = tid; d < K; d += 256) ws[WS::EG / 4 + d] = __expf(sG[15][d]);
    if (BWD) {                        // the inverse and the Gram, for the local gradients
        ws[WsF32B<K, V>::XM / 4 + i * 16 + jj] = sI[i][jj];
        ws[WsF32B<K, V>::GM / 4 + i * 16 + jj] = i > jj ? Lij : 0.f;
        // dO in the grads chain's operand order (a 16-byte load per lane): element (t, d) at
        // [d / 16][lane (t / 4, d % 16)][t % 4]; each thread writes whole 16-byte groups (four
        // rows of its column)
        const __amdgpu_buffer_rsrc_t dr = buffer_rsrc(ws + WsF32B<K, V>::DO / 4, 16 * V * 4);
        const int d = tid % V;
#pragma unroll
        for (int e = 0; e < NEV; e += 4) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = do0 + e + i < nvalid ? to_f32(rdo[e + i]) : 0.f;
            const int off = ((d / 16) * 64 + ((do0 + e) / 4) * 16 + d % 16) * 16;
            bstore16<0>(dr, off, 0, f32x4{x[0], x[1], x[2], x[3]});
        }
    }
}

template <int K, int V>
hipError_t launch_prepare_bf16(const FwdParams &p, hipStream_t st)
{
    dim3 grid(p.seq.n_slots, p.HV);
    prepare_bf16_kernel<K, V><<<grid, dim3(64), 0, st>>>(p);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_prepare_f32(const FwdParams &p, hipStream_t st, bool in_bf16,
                              bool for_backward)
{
    dim3 grid(p.seq.n_slots, p.HV);
    if (in_bf16 && for_backward)
        prepare_f32_kernel<K, V, uint16_t, true><<<grid, dim3(256), 0, st>>>(p);
    else if (in_bf16)
        prepare_f32_kernel<K, V, uint16_t, false><<<grid, dim3(256), 0, st>>>(p);
    else if (for_backward)
        prepare_f32_kernel<K, V, float, true><<<grid, dim3(256), 0, st>>>(p);
    else
        prepare_f32_kernel<K, V, float, false><<<grid, dim3(256), 0, st>>>(p);
    return hipGetLastError();
}

#define KDA_INST(K, V)                                                               \
    template hipError_t launch_prepare_bf16<K, V>(const FwdParams &, hipStream_t);  \
    template hipError_t launch_prepare_f32<K, V>(const FwdParams &, hipStream_t, bool, bool);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
