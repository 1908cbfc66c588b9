// kda_prep32.h -- stage 1 with 32-token chunks: everything that depends only on one
// 32-token chunk of one value head, so that the state kernel takes one serial step per 32
// tokens ("手撕KDA" section 1 chunks at 64 by default; the FlashKDA kernel of
// "KDA源码剖析之FlashKDA（上）" uses 16-token tiles and a 16x16 Neumann inverse).
//
// The chunk is two 16-token row blocks a (tokens 0..15) and b (16..31), one wave each. With
// Gam the cumsum of g from the chunk start and gam its value at the last token,
//     L   = beta_row * strict_tril(k e^{Gam} . (k e^{-Gam})^T)    (32 x 32, block lower
//           triangular: L_aa, L_bb strictly lower, L_ba full, L_ab = 0)
//     X   = (I + L)^{-1} = [[X_aa, 0], [X_ba, X_bb]],  X_aa, X_bb by the Neumann doubling product
//           of "KDA源码剖析之FlashKDA（上）" part 12, X_ba = -X_bb L_ba X_aa (block forward
//           substitution; every factor stays as bounded as the inverse itself)
//     A   = X diag(beta),  W = A (k e^{Gam}),  U = A v,  QD = scale q e^{Gam},
//     KR  = k e^{gam - Gam},  Mqk = tril(QD' . KI'^T) (32 x 32),  e^{gam}
// (U is stored negated, see WsBf16x32)
// which is the chunk half of naive_chunk_kda ("手撕KDA" section 1) for a 32-token chunk.
//
// The per-block work is the 16-token kernel of kda_prepare.hip (same layouts, same numerics:
// token-centred hi+lo bf16 factors, fp32 Neumann, identity-MFMA layout changes). Block b also
// needs block a's cumsum total, its k e^{-Gam} factors, X_aa, its column-per-lane k e^{Gam} and
// v tiles and its beta, which wave a hands over through LDS (about 19 KB).
#pragma once

#include "kda_internal.h"

namespace kda {

template <int K, int V>
struct Prep32Share {
    static constexpr int MAXKV = K > V ? K : V;
    static constexpr int STAGE = 16 * (2 * MAXKV + 16);   // one block's 16 rows, padded
    float tot_a[K];              // Gam (log2 units) at the last token of block a
    float tot_ab[K];             // Gam at the last token of the chunk
    bf16x8 kih[K / 32][64];      // block a: k e^{ref - Gam}, hi part, 16x16x32 B operand
    bf16x8 kil[K / 32][64];      //          lo part
    f32x4 xaa[64];               // C(X_aa)
    float beta_a[16];
    union {
        struct {
            f32x4 g2b[K / 16][64];       // block b: Gam in TPL, one tile per entry
            union {                      // block a: its Gam tiles, then (once both of its
                f32x4 g2a[K / 16][64];   // factor phases are done) its column-per-lane KD
                struct {                 // and V tiles
                    bf16x4 kdc[K / 16][64];
                    bf16x4 vc[V / 16][64];
                } cols;
            } a;
        } ph;
        uint8_t stage[2][STAGE];         // per block: input rows on their way to TPL (first)
    } u;
    __device__ __forceinline__ f32x4 &g2(int wave, int c, int lane) {
        return wave == 0 ? u.ph.a.g2a[c][lane] : u.ph.g2b[c][lane];
    }
};

// Carried from the first to the second chunk of a 64-token pair (one workgroup processes both,
// in order): the first chunk's KR in TPL (fp16, one 16x16x32 operand per 32-dim slab and block)
// and its e^{gam}.
template <int K>
struct PairStash {
    f16x8 kr0[2][K / 32][64];
    float eg0[K];
};

// Inputs of one 32-token chunk as each lane loads them: the 16 rows of its block (wave)
// row-contiguously, 16 bytes per lane (row RPI u + lane / CPR, 8 columns from 8 (lane % CPR)),
// so that every quarter-wave reads one or two whole cache lines.
template <int K, int V>
struct Prep32In {
    u32x4 q[K / 32], k[K / 32], g[K / 32], v[V / 32];
    unsigned beta;               // bf16 bits of beta of row lane % 16 (0 past the valid rows)
    int nrows;                   // valid rows of the block (the rest are zero padding)
    int64_t tok0;                // packed-axis index of the block's first token
};

// The loads go through a buffer resource whose range ends with the block's last valid row:
// rows past it read as zero (the hardware's range check), so no load sits under a branch. A
// branch around a load had made the compiler wait for it right there (a register copy of the
// loaded value inside the branch), which serialised the whole load phase.
template <int RL>
__device__ __forceinline__ void load_rows(const uint16_t *base, int64_t row_elems, int nrows,
                                          int lane, u32x4 (&x)[RL / 32])
{
    constexpr int CPR = RL / 8, RPI = 64 / CPR;     // 16-byte chunks per row, rows per load
    const uint32_t row_bytes = (uint32_t)row_elems * 2u;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(base, nrows > 0 ? (uint32_t)(nrows - 1) * row_bytes + 2u * RL : 0u);
#pragma unroll
    for (int u = 0; u < RL / 32; ++u)
        x[u] = bload16(rs, (int)((RPI * u + lane / CPR) * row_bytes) + 16 * (lane % CPR), 0);
}

template <int K, int V>
__device__ __forceinline__ void prep32_load(const FwdParams &p, int64_t bos, int nvalid, int j,
                                            int wave, int lane, Prep32In<K, V> &in)
{
    const int r = lane & 15;
    // the block index is the same in every lane: read it as a scalar so that the buffer
    // resources below are scalar too (a per-lane one needs a loop around every load)
    const int blk = __builtin_amdgcn_readfirstlane(wave);
    const int64_t tok0 = bos + 16 * blk;
    const int nrows = nvalid - 16 * blk;            // valid rows of this block (may be <= 0)
    const int h = j / p.G;
    load_rows<K>((const uint16_t *)p.g + (tok0 * p.HV + j) * K, (int64_t)p.HV * K, nrows, lane,
                 in.g);
    load_rows<K>((const uint16_t *)p.k + (tok0 * p.H + h) * K, (int64_t)p.H * K, nrows, lane,
                 in.k);
    load_rows<K>((const uint16_t *)p.q + (tok0 * p.H + h) * K, (int64_t)p.H * K, nrows, lane,
                 in.q);
    load_rows<V>((const uint16_t *)p.v + (tok0 * p.HV + j) * V, (int64_t)p.HV * V, nrows, lane,
                 in.v);
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc((const uint16_t *)p.beta + tok0 * p.HV + j,
                    nrows > 0 ? (uint32_t)((nrows - 1) * p.HV) * 2u + 2u : 0u);
    in.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, r * p.HV * 2, 0, 0);
    in.nrows = nrows;
    in.tok0 = tok0;
}

// Row-contiguous input rows -> TPL (lane (g, r): row r, columns 16c + 4g .. + 3) through this
// wave's LDS stage. The row stride is padded by 16 bytes, so the 16 rows read by a quarter-wave
// fall in distinct banks. Only this wave touches its stage, and one wave's LDS accesses are
// performed in order.
template <int RL>
__device__ __forceinline__ void rows_to_tpl(const u32x4 (&x)[RL / 32], uint2 (&out)[RL / 16],
                                            uint8_t *stage, int lane)
{
    constexpr int CPR = RL / 8, RPI = 64 / CPR, STRIDE = 2 * RL + 16;
#pragma unroll
    for (int u = 0; u < RL / 32; ++u)
        *(u32x4 *)(stage + (RPI * u + lane / CPR) * STRIDE + 16 * (lane % CPR)) = x[u];
    const int grp = lane >> 4, r = lane & 15;
#pragma unroll
    for (int c = 0; c < RL / 16; ++c)
        out[c] = *(const uint2 *)(stage + r * STRIDE + 32 * c + 8 * grp);
}

// One 32-token chunk of one value head from its loaded inputs; both waves of the workgroup
// call it together (it synchronises the workgroup).
//
// `wr` is a buffer resource over the chunk's workspace record (a zero-sized one drops every
// store) of value head j; AUX is the cache policy of the stores. NORM: q and k are divided by
// their L2 norms (pre-stage); the factor of each token's row is applied in fp32 wherever q or
// k is unpacked, so the bf16 inputs are not rounded again. A gate activation (pre-stage) is
// applied to g before the cumsum, to valid rows only (padding rows keep g = 0).
//
// PAIR: 0 for a stand-alone 32-token record; 1 and 2 for the first and second chunk of a
// 64-token pair (WsPair records, the state kernel's 64-token step). The first chunk also leaves
// its KR (TPL) and e^{gam} in `ps`; the second stores its W scaled by the first chunk's e^{gam}
// per key dim and the 32 x 32 product P = W KR_first^T as the A operand of the state kernel's
// delta correction (WsPair::PT).
//
// `after_inputs` runs as soon as this chunk's inputs have arrived (the caller issues the next
// chunk's loads there, so they stream in while this chunk is processed instead of competing
// with this chunk's own loads).
struct NoOp {
    __device__ void operator()() const {}
};

template <int K, int V, bool NORM = false, int AUX = 0, int PAIR = 0, class AFTER = NoOp>
__device__ __forceinline__ void prep32_chunk(const FwdParams &p, Prep32Share<K, V> &sh,
                                             PairStash<K> *ps, const Prep32In<K, V> &in,
                                             __amdgpu_buffer_rsrc_t wr, int j, int wave,
                                             int lane, AFTER after_inputs = NoOp())
{
    constexpr int NK = K / 16, NV = V / 16, NS = K / 32;
    using WS = WsBf16x32<K, V>;
    const int grp = lane >> 4;
    const int r = lane & 15;                 // TPL: token row in the block; C-layout: column
    // q, k and v stay as packed bf16 pairs until each use: every phase below rebuilds the fp32
    // values it needs from them, which keeps the live register set small enough for several
    // waves per SIMD.
    // gate parameters of this value head, loaded first so their latency is covered
    const bool gated = p.pre.gate != 0;
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
    uint2 qr[NK], kr[NK], gr[NK], vraw[NV];
    uint8_t *stage = sh.u.stage[wave];
    rows_to_tpl<K>(in.g, gr, stage, lane);
    rows_to_tpl<K>(in.k, kr, stage, lane);
    rows_to_tpl<K>(in.q, qr, stage, lane);
    rows_to_tpl<V>(in.v, vraw, stage, lane);
    after_inputs();
    float beta_r = bf16_bits_to_f32((uint16_t)in.beta);
    if (p.pre.beta_sigmoid && r < in.nrows) beta_r = sigmoid_f(beta_r);   // pre-stage
    // L2-norm factors of this lane's token row (its other columns are in the three other lane
    // groups); padding rows are zero and stay zero
    float rk = 1.f, rq = 1.f;
    if constexpr (NORM) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            float kk[4], qq[4];
            unpack_bf16x4(kr[c], kk);
            unpack_bf16x4(qr[c], qq);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sk += kk[i] * kk[i];
                sq += qq[i] * qq[i];
            }
        }
        rk = l2norm_factor(sum_lane_groups(sk));
        rq = l2norm_factor(sum_lane_groups(sq));
    }

    // ---------------------------------------------------------------- cumsum over 32 tokens
    float G2[NK][4];
    if (!gated) {
        // The block's running sums on the matrix core: the identity product turns the TPL tile
        // of g into C layout (lane (g, n): tokens 4g .. 4g + 3 of column n), which read as an A
        // operand is g^T; times the upper-triangular ones matrix T (T[s][t] = 1 for s <= t) it
        // gives C(g^T T), whose lane (g, r) holds the sums over tokens 0 .. r of columns
        // 4g .. 4g + 3: TPL again. g is bf16, so both products are exact up to the fp32 sums.
        // (A DPP scan per element cost about nine VALU instructions and hazard waits each.)
        float eye[4], up[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            eye[i] = 4 * grp + i == r ? 1.f : 0.f;
            up[i] = 4 * grp + i <= r ? 1.f : 0.f;
        }
        const bf16x4 Ib = to_bf16x4(eye), Tb = to_bf16x4(up);
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            const f32x4 gc = mfma16(__builtin_bit_cast(bf16x4, gr[c]), Ib, zero4());
            const f32x4 cs = mfma16(to_bf16x4(gc), Tb, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) G2[c][i] = cs[i] * LOG2E;
        }
    } else {
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            float gl[4];
            unpack_bf16x4(gr[c], gl);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                gl[i] = r < in.nrows ? gate_activation(p.pre, gl[i] + dtv[c][i], aexp) : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) G2[c][i] = row_inclusive_scan(gl[i] * LOG2E);
        }
    }
    if (wave == 0) {
        if (r == 15) {
#pragma unroll
            for (int c = 0; c < NK; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) sh.tot_a[16 * c + 4 * grp + i] = G2[c][i];
        }
        if (grp == 0) sh.beta_a[r] = beta_r;
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            const float4 t = *(const float4 *)&sh.tot_a[16 * c + 4 * grp];
            G2[c][0] += t.x; G2[c][1] += t.y; G2[c][2] += t.z; G2[c][3] += t.w;
        }
        if (r == 15) {
#pragma unroll
            for (int c = 0; c < NK; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) sh.tot_ab[16 * c + 4 * grp + i] = G2[c][i];
        }
    }
    // Gam goes to LDS and is read back one tile at a time by both factor phases
#pragma unroll
    for (int c = 0; c < NK; ++c)
        sh.g2(wave, c, lane) = f32x4{G2[c][0], G2[c][1], G2[c][2], G2[c][3]};
    __syncthreads();

    float b4[4], eye[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b4[i] = lane_read(beta_r, 4 * grp + i);        // beta of row 4g + i of this block
        eye[i] = 4 * grp + i == r ? 1.f : 0.f;
    }
    const bf16x4 Ib = to_bf16x4(eye);
    const f16x4 Ih = to_f16x4(eye);

    // The two factor phases below are independent except that block b's off-diagonal Gram
    // products need block a's KI factors. Block a therefore forms its Gram products first and
    // block b its QD / KR phase; after the hand-over each does the other phase, and block b
    // builds its diagonal and off-diagonal products slab by slab without keeping any factors.
    const float sc = p.scale * rq;            // the output scale and q's norm factor
    bf16x4 kdC[NK];
    f32x4 Lacc = zero4(), Macc = zero4(), Lba = zero4(), Mba = zero4();

    // QD, KR, e^{gam}, KD: factors relative to the chunk start, stored as soon as they are
    // formed; KD is kept in column-per-lane form (identity MFMA) for W
    auto qd_kr_phase = [&]() {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            float QD[2][4];
            f16x4 krh[2];                    // this slab's KR tiles in TPL (fp16)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = 2 * st + u;
                const float4 gm = *(const float4 *)&sh.tot_ab[16 * c + 4 * grp];
                const float gam[4] = {gm.x, gm.y, gm.z, gm.w};
                const f32x4 gc = sh.g2(wave, c, lane);
                float kk[4], qq[4], KD[4], KRv[4];
                unpack_bf16x4(kr[c], kk);
                unpack_bf16x4(qr[c], qq);
                if constexpr (NORM) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) kk[i] *= rk;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float eA = __builtin_amdgcn_exp2f(gc[i]);
                    const float eR = __builtin_amdgcn_exp2f(gam[i] - gc[i]);
                    KD[i] = kk[i] * eA;
                    QD[u][i] = sc * qq[i] * eA;
                    KRv[i] = kk[i] * eR;
                }
                kdC[c] = to_bf16x4(mfma16(to_bf16x4(KD), Ib, zero4()));
                krh[u] = to_f16x4(KRv);
                bstore8<AUX>(wr, lane * 16 + wave * 8, WS::KR + c * 1024,
                             to_f16x4(mfma16(krh[u], Ih, zero4())));
            }
            if constexpr (PAIR == 1) ps->kr0[wave][st][lane] = cat(krh[0], krh[1]);
            bstore16<AUX>(wr, lane * 16, WS::QD + (wave * NS + st) * 1024,
                          cat(to_f16x4(QD[0]), to_f16x4(QD[1])));
        }
        if (wave == 1 && r == 15) {
#pragma unroll
            for (int c = 0; c < NK; ++c) {
                const f32x4 gc = sh.u.ph.g2b[c][lane];
                f32x4 e;
#pragma unroll
                for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(gc[i]);
                bstore16<AUX>(wr, grp * 16, WS::EG + 64 * c, e);
                if constexpr (PAIR == 1) *(f32x4 *)&ps->eg0[16 * c + 4 * grp] = e;
            }
        }
    };

    // Gram products L = KD KI^T and Mqk = QD KI^T with factors centred on the block boundary
    // (token 15, the middle of the chunk), each as hi + lo bf16 in three passes (hi hi, hi lo,
    // lo hi), one 32-column slab at a time. Block a publishes its KI factors; block b also
    // contracts its rows against them (the off-diagonal blocks L_ba, Mqk_ba).
    auto gram_phase = [&]() {
        float span = 0.f;                    // largest |exponent| of this block's factors
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            bf16x8 kdh, kdl, kih, kil, qdh, qdl;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = 2 * st + u;
                const float4 rf = *(const float4 *)&sh.tot_a[16 * c + 4 * grp];
                const float ref[4] = {rf.x, rf.y, rf.z, rf.w};
                const f32x4 gc = sh.g2(wave, c, lane);
                float kk[4], qq[4];
                unpack_bf16x4(kr[c], kk);
                unpack_bf16x4(qr[c], qq);
                if constexpr (NORM) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) kk[i] *= rk;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d1 = gc[i] - ref[i];
                    span = fmaxf(span, fabsf(d1));
                    const float e1 = __builtin_amdgcn_exp2f(d1);
                    const float e2 = __builtin_amdgcn_exp2f(-d1);
                    const float xd = kk[i] * e1, xi = kk[i] * e2, xq = sc * qq[i] * e1;
                    const int e = u * 4 + i;
                    const __bf16 hd = (__bf16)xd, hi_ = (__bf16)xi, hq = (__bf16)xq;
                    kdh[e] = hd; kdl[e] = (__bf16)(xd - (float)hd);
                    kih[e] = hi_; kil[e] = (__bf16)(xi - (float)hi_);
                    qdh[e] = hq; qdl[e] = (__bf16)(xq - (float)hq);
                }
            }
            Lacc = mfma32(kdh, kih, Lacc);
            Macc = mfma32(qdh, kih, Macc);
            Lacc = mfma32(kdh, kil, Lacc);
            Macc = mfma32(qdh, kil, Macc);
            Lacc = mfma32(kdl, kih, Lacc);
            Macc = mfma32(qdl, kih, Macc);
            if (wave == 0) {
                sh.kih[st][lane] = kih;
                sh.kil[st][lane] = kil;
            } else {
                const bf16x8 ah = sh.kih[st][lane], al = sh.kil[st][lane];
                Lba = mfma32(kdh, ah, Lba);
                Mba = mfma32(qdh, ah, Mba);
                Lba = mfma32(kdh, al, Lba);
                Mba = mfma32(qdh, al, Mba);
                Lba = mfma32(kdl, ah, Lba);
                Mba = mfma32(qdl, ah, Mba);
            }
        }
        // The factors above are centred on the chunk middle, which bounds every factor of the
        // off-diagonal block (rows after, columns before the middle) by 1 whatever the decay;
        // the diagonal block's factors span the decay between the middle and the block's far
        // end. Beyond FACTOR_SPAN_MAX that block's products are formed from exact per-token
        // decay products instead (wave-uniform branch; no barrier inside).
        if (__builtin_amdgcn_ballot_w64(span > FACTOR_SPAN_MAX) != 0) {
            const int h = j / p.G;
            const BlockRows br{(const uint16_t *)p.q + (in.tok0 * p.H + h) * K,
                               (const uint16_t *)p.k + (in.tok0 * p.H + h) * K,
                               (const uint16_t *)p.g + (in.tok0 * p.HV + j) * K,
                               (int64_t)p.H * K, (int64_t)p.HV * K, in.nrows};
            exact_block_gram<K>(br, p.pre, j, aexp, rk, sc, lane, Lacc, Macc);
        }
    };

    if (wave == 0) gram_phase(); else qd_kr_phase();
    __syncthreads();
    if (wave == 0) qd_kr_phase(); else gram_phase();

    float Mq[4];
    f32x4 L;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 4 * grp + i;
        L[i] = rr > r ? b4[i] * Lacc[i] : 0.f;
        Mq[i] = rr >= r ? Macc[i] : 0.f;
    }
    const f32x4 eyev = {eye[0], eye[1], eye[2], eye[3]};

    // Neumann product of the diagonal block on the fp32 matrix core (see kda_prepare.hip):
    // INV = C(X^T); block a also forms C(X) for block b's off-diagonal solve
    const f32x4 Mf = mm16_f32(L, eyev, zero4());
    const f32x4 P2 = mm16_f32(L, Mf, zero4());
    const f32x4 Q2 = mm16_f32(Mf, L, zero4());
    const f32x4 P4 = mm16_f32(Q2, P2, zero4());
    const f32x4 Q4 = mm16_f32(P2, Q2, zero4());
    const f32x4 Q8 = mm16_f32(P4, Q4, zero4());
    f32x4 INV = eyev - Mf;
    INV = mm16_f32(Q2, INV, INV);
    INV = mm16_f32(Q4, INV, INV);
    INV = mm16_f32(Q8, INV, INV);
    if (wave == 0) {
        const f32x4 P8 = mm16_f32(Q4, P4, zero4());       // C(M^8) == A16 of L^8
        f32x4 XN = eyev - L;                               // C(I - L)
        XN = mm16_f32(P2, XN, XN);                         // (I + L^2)(I - L)
        XN = mm16_f32(P4, XN, XN);
        XN = mm16_f32(P8, XN, XN);                         // C(X_aa)
        sh.xaa[lane] = XN;
    }

    // column-per-lane KD and V tiles of block a for block b's W and U rows
    bf16x4 vC[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c)
        vC[c] = to_bf16x4(mfma16(__builtin_bit_cast(bf16x4, vraw[c]), Ib, zero4()));
    if (wave == 0) {
#pragma unroll
        for (int c = 0; c < NK; ++c) sh.u.ph.a.cols.kdc[c][lane] = kdC[c];
#pragma unroll
        for (int c = 0; c < NV; ++c) sh.u.ph.a.cols.vc[c][lane] = vC[c];
    }
    __syncthreads();

    // ---------------------------------------------------------------- W, U, Mqk
    float AT[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) AT[i] = INV[i] * b4[i];     // C(A_xx^T) = diag(beta) X_xx^T
    const bf16x4 ATb = to_bf16x4(AT);
    const f16x4 MqT = to_f16x4(mfma16(to_f16x4(Mq), Ih, zero4()));   // C(Mqk_xx^T)
    // W rows of this block, slab st, from the two TPL tiles t0, t1 (fp32). The second chunk of
    // a pair also contracts them against the first chunk's KR (C(P^T) for both of its blocks)
    // and stores them scaled by the first chunk's e^{gam} per key dim.
    f32x4 Pa = zero4(), Pb = zero4();
    auto store_w = [&](int st, f32x4 t0, f32x4 t1) {
        const f16x8 wf = cat(to_f16x4(t0), to_f16x4(t1));
        if constexpr (PAIR == 2) {
            Pa = mfma32(ps->kr0[0][st][lane], wf, Pa);
            Pb = mfma32(ps->kr0[1][st][lane], wf, Pb);
            const f32x4 e0 = *(const f32x4 *)&ps->eg0[32 * st + 4 * grp];
            const f32x4 e1 = *(const f32x4 *)&ps->eg0[32 * st + 16 + 4 * grp];
            bstore16<AUX>(wr, lane * 16, WS::W + (wave * NS + st) * 1024,
                          cat(to_f16x4(t0 * e0), to_f16x4(t1 * e1)));
        } else {
            bstore16<AUX>(wr, lane * 16, WS::W + (wave * NS + st) * 1024, wf);
        }
    };
    if (wave == 0) {
#pragma unroll
        for (int st = 0; st < NS; ++st)
            store_w(st, mfma16(kdC[2 * st], ATb, zero4()), mfma16(kdC[2 * st + 1], ATb, zero4()));
#pragma unroll
        for (int c = 0; c < NV; ++c)
            bstore8<AUX>(wr, lane * 16, WS::NU + c * 1024,
                         to_f16x4(-mfma16(ATb, vC[c], zero4())));
        bstore8<AUX>(wr, lane * 8, WS::MQKA, MqT);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) Lba[i] *= b4[i];
        // X_ba^T = -X_aa^T L_ba^T X_bb^T
        const f32x4 Pm = mm16_f32(Lba, INV, zero4());       // C(L_ba^T X_bb^T)
        const f32x4 XbaT = mm16_f32(sh.xaa[lane], Pm, zero4());
        float ABT[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ABT[i] = -XbaT[i] * sh.beta_a[4 * grp + i];
        const bf16x4 ABTb = to_bf16x4(ABT);                  // C(A_ba^T)
        const bf16x8 Arow = cat(ABTb, ATb);                  // [A_ba | A_bb] as A (16 x 32)
#pragma unroll
        for (int st = 0; st < NS; ++st)
            store_w(st,
                    mfma32(cat(sh.u.ph.a.cols.kdc[2 * st][lane], kdC[2 * st]), Arow, zero4()),
                    mfma32(cat(sh.u.ph.a.cols.kdc[2 * st + 1][lane], kdC[2 * st + 1]), Arow,
                           zero4()));
#pragma unroll
        for (int c = 0; c < NV; ++c)
            bstore8<AUX>(wr, lane * 16 + 8, WS::NU + c * 1024,
                         to_f16x4(-mfma32(Arow, cat(sh.u.ph.a.cols.vc[c][lane], vC[c]), zero4())));
        const f16x4 MqbaT = to_f16x4(mfma16(to_f16x4(Mba), Ih, zero4()));  // C(Mqk_ba^T)
        bstore16<AUX>(wr, lane * 16, WS::MQKB, cat(MqbaT, MqT));
    }
    // C(P_{x,a}^T), C(P_{x,b}^T) side by side: lane (g, n) holds row n of this block's P
    // against tokens 4g .. 4g + 3 of the first chunk's blocks a and b, the 16x16x32 A operand
    // that pairs with the first chunk's delta in the state kernel
    if constexpr (PAIR == 2)
        bstore16<AUX>(wr, lane * 16, WsPair<K, V>::PT + wave * 1024,
                      cat(to_f16x4(Pa), to_f16x4(Pb)));
}

}  // namespace kda
