// kda_state64.h -- stage 2 with 64-token steps: the chunk-sequential state pass over pairs of
// 32-token chunk records (WsPair), one serial step per 64 tokens.
//
// Per pair of chunks (c, c + 1), with S the K x V state at the pair's start ("手撕KDA"
// section 1, the chunk loop of naive_chunk_kda, two chunks at a time):
//     delta_c     = U_c - W_c S
//     S_{c+1}     = diag(e^{gam_c}) S + KR_c^T delta_c
//     delta_{c+1} = U_{c+1} - W_{c+1} S_{c+1}
//                 = U_{c+1} - (W_{c+1} diag(e^{gam_c})) S - P delta_c,    P = W_{c+1} KR_c^T
//     S_{c+2}     = diag(e^{gam_{c+1}}) S_{c+1} + KR_{c+1}^T delta_{c+1}
//     o_c = QD_c S + Mqk_c delta_c,   o_{c+1} = QD_{c+1} S_{c+1} + Mqk_{c+1} delta_{c+1}
// The prepare kernel stores W_{c+1} diag(e^{gam_c}) and P, so both deltas follow from the state
// at the pair's start with ONE contraction over the key dimension: the two chain waves (each
// owning half of S's key rows) form their halves of W_c S and W'_{c+1} S and exchange them
// through LDS once per 64 tokens; P delta_c is a 32 x 32 x 16 product after the exchange.
//
// Workgroup per (sequence, value head, 16-column slice of V), four waves: two chain waves as in
// kda_state32.h and two output waves, one per chunk of the pair, which form o after barrier
// m + 1 from the fp16 copies of S_c and S_{c+1} the chain waves hand over and the deltas.
#pragma once

#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ bool state_unit64(int wg, int NV, int units, int *unit, int *slice) {
    // all V/16 slices of one (sequence, value head) on one XCD (dispatch is round-robin over
    // the 8 XCDs, each with its own L2), so they share the records in L2
    const int xcd = wg & 7, idx = wg >> 3;
    *unit = (idx / NV) * 8 + xcd;
    *slice = idx % NV;
    return *unit < units;
}

// Operands of one pair for the chain wave that owns key rows [K/2 h, K/2 (h + 1)), in two
// groups: W (used before the step's exchange; two register sets, loaded two pairs ahead) and
// the rest (used after it; one set, refilled right after its last use, one pair ahead).
template <int K, int V>
struct PairFragW {
    static constexpr int NSH = K / 64;     // 32-row slabs owned
    f16x8 w0[2][NSH];         // W_c rows of blocks a, b (this half's key columns)
    f16x8 w1[2][NSH];         // W_{c+1} diag(e^{gam_c}) rows of blocks a, b
    f16x8 nu0, nu1;           // -U_c, -U_{c+1} of this slice (half 0 only)
};

template <int K, int V>
struct PairFragK {
    static constexpr int NKH = K / 32;     // 16-row tiles owned
    u32x4 egr0, egr1;         // e^{gam_c}, e^{gam_{c+1}} of this half's rows (expand_rows)
    f16x8 kr0[NKH], kr1[NKH]; // KR_c^T, KR_{c+1}^T tiles of this half over 32 tokens
    f16x8 pt[2];              // P rows of chunk c+1's blocks a, b (A operand over chunk c)
};

// Output operands of one chunk of a pair (each output wave forms o of one chunk).
template <int K, int V>
struct PairOutFrag {
    f16x8 qd[2][K / 32];      // [block][slab]
    f16x4 mqa;
    f16x8 mqb;
};

// The two records of one pair through one buffer resource (scalar base = the first record);
// field offsets are scalar, the per-lane part is lane * size. AUX: cache policy of the loads.
template <int K, int V, int AUX = 0>
struct Pair64 {
    using WS = WsBf16x32<K, V>;
    using WP = WsPair<K, V>;
    static constexpr int NS = K / 32;
    static constexpr int NSH = K / 64, NKH = K / 32;
    __amdgpu_buffer_rsrc_t rs;
    int lane, slice;
    template <int h>
    __device__ __forceinline__ void load_w(PairFragW<K, V> &f) const {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int j = 0; j < NSH; ++j) {
                    const f16x8 x = __builtin_bit_cast(
                        f16x8, bload16<AUX>(rs, lane * 16,
                                            c * WP::BYTES + WS::W + (b * NS + h * NSH + j) * 1024));
                    if (c == 0) f.w0[b][j] = x; else f.w1[b][j] = x;
                }
        if constexpr (h == 0) {
            f.nu0 = __builtin_bit_cast(f16x8, bload16<AUX>(rs, lane * 16, WS::NU + slice * 1024));
            f.nu1 = __builtin_bit_cast(
                f16x8, bload16<AUX>(rs, lane * 16, WP::BYTES + WS::NU + slice * 1024));
        }
    }
    template <int h>
    __device__ __forceinline__ void load_k(PairFragK<K, V> &f) const {
        const int grp = lane >> 4;
        const int egoff = ((lane & 15) % NKH) * 64 + grp * 16;
        f.egr0 = bload16<AUX>(rs, egoff, WS::EG + h * NKH * 64);
#pragma unroll
        for (int t = 0; t < NKH; ++t)
            f.kr0[t] = __builtin_bit_cast(
                f16x8, bload16<AUX>(rs, lane * 16, WS::KR + (h * NKH + t) * 1024));
#pragma unroll
        for (int b = 0; b < 2; ++b)
            f.pt[b] = __builtin_bit_cast(
                f16x8, bload16<AUX>(rs, lane * 16, WP::BYTES + WP::PT + b * 1024));
        f.egr1 = bload16<AUX>(rs, egoff, WP::BYTES + WS::EG + h * NKH * 64);
#pragma unroll
        for (int t = 0; t < NKH; ++t)
            f.kr1[t] = __builtin_bit_cast(
                f16x8, bload16<AUX>(rs, lane * 16, WP::BYTES + WS::KR + (h * NKH + t) * 1024));
    }
    template <int k>
    __device__ __forceinline__ void load_out(PairOutFrag<K, V> &f) const {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int st = 0; st < NS; ++st)
                f.qd[b][st] = __builtin_bit_cast(
                    f16x8, bload16<AUX>(rs, lane * 16,
                                        k * WP::BYTES + WS::QD + (b * NS + st) * 1024));
        f.mqa = __builtin_bit_cast(f16x4, bload8<AUX>(rs, lane * 8, k * WP::BYTES + WS::MQKA));
        f.mqb = __builtin_bit_cast(f16x8, bload16<AUX>(rs, lane * 16, k * WP::BYTES + WS::MQKB));
    }
};

template <int K>
struct Handoff64 {
    f16x8 sh[3][2][K / 32][64];  // S_c and S_{c+1} (fp16) of pair m in slot m % 3
    f32x4 xp[2][2][4][64];       // [pair parity][half][a_c, b_c, a_{c+1}, b_{c+1}] partials
    f16x4 dh[2][4][64];          // [pair parity][a_c, b_c, a_{c+1}, b_{c+1}] delta
};

// Chain wave h, pair m (S = its rows of the state at the pair's start), up to and including
// barrier m: fp16 rows of S to the hand-off, then its halves of W_c S and W'_{c+1} S (half 0
// starts both from -U) to the other half.
template <int K, int V, int h>
__device__ __forceinline__ void chain64_a(const PairFragW<K, V> &f, const f32x4 (&S)[K / 32],
                                          f32x4 (&X)[4], Handoff64<K> &ho, int slot, int par,
                                          int lane)
{
    constexpr int NSH = K / 64;
    if constexpr (h == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            X[0][i] = (float)f.nu0[i];
            X[1][i] = (float)f.nu0[4 + i];
            X[2][i] = (float)f.nu1[i];
            X[3][i] = (float)f.nu1[4 + i];
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) X[q] = zero4();
    }
#pragma unroll
    for (int j = 0; j < NSH; ++j) {
        const f16x8 Sh = cat(to_f16x4(S[2 * j]), to_f16x4(S[2 * j + 1]));
        ho.sh[slot][0][h * NSH + j][lane] = Sh;
        X[0] = mfma32(f.w0[0][j], Sh, X[0]);
        X[1] = mfma32(f.w0[1][j], Sh, X[1]);
        X[2] = mfma32(f.w1[0][j], Sh, X[2]);
        X[3] = mfma32(f.w1[1][j], Sh, X[3]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) ho.xp[par][h][q][lane] = X[q];
    lds_barrier();
}

// Chain wave h after barrier m: both deltas from the two halves' partials (the same fp32
// operands in both halves, so both hold the same deltas), S_{c+1} (its fp16 rows to the
// hand-off for the output wave), then S_{c+2}. The W group is refilled from `nxw` (two pairs
// ahead) right after the exchange, the other group from `nxk` (the next pair) after its last
// use.
template <int K, int V, int h, int AUX>
__device__ __forceinline__ void chain64_b(PairFragW<K, V> &fw, PairFragK<K, V> &fk,
                                          const f32x4 (&eg0)[K / 32],
                                          const f32x4 (&eg1)[K / 32],
                                          const Pair64<K, V, AUX> &nxw,
                                          const Pair64<K, V, AUX> &nxk, f32x4 (&S)[K / 32],
                                          const f32x4 (&X)[4], Handoff64<K> &ho, int slot,
                                          int par, int lane)
{
    constexpr int NKH = K / 32, NSH = K / 64;
    f32x4 Po[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) Po[q] = ho.xp[par][1 - h][q][lane];
    nxw.template load_w<h>(fw);
    f16x4 d0a, d0b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d0a[i] = (_Float16)(-(X[0][i] + Po[0][i]));
        d0b[i] = (_Float16)(-(X[1][i] + Po[1][i]));
    }
    const f16x8 d0 = cat(d0a, d0b);
    // P delta_c, rows of chunk c + 1's blocks a and b
    const f32x4 Ya = mfma32(fk.pt[0], d0, zero4());
    const f32x4 Yb = mfma32(fk.pt[1], d0, zero4());
    // S_{c+1} = e^{gam_c} S + KR_c^T delta_c
#pragma unroll
    for (int t = 0; t < NKH; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] *= eg0[t][i];
        S[t] = mfma32(fk.kr0[t], d0, S[t]);
    }
    f16x4 d1a, d1b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d1a[i] = (_Float16)(-((X[2][i] + Po[2][i]) + Ya[i]));
        d1b[i] = (_Float16)(-((X[3][i] + Po[3][i]) + Yb[i]));
    }
    if constexpr (h == 0) {
        ho.dh[par][0][lane] = d0a;
        ho.dh[par][1][lane] = d0b;
        ho.dh[par][2][lane] = d1a;
        ho.dh[par][3][lane] = d1b;
    }
#pragma unroll
    for (int j = 0; j < NSH; ++j)
        ho.sh[slot][1][h * NSH + j][lane] = cat(to_f16x4(S[2 * j]), to_f16x4(S[2 * j + 1]));
    // S_{c+2} = e^{gam_{c+1}} S_{c+1} + KR_{c+1}^T delta_{c+1}
    const f16x8 d1 = cat(d1a, d1b);
#pragma unroll
    for (int t = 0; t < NKH; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] *= eg1[t][i];
        S[t] = mfma32(fk.kr1[t], d1, S[t]);
    }
    nxk.template load_k<h>(fk);
}

template <int K, int V, int h, int AUX>
__device__ __forceinline__ void chain64_step(PairFragW<K, V> &fw, PairFragK<K, V> &fk,
                                             const Pair64<K, V, AUX> &nxw,
                                             const Pair64<K, V, AUX> &nxk, f32x4 (&S)[K / 32],
                                             Handoff64<K> &ho, int m, int par, int lane)
{
    f32x4 X[4], eg0[K / 32], eg1[K / 32];
    // independent of S: scheduled into the exchange's products
    expand_rows(fk.egr0, eg0);
    expand_rows(fk.egr1, eg1);
    chain64_a<K, V, h>(fw, S, X, ho, m % 3, par, lane);
    chain64_b<K, V, h, AUX>(fw, fk, eg0, eg1, nxw, nxk, S, X, ho, m % 3, par, lane);
}

// Chain wave h over the whole sequence: S rows [K/2 h, K/2 (h + 1)) from initial_state (or 0),
// the pair loop, barrier np, and the final state.
template <int K, int V, int h, int AUX, bool TWOK>
__device__ __forceinline__ void chain64_wave(const FwdParams &p, Handoff64<K> &ho,
                                             const uint8_t *base, int np, int s, int j, int col,
                                             int slice, int lane)
{
    constexpr int NKH = K / 32;
    using WP = WsPair<K, V>;
    const int grp = lane >> 4;
    const int row0 = h * (K / 2);
    auto at = [&](int m) {
        return Pair64<K, V, AUX>{
            buffer_rsrc(base + (size_t)min(m, np - 1) * 2 * WP::BYTES, 2 * WP::BYTES), lane,
            slice};
    };
    f32x4 S[NKH];
    if (p.h0) {
        const float *h0 = p.h0 + ((size_t)s * p.HV + j) * (size_t)K * V + col;
#pragma unroll
        for (int t = 0; t < NKH; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[t][i] = h0[(size_t)(row0 + 16 * t + 4 * grp + i) * V];
    } else {
#pragma unroll
        for (int t = 0; t < NKH; ++t) S[t] = zero4();
    }
    if (np > 0) {
        PairFragW<K, V> wa, wb;
        at(0).template load_w<h>(wa);
        at(1).template load_w<h>(wb);
        int m = 0;
        if constexpr (TWOK) {
            // both groups in two register sets, every load two pairs ahead
            PairFragK<K, V> ka, kb;
            at(0).template load_k<h>(ka);
            at(1).template load_k<h>(kb);
            vm_drain();
            for (; m + 2 <= np; m += 2) {
                chain64_step<K, V, h, AUX>(wa, ka, at(m + 2), at(m + 2), S, ho, m, 0, lane);
                chain64_step<K, V, h, AUX>(wb, kb, at(m + 3), at(m + 3), S, ho, m + 1, 1, lane);
            }
            if (m < np)
                chain64_step<K, V, h, AUX>(wa, ka, at(m + 2), at(m + 2), S, ho, m, 0, lane);
        } else {
            PairFragK<K, V> fk;
            at(0).template load_k<h>(fk);
            // drain the prologue loads: the loop header then carries only the loop's own
            // pending loads, and the waits inside the loop count back to the right group
            vm_drain();
            // no exit between the loop body's two steps (see kda_state32.h)
            for (; m + 2 <= np; m += 2) {
                chain64_step<K, V, h, AUX>(wa, fk, at(m + 2), at(m + 1), S, ho, m, 0, lane);
                chain64_step<K, V, h, AUX>(wb, fk, at(m + 3), at(m + 2), S, ho, m + 1, 1, lane);
            }
            if (m < np)
                chain64_step<K, V, h, AUX>(wa, fk, at(m + 2), at(m + 1), S, ho, m, 0, lane);
        }
        lds_barrier();    // barrier np: the deltas and S_{c+1} of the last pair are handed over
    }
    if (p.ht) {
        float *ht = p.ht + ((size_t)s * p.HV + j) * (size_t)K * V + col;
#pragma unroll
        for (int t = 0; t < NKH; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ht[(size_t)(row0 + 16 * t + 4 * grp + i) * V] = S[t][i];
    }
}

// Output wave k, pair m, after barrier m + 1: o of the pair's chunk k (rows 32 k .. 32 k + 31)
// from QD, Mqk, the fp16 state at that chunk's start and its delta, as two 16-row blocks
// transposed on the matrix core to row segments and stored as bf16. `nxt` is the pair two
// steps ahead.
template <int K, int V, int AUX, int k>
__device__ __forceinline__ void out_step64(PairOutFrag<K, V> &f, const Pair64<K, V, AUX> &nxt,
                                           const Handoff64<K> &ho, int slot, int par, int lane,
                                           __amdgpu_buffer_rsrc_t orows, const int (&ooff)[4],
                                           bf16x4 Ib)
{
    constexpr int NS = K / 32;
    lds_barrier();
    f16x8 Sh[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) Sh[st] = ho.sh[slot][k][st][lane];
    const f16x4 da = ho.dh[par][2 * k][lane], db = ho.dh[par][2 * k + 1][lane];
    f32x4 Y0 = zero4(), Y1 = zero4();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        Y0 = mfma32(f.qd[0][st], Sh[st], Y0);
        Y1 = mfma32(f.qd[1][st], Sh[st], Y1);
    }
    // block a's Mqk product in the 16x16x32 shape of the products it accumulates onto (see
    // the output step of kda_state32.h)
    const f16x8 d32 = cat(da, db);
    const f32x4 O0 = mfma32(cat(f.mqa, f16x4{0, 0, 0, 0}), d32, Y0);
    const f32x4 O1 = mfma32(f.mqb, d32, Y1);
    nxt.template load_out<k>(f);
    const bf16x4 T0 = to_bf16x4(mfma16(to_bf16x4(O0), Ib, zero4()));
    const bf16x4 T1 = to_bf16x4(mfma16(to_bf16x4(O1), Ib, zero4()));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, T0), orows, ooff[2 * k], 0,
                                          0);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, T1), orows,
                                          ooff[2 * k + 1], 0, 0);
}

// The output wave of chunk k of every pair (see out_step64).
template <int K, int V, int AUX, int k>
__device__ __forceinline__ void out_wave64(const FwdParams &p, const Handoff64<K> &ho,
                                           const uint8_t *base, int np, int64_t bos, int64_t eos,
                                           int j, int slice, int lane)
{
    constexpr int CT = 64;
    using WP = WsPair<K, V>;
    const int grp = lane >> 4, n = lane & 15;
    auto at = [&](int m) {
        return Pair64<K, V, AUX>{
            buffer_rsrc(base + (size_t)min(m, np - 1) * 2 * WP::BYTES, 2 * WP::BYTES), lane,
            slice};
    };
    const int64_t row_bytes = (int64_t)p.HV * V * 2, head_bytes = (int64_t)j * V * 2;
    // after the transposing product lane (g, n) holds row n of each 16-row block, columns
    // 16 slice + 4g .. + 3
    const int ocol = 16 * slice + 4 * grp;
    int ooff[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) ooff[b] = (int)((16 * b + n) * row_bytes + ocol * 2);
    float eye[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = 4 * grp + i == n ? 1.f : 0.f;
    const bf16x4 Ib = to_bf16x4(eye);
    auto rows = [&](int m) {
        // range ends after the pair's last valid token: later rows' stores are dropped
        const int64_t r0 = bos + CT * m;
        const int64_t nv = eos - r0;
        uint8_t *ob = (uint8_t *)p.o + r0 * row_bytes + head_bytes;
        const int num = (int)((nv < CT ? nv : CT) * row_bytes - head_bytes);
        return __builtin_amdgcn_make_buffer_rsrc(ob, 0, num, 0x00020000);
    };
    PairOutFrag<K, V> fa, fb;
    at(0).template load_out<k>(fa);
    at(1).template load_out<k>(fb);
    vm_drain();
    lds_barrier();        // barrier 0
    int m = 0;
    for (; m + 2 <= np; m += 2) {
        out_step64<K, V, AUX, k>(fa, at(m + 2), ho, m % 3, 0, lane, rows(m), ooff, Ib);
        out_step64<K, V, AUX, k>(fb, at(m + 3), ho, (m + 1) % 3, 1, lane, rows(m + 1), ooff, Ib);
    }
    if (m < np) out_step64<K, V, AUX, k>(fa, at(m + 2), ho, m % 3, 0, lane, rows(m), ooff, Ib);
}

// Barrier schedule for np pairs: every wave passes np + 1 barriers. Barrier m (m < np) follows
// the chain waves' hand-off of pair m's first half (fp16 S_c in slot m % 3 and the partials in
// parity m % 2); between barriers m and m + 1 the chain waves form both deltas (half 0 writes
// them to parity m % 2), S_{c+1} (fp16 rows to slot m % 3) and S_{c+2}, then pair m + 1's
// hand-off; the output waves, after barrier m + 1, read slot m % 3 and the deltas of parity
// m % 2. Slot m % 3 is rewritten at pair m + 3, the partials at pair m + 2 (before barrier
// m + 2, once the other half has read them after barrier m) and the deltas at pair m + 2
// (after barrier m + 2, once the output waves have read them).

// One V-slice (16 columns of S and o) of one (sequence, value head) unit, as four waves: roles
// 0 and 1 are the chain halves, roles 2 and 3 the output waves of the first and second chunk
// of each pair; every role passes the same barriers.
// TWOK: the chain waves keep two register sets of every operand group (all loads two pairs
// ahead; more registers, one wave per SIMD) instead of one set of the post-exchange group.
template <int K, int V, int AUX, bool TWOK>
__device__ __forceinline__ void state64_slice(const FwdParams &p, Handoff64<K> &ho, int unit,
                                              int slice, int role, int lane)
{
    constexpr int CT = 64;
    using WP = WsPair<K, V>;
    const int grp = lane >> 4, n = lane & 15;
    const int j = unit % p.HV;
    const int s = unit / p.HV;
    const int64_t bos = seq_bos(p.seq, s);
    const int64_t eos = seq_eos(p.seq, s, bos);
    const int np = (int)((eos - bos + CT - 1) / CT);
    const int col = 16 * slice + n;
    const uint8_t *base =
        p.ws + ((size_t)j * 2 * p.seq.n_slots + 2 * (size_t)(bos / CT + s)) * (size_t)WP::BYTES;
    if (role == 0) {
        chain64_wave<K, V, 0, AUX, TWOK>(p, ho, base, np, s, j, col, slice, lane);
    } else if (role == 1) {
        chain64_wave<K, V, 1, AUX, TWOK>(p, ho, base, np, s, j, col, slice, lane);
    } else if (np > 0) {
        if (role == 2)
            out_wave64<K, V, AUX, 0>(p, ho, base, np, bos, eos, j, slice, lane);
        else
            out_wave64<K, V, AUX, 1>(p, ho, base, np, bos, eos, j, slice, lane);
    }
}

}  // namespace

}  // namespace kda
