// kda_state32.h -- stage 2 with 32-token chunks: the chunk-sequential state pass, one serial
// step per 32 tokens.
//
// Per chunk, with S the K x V state at the chunk start ("手撕KDA" section 1, chunk loop of
// naive_chunk_kda, here with chunk 32):
//     delta = U - W S                      (32 x V)
//     o     = QD S + Mqk delta             (32 x V), rows past the sequence end not stored
//     S    <- diag(e^{gam}) S + KR^T delta
//
// Per (sequence, value head, 16-column slice of V) two chain waves that each own half of the
// key rows of S (fp32 registers), and an output wave. With several slices of a unit in one
// workgroup an output wave, and with four a chain wave too, serves two slices, whose operands
// are the same but for -U (kda_state32.hip).
// A chain step is split where the contraction over the key dimension allows it: each chain
// wave forms its half of W S from its fp16 rows and hands the 32 x 16 fp32 partial to the
// other through LDS; after the step's barrier both add the two partials (in the same order of
// operands, so both hold the same delta), and each updates its own rows. The per-step VMEM,
// VALU and MFMA work of one chain wave is half of a single-wave chain's, which is what bounds
// the step: the serial path per 32 tokens is one LDS exchange, four update MFMAs and four W S
// MFMAs. The output wave computes o for chunk c one barrier later, from the fp16 copy of S
// the chain waves wrote and delta.
//
// Fragments are loaded two chunks ahead through buffer resources (scalar base = the chunk
// record, clamped to the last chunk), in the lane order the prepare kernel wrote them.
#pragma once

#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ bool state_unit32(int wg, int NV, int units, int *unit, int *slice) {
    // all V/16 slices of one (sequence, value head) on one XCD (dispatch is round-robin over
    // the 8 XCDs, each with its own L2), so they share the chunk operands in L2
    const int xcd = wg & 7, idx = wg >> 3;
    *unit = (idx / NV) * 8 + xcd;
    *slice = idx % NV;
    return *unit < units;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(void *o, int64_t row0, int nvalid,
                                                            int64_t row_bytes,
                                                            int64_t head_bytes) {
    // range ends after the last valid token: stores to later rows are dropped by the hardware
    uint8_t *base = (uint8_t *)o + row0 * row_bytes + head_bytes;
    const int num = (int)(nvalid * row_bytes - head_bytes);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, num, 0x00020000);
}

// Operands of one chunk for the chain wave that owns key rows [K/2 h, K/2 (h + 1)).
template <int K, int V, int CS = 1>
struct HalfFrag {
    static constexpr int NSH = K / 64, NKH = K / 32;   // 32-row slabs and 16-row tiles owned
    f16x8 w[2][NSH];          // W rows of blocks a and b, this half's columns
    f16x8 kr[NKH];            // KR^T tiles of this half over the 32 tokens
    f32x4 eg[NKH];            // exp(gam) of the four rows 16t + 4g + i each lane holds
    float e1;                 // exp(gam) of row K/2 h + lane % (K/2) as loaded; it reaches eg
                              // through this wave's LDS stage one step later (stage_eg)
    f16x8 nu[CS];             // -U of blocks a (0..3) and b (4..7) of each slice (half 0 only)
};

template <int K, int V>
struct OutFrag32 {
    f16x8 qd[2][K / 32];
    f16x4 mqa;
    f16x8 mqb;
};

// One chunk record seen through a buffer resource (scalar base = the record); field offsets
// are scalar constants and the per-lane part is lane * size.
// AUX is the cache policy of the loads.
template <int K, int V, int AUX = 0>
struct Chunk32 {
    using WS = WsBf16x32<K, V>;
    static constexpr int NS = K / 32, NV = V / 16;
    static constexpr int NSH = HalfFrag<K, V>::NSH, NKH = HalfFrag<K, V>::NKH;
    __amdgpu_buffer_rsrc_t rs;
    int lane, slice;
    template <int h, int CS, bool IDN = false>
    __device__ __forceinline__ void load_w(HalfFrag<K, V, CS> &f) const {
        // first, so that waiting for it (one step later) waits for no load issued after it
        f.e1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rs, (lane % (K / 2)) * 4, WS::EG + h * (K / 2) * 4,
                                             AUX));
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < NSH; ++j)
                f.w[b][j] = __builtin_bit_cast(
                    f16x8, bload16<AUX>(rs, lane * 16, WS::W + (b * NS + h * NSH + j) * 1024));
        if constexpr (h == 0 && !IDN) {
#pragma unroll
            for (int q = 0; q < CS; ++q)
                f.nu[q] = __builtin_bit_cast(
                    f16x8, bload16<AUX>(rs, lane * 16, WS::NU + (slice + q) * 1024));
        }
    }
    template <int h, int CS>
    __device__ __forceinline__ void load_kreg(HalfFrag<K, V, CS> &f) const {
#pragma unroll
        for (int t = 0; t < NKH; ++t)
            f.kr[t] = __builtin_bit_cast(f16x8,
                                         bload16<AUX>(rs, lane * 16, WS::KR + (h * NKH + t) * 1024));
    }
    __device__ __forceinline__ void load_out(OutFrag32<K, V> &f) const {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int st = 0; st < NS; ++st)
                f.qd[b][st] = __builtin_bit_cast(f16x8, bload16<AUX>(rs, lane * 16,
                                                                WS::QD + (b * NS + st) * 1024));
        f.mqa = __builtin_bit_cast(f16x4, bload8<AUX>(rs, lane * 8, WS::MQKA));
        f.mqb = __builtin_bit_cast(f16x8, bload16<AUX>(rs, lane * 16, WS::MQKB));
    }
};

template <int K>
struct Handoff32 {
    f16x8 sh[3][K / 32][64];     // S (fp16) of chunk c in slot c % 3
    f32x4 xp[2][2][2][64];       // [chunk parity][half][block] partial W S (half 0: + (-U))
    f16x4 dh[2][2][64];          // [chunk parity][block] delta
    float egs[2][64];            // [half] exp(gam) of the chain wave's rows, on their way from
                                 // one value per lane to the four-rows-per-lane tiles of eg
};

// exp(gam) of the fragment `o` from one value per lane (o.e1, row K/2 h + lane) to the C-layout
// rows each lane decays (rows 16t + 4g .. + 3 of tile t, the same for the 16 lanes of a group):
// through this wave's own LDS stage, whose write and reads are ordered by the wave's LDS queue.
// A 16-byte load per tile had fetched every value 16 times through the CU's vector-memory path,
// a quarter of the chain waves' operand traffic (46.4 -> 45.5 us at 16 heads x 4096 tokens,
// 0.465 -> 0.428 ms at 4 x 8192 tokens x 32 value heads).
template <int K, int V, int h, int CS>
__device__ __forceinline__ void stage_eg(HalfFrag<K, V, CS> &o, Handoff32<K> &ho, int lane)
{
    ho.egs[h][lane] = o.e1;
#pragma unroll
    for (int t = 0; t < K / 32; ++t)
        o.eg[t] = *(const f32x4 *)&ho.egs[h][16 * t + 4 * (lane >> 4)];
}

// Chain wave h, one 32-token chunk c (S = its rows of the state at the chunk start), up to
// and including barrier c: fp16 rows to the hand-off and the partial of W S to the other half;
// the decay of its rows by e^{gam} fills the W S products' latency. No load precedes the
// barrier (loads issued here delayed both halves' arrival: 46.3 -> 47.9 us at 16 x 4096).
template <int K, int V, int h, int CS, bool IDN>
__device__ __forceinline__ void chain_half_a(const HalfFrag<K, V, CS> &f,
                                             f32x4 (&S)[CS][K / 32], f32x4 (&Xa)[CS],
                                             f32x4 (&Xb)[CS], Handoff32<K> *ho, int slot,
                                             int par, int lane)
{
    constexpr int NSH = K / 64;
#pragma unroll
    for (int q = 0; q < CS; ++q) {
        if constexpr (h == 0 && !IDN) {
            // -U of both blocks is stored in the B layout of a 16x16x16 product (lane (n, g):
            // rows 4g .. 4g + 3 of column n), so the identity times it is -U in C layout,
            // exactly: two matrix-core products instead of eight conversions in this wave's
            // stream. They are 16x16x32 products (the four upper k of each lane zero), the
            // W S products' own shape: copies that fed a 16x16x16 result into a 16x16x32
            // accumulator four or five instructions later computed wrong sums (the compiler's
            // wait for that pair is too short on this part); tests/test_codegen.py keeps the
            // pair out of the library.
            const int n = lane & 15, g = lane >> 4;
            f16x8 ih;
#pragma unroll
            for (int i = 0; i < 8; ++i) ih[i] = (_Float16)(i < 4 && 4 * g + i == n ? 1.f : 0.f);
            const f16x4 z = {0, 0, 0, 0};
            Xa[q] = mfma32(ih, cat(__builtin_shufflevector(f.nu[q], f.nu[q], 0, 1, 2, 3), z),
                           zero4());
            Xb[q] = mfma32(ih, cat(__builtin_shufflevector(f.nu[q], f.nu[q], 4, 5, 6, 7), z),
                           zero4());
        } else {
            Xa[q] = zero4();
            Xb[q] = zero4();
        }
    }
#pragma unroll
    for (int j = 0; j < NSH; ++j)
#pragma unroll
        for (int q = 0; q < CS; ++q) {
            const f16x8 Sh = cat(to_f16x4(S[q][2 * j]), to_f16x4(S[q][2 * j + 1]));
            ho[q].sh[slot][h * NSH + j][lane] = Sh;
            Xa[q] = mfma32(f.w[0][j], Sh, Xa[q]);
            Xb[q] = mfma32(f.w[1][j], Sh, Xb[q]);
        }
    // the decay behind every W S product (left to itself the compiler put some of it ahead of
    // the first product, on the chain: 45.3 against 46.4 us at 16 heads x 4096 tokens)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CS; ++q)
#pragma unroll
        for (int t = 0; t < K / 32; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[q][t][i] *= f.eg[t][i];
#pragma unroll
    for (int q = 0; q < CS; ++q) {
        ho[q].xp[par][h][0][lane] = Xa[q];
        ho[q].xp[par][h][1][lane] = Xb[q];
    }
    lds_barrier();
}

// Chain wave h after barrier c: the other half's partial is read first, and the refill of the
// W / exp(gam) / -U group from `nxt` (two chunks ahead) is issued in its LDS latency; then
// delta = -(own partial + other partial) (half 0 hands it to the output wave) and the update of
// its rows; the KR^T group is refilled last, and the other fragment `o` (the next chunk's) gets
// its exp(gam) tiles from its staged value. The scheduling barriers keep the compiler from
// moving the refills between the update products, where their issue delayed the next step
// (48.8 -> 46.3 us per launch at 16 x 4096, 0.474 -> 0.461 ms at 4 x 8192 x 32 heads).
template <int K, int V, int h, int AUX, int CS, bool IDN>
__device__ __forceinline__ void chain_half_b(HalfFrag<K, V, CS> &f, HalfFrag<K, V, CS> &o,
                                             const Chunk32<K, V, AUX> &nxt,
                                             f32x4 (&S)[CS][K / 32], const f32x4 (&Xa)[CS],
                                             const f32x4 (&Xb)[CS], Handoff32<K> *ho, int par,
                                             int lane)
{
    constexpr int NKH = K / 32;
    f32x4 Pa[CS], Pb[CS];
#pragma unroll
    for (int q = 0; q < CS; ++q) {
        Pa[q] = ho[q].xp[par][1 - h][0][lane];
        Pb[q] = ho[q].xp[par][1 - h][1][lane];
    }
    __builtin_amdgcn_sched_barrier(0);
    nxt.template load_w<h, CS, IDN>(f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CS; ++q) {
        f16x4 dh0, dh1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // half 0 adds (own + other) and half 1 (other + own): the same two fp32 operands,
            // so both halves round to the same delta
            dh0[i] = (_Float16)(-(Xa[q][i] + Pa[q][i]));
            dh1[i] = (_Float16)(-(Xb[q][i] + Pb[q][i]));
        }
        if constexpr (h == 0) {
            ho[q].dh[par][0][lane] = dh0;
            ho[q].dh[par][1][lane] = dh1;
        }
        const f16x8 d32 = cat(dh0, dh1);
#pragma unroll
        for (int t = 0; t < NKH; ++t) S[q][t] = mfma32(f.kr[t], d32, S[q][t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    nxt.template load_kreg<h, CS>(f);
    __builtin_amdgcn_sched_barrier(0);
    stage_eg<K, V, h, CS>(o, ho[0], lane);     // the next chunk's exp(gam), loaded one step ago
}

template <int K, int V, int h, int AUX, int CS, bool IDN>
__device__ __forceinline__ void chain_step(HalfFrag<K, V, CS> &f, HalfFrag<K, V, CS> &o,
                                           const Chunk32<K, V, AUX> &nxt,
                                           f32x4 (&S)[CS][K / 32], Handoff32<K> *ho, int c,
                                           int par, int lane)
{
    f32x4 Xa[CS], Xb[CS];
    chain_half_a<K, V, h, CS, IDN>(f, S, Xa, Xb, ho, c % 3, par, lane);
    chain_half_b<K, V, h, AUX, CS, IDN>(f, o, nxt, S, Xa, Xb, ho, par, lane);
}

// Chain wave h of CS consecutive slices (slice ..) over nc chunks from `base`: their S rows
// [K/2 h, K/2 (h + 1)) from h0u (the unit's K x V initial state, or 0 when null), the chunk
// loop, barrier nc, and the state at the end to htu (when not null). The slices share every
// operand but -U, so one wave serving two loads W, KR and e^gam once for both.
// IDN: the slices are 16-column slices of the K x K transition instead: S starts from the
// identity (row == column) and U is taken as 0, so the chain runs the homogeneous recurrence
// S <- (diag(e^gam) - KR^T W) S.
// FIN says how the end state goes out (CS = 1 for the two fragment forms):
//   FIN_ROWS  fp32 rows of the unit's K x V state at htu;
//   FIN_BFRAG the 16x16x32 B operands of the slice in fp16 (Split32::smf, the unit's
//             fragments at htu: [V/16][K/32][64][8]);
//   FIN_TTILE each 16 x 16 tile transposed, in fp16 (Split32::phf, [K/16][K/16][64][4]).
enum { FIN_ROWS = 0, FIN_BFRAG = 1, FIN_TTILE = 2 };

template <int K, int V, int h, int AUX, int CS, bool IDN = false, int FIN = FIN_ROWS>
__device__ __forceinline__ void chain_wave(Handoff32<K> *ho, const uint8_t *base, int nc,
                                           const float *h0u, void *htu, int slice, int lane)
{
    constexpr int NKH = K / 32;
    using WS = WsBf16x32<K, V>;
    const int grp = lane >> 4;
    const int row0 = h * (K / 2);
    auto at = [&](int c) {
        return Chunk32<K, V, AUX>{
            buffer_rsrc(base + (size_t)min(c, nc - 1) * WS::BYTES, WS::BYTES), lane, slice};
    };
    f32x4 S[CS][NKH];
#pragma unroll
    for (int q = 0; q < CS; ++q) {
        const int col = 16 * (slice + q) + (lane & 15);
        if (IDN) {
#pragma unroll
            for (int t = 0; t < NKH; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[q][t][i] = row0 + 16 * t + 4 * grp + i == col ? 1.f : 0.f;
        } else if (h0u) {
            const float *h0 = h0u + col;
#pragma unroll
            for (int t = 0; t < NKH; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[q][t][i] = h0[(size_t)(row0 + 16 * t + 4 * grp + i) * V];
        } else {
#pragma unroll
            for (int t = 0; t < NKH; ++t) S[q][t] = zero4();
        }
    }
    if (nc > 0) {
        HalfFrag<K, V, CS> fa, fb;
        at(0).template load_w<h, CS, IDN>(fa); at(0).template load_kreg<h, CS>(fa);
        at(1).template load_w<h, CS, IDN>(fb); at(1).template load_kreg<h, CS>(fb);
        // drain the prologue loads: the loop header then carries only the loop's own pending
        // loads, and the waits inside the loop count back to the right group
        vm_drain();
        stage_eg<K, V, h, CS>(fa, ho[0], lane);    // chunk 1's is staged by step 0
        // no exit between the loop body's two steps: an exit there would merge a half-step
        // state into the loop header and make every iteration wait for the loads just issued
        int c = 0;
        for (; c + 2 <= nc; c += 2) {
            chain_step<K, V, h, AUX, CS, IDN>(fa, fb, at(c + 2), S, ho, c, 0, lane);
            chain_step<K, V, h, AUX, CS, IDN>(fb, fa, at(c + 3), S, ho, c + 1, 1, lane);
        }
        if (c < nc) chain_step<K, V, h, AUX, CS, IDN>(fa, fb, at(c + 2), S, ho, c, 0, lane);
        lds_barrier();    // barrier nc: delta of the last chunk is in the hand-off
    }
    if (!htu) return;
    if constexpr (FIN == FIN_ROWS) {
#pragma unroll
        for (int q = 0; q < CS; ++q) {
            const int col = 16 * (slice + q) + (lane & 15);
            float *ht = (float *)htu + col;
#pragma unroll
            for (int t = 0; t < NKH; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ht[(size_t)(row0 + 16 * t + 4 * grp + i) * V] = S[q][t][i];
        }
    } else if constexpr (FIN == FIN_BFRAG) {
        // the hand-off's own operand: slab h K/64 + j pairs tiles 2j, 2j + 1 of this half
        const __amdgpu_buffer_rsrc_t fr = buffer_rsrc(htu, (uint32_t)(K * V * 2));
#pragma unroll
        for (int j = 0; j < K / 64; ++j) {
            const int at = (slice * (K / 32) + h * (K / 64) + j) * 64 + lane;
            bstore16<0>(fr, at * 16, 0, cat(to_f16x4(S[0][2 * j]), to_f16x4(S[0][2 * j + 1])));
        }
    } else {
        // C(X^T) of each tile by the identity product: lane (g, n) then holds row n of the
        // tile, columns 4g .. 4g + 3 (fp16 values, so the product is exact)
        f16x4 Ih;
#pragma unroll
        for (int i = 0; i < 4; ++i) Ih[i] = (_Float16)(4 * grp + i == (lane & 15) ? 1.f : 0.f);
        const __amdgpu_buffer_rsrc_t fr = buffer_rsrc(htu, (uint32_t)(K * K * 2));
#pragma unroll
        for (int t = 0; t < NKH; ++t) {
            const int rt = h * NKH + t;
            bstore8<0>(fr, ((rt * (K / 16) + slice) * 64 + lane) * 8, 0,
                       to_f16x4(mfma16(to_f16x4(S[0][t]), Ih, zero4())));
        }
    }
}

// Barrier schedule for nc chunks: every wave passes nc + 1 barriers. Barrier c (c < nc)
// follows the chain waves' hand-off of chunk c (fp16 rows of S in slot c % 3, the W S
// partials in slot c % 2); between barriers c and c+1 the chain waves form delta_c (half 0
// writes it to slot c % 2) and update S, then write chunk c+1's hand-off; the output wave,
// after barrier c+1, reads the fp16 rows and delta_c. The fp16 rows are rewritten three
// chunks later (after barrier c+2), the partials and delta two chunks later (after barrier
// c+1 and c+2 respectively), each after its readers are done. The chain waves pass barrier nc
// after their last update.

// The record base and chunk count of one (sequence, value head) unit.
template <int K, int V, int AUX>
struct Unit32 {
    using WS = WsBf16x32<K, V>;
    int j, s, nc;
    int64_t bos, eos;
    const uint8_t *base;
    __device__ Unit32(const FwdParams &p, int unit) {
        j = unit % p.HV;
        s = unit / p.HV;
        bos = seq_bos(p.seq, s);
        eos = seq_eos(p.seq, s, bos);
        nc = (int)((eos - bos + 31) / 32);
        base = p.ws + ((size_t)j * p.seq.n_slots + (size_t)(bos / 32 + s)) * (size_t)WS::BYTES;
    }
    __device__ Chunk32<K, V, AUX> at(int c, int lane, int slice) const {
        return Chunk32<K, V, AUX>{
            buffer_rsrc(base + (size_t)min(c, nc - 1) * WS::BYTES, WS::BYTES), lane, slice};
    }
};

// Output wave, chunk c, after barrier c + 1, for OPW slices of one unit (handoffs ho[0 ..]):
// o = QD S + Mqk delta of each, handed to store(q, C(O_a^T), C(O_b^T)) per slice q (blocks a
// and b). The QD / Mqk operands are the same for every slice of the unit, so an output wave
// serving two slices loads them once.
template <int K, int V, int AUX, int OPW, class STORE>
__device__ __forceinline__ void out_step32(OutFrag32<K, V> &f, const Chunk32<K, V, AUX> &nxt,
                                           const Handoff32<K> *ho, int slot, int par, int lane,
                                           const STORE &store)
{
    constexpr int NS = K / 32;
    lds_barrier();
    f32x4 O0[OPW], O1[OPW];
#pragma unroll
    for (int q = 0; q < OPW; ++q) {
        f16x8 Sh[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) Sh[st] = ho[q].sh[slot][st][lane];
        const f16x4 dh0 = ho[q].dh[par][0][lane], dh1 = ho[q].dh[par][1][lane];
        // Each product takes its operands in swapped roles, so it forms the transpose of the
        // block's output: (A B)^T = B^T A^T, and the A operand registers of a matrix are the B
        // operand registers of its transpose. C(O^T) holds four consecutive columns of one
        // token row per lane, the layout of an 8-byte row store.
        f32x4 Y0 = zero4(), Y1 = zero4();
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            Y0 = mfma32(Sh[st], f.qd[0][st], Y0);
            Y1 = mfma32(Sh[st], f.qd[1][st], Y1);
        }
        // both blocks accumulate onto the 16x16x32 products with a 16x16x32 product (block a's
        // Mqk in the lower four k of each lane, zeros above): a 16x16x16 product taking a
        // 16x16x32 result as its accumulator a few instructions later read it too early
        const f16x8 d32 = cat(dh0, dh1);
        O0[q] = mfma32(d32, cat(f.mqa, f16x4{0, 0, 0, 0}), Y0);
        O1[q] = mfma32(d32, f.mqb, Y1);
    }
    nxt.load_out(f);
#pragma unroll
    for (int q = 0; q < OPW; ++q) store(q, O0[q], O1[q]);
}

// Stores of one chunk of o as bf16 rows: lane (g, n) of C(O^T) holds token n (block a) /
// 16 + n (block b), columns 16 slice + 4g .. + 3, one 8-byte store per block.
template <int OPW>
struct RowStore32 {
    __amdgpu_buffer_rsrc_t orows;
    const int (&ooff)[OPW][2];
    __device__ __forceinline__ void operator()(int q, f32x4 Oa, f32x4 Ob) const {
        const bf16x4 T0 = to_bf16x4(Oa);
        const bf16x4 T1 = to_bf16x4(Ob);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, T0), orows, ooff[q][0],
                                              0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, T1), orows, ooff[q][1],
                                              0, 0);
    }
};

// Chain half h of CS consecutive V-slices (slice ..) of one unit, with hand-offs ho[0 ..].
// AUX is the cache policy of the workspace loads.
template <int K, int V, int AUX, int CS>
__device__ __forceinline__ void state32_chain(const FwdParams &p, Handoff32<K> *ho,
                                              const Unit32<K, V, AUX> &u, int slice, int h,
                                              int lane)
{
    const size_t st = ((size_t)u.s * p.HV + u.j) * (size_t)K * V;
    const float *h0u = p.h0 ? p.h0 + st : nullptr;
    float *htu = p.ht ? p.ht + st : nullptr;
    if (h == 0)
        chain_wave<K, V, 0, AUX, CS>(ho, u.base, u.nc, h0u, htu, slice, lane);
    else
        chain_wave<K, V, 1, AUX, CS>(ho, u.base, u.nc, h0u, htu, slice, lane);
}

// The output wave of OPW consecutive V-slices (slice0 ..) of one unit, whose hand-offs are
// ho[0 .. OPW - 1]; it passes the same barriers as their chain waves.
template <int K, int V, int AUX, int OPW>
__device__ __forceinline__ void state32_out(const FwdParams &p, const Handoff32<K> *ho,
                                            const Unit32<K, V, AUX> &u, int slice0, int lane)
{
    constexpr int CT = 32;
    if (u.nc == 0) return;
    const int grp = lane >> 4, n = lane & 15;
    const int64_t row_bytes = (int64_t)p.HV * V * 2, head_bytes = (int64_t)u.j * V * 2;
    // the output products leave lane (g, n) with row n (block a) / 16 + n (block b), columns
    // 16 slice + 4g .. + 3
    int ooff[OPW][2];
#pragma unroll
    for (int q = 0; q < OPW; ++q) {
        const int ocol = 16 * (slice0 + q) + 4 * grp;
        ooff[q][0] = (int)(n * row_bytes + ocol * 2);
        ooff[q][1] = (int)((16 + n) * row_bytes + ocol * 2);
    }
    auto rows = [&](int c) {
        const int64_t r0 = u.bos + CT * c;
        const int64_t nv = u.eos - r0;
        return rows_rsrc(p.o, r0, (int)(nv < CT ? nv : CT), row_bytes, head_bytes);
    };
    const int nc = u.nc;
    OutFrag32<K, V> fa, fb;
    u.at(0, lane, slice0).load_out(fa);
    u.at(1, lane, slice0).load_out(fb);
    vm_drain();
    lds_barrier();        // barrier 0
    int c = 0;
    for (; c + 2 <= nc; c += 2) {
        out_step32<K, V, AUX, OPW>(fa, u.at(c + 2, lane, slice0), ho, c % 3, 0, lane,
                                   RowStore32<OPW>{rows(c), ooff});
        out_step32<K, V, AUX, OPW>(fb, u.at(c + 3, lane, slice0), ho, (c + 1) % 3, 1, lane,
                                   RowStore32<OPW>{rows(c + 1), ooff});
    }
    if (c < nc)
        out_step32<K, V, AUX, OPW>(fa, u.at(c + 2, lane, slice0), ho, c % 3, 0, lane,
                                   RowStore32<OPW>{rows(c), ooff});
}

// Segment B of the two-segment pass (Split32): the stores of one chunk for the slice pair of
// a workgroup, slice q = 0 the value slice (its output from a zero state, C(O^T)) and q = 1
// the same-numbered 16-column slice of the transition (C(Y^T)). Both go to the unit's scratch
// in fp16 as 64-lane fragments, chunk c block b at [c][b][slice][lane]. fp16 keeps 11
// significant bits, so o0 rounded there moves o by at most 2^-12 of its magnitude before the
// correction's one bf16 rounding; its range is that of the chain's own fp16 S and delta.
template <int K, int V>
struct SplitStore32 {
    __amdgpu_buffer_rsrc_t o0, y;
    int c, slice, lane;
    __device__ __forceinline__ void operator()(int q, f32x4 Oa, f32x4 Ob) const {
        if (q == 0) {
            const int at = ((2 * c) * (V / 16) + slice) * 64 + lane;
            bstore8<0>(o0, at * 8, 0, to_f16x4(Oa));
            bstore8<0>(o0, (at + (V / 16) * 64) * 8, 0, to_f16x4(Ob));
        } else {
            const int at = ((2 * c) * (K / 16) + slice) * 64 + lane;
            bstore8<0>(y, at * 8, 0, to_f16x4(Oa));
            bstore8<0>(y, (at + (K / 16) * 64) * 8, 0, to_f16x4(Ob));
        }
    }
};

// The output wave of a segment-B workgroup (hand-offs ho[0]: the value slice, ho[1]: the
// transition slice); `unit_idx` numbers the unit's scratch.
template <int K, int V>
__device__ __forceinline__ void state32_out_split(const FwdParams &p, const Handoff32<K> *ho,
                                                  const Unit32<K, V, 0> &u, size_t unit_idx,
                                                  int slice, int lane)
{
    const int nc = u.nc;
    if (nc == 0) return;
    const size_t o0_bytes = (size_t)nc * 2 * (V / 16) * 64 * 8;
    const size_t y_bytes = (size_t)nc * 2 * (K / 16) * 64 * 8;
    const __amdgpu_buffer_rsrc_t o0 =
        buffer_rsrc((uint8_t *)p.split.o0 + unit_idx * o0_bytes, (uint32_t)o0_bytes);
    const __amdgpu_buffer_rsrc_t y =
        buffer_rsrc((uint8_t *)p.split.y + unit_idx * y_bytes, (uint32_t)y_bytes);
    OutFrag32<K, V> fa, fb;
    u.at(0, lane, slice).load_out(fa);
    u.at(1, lane, slice).load_out(fb);
    vm_drain();
    lds_barrier();        // barrier 0
    int c = 0;
    for (; c + 2 <= nc; c += 2) {
        out_step32<K, V, 0, 2>(fa, u.at(c + 2, lane, slice), ho, c % 3, 0, lane,
                               SplitStore32<K, V>{o0, y, c, slice, lane});
        out_step32<K, V, 0, 2>(fb, u.at(c + 3, lane, slice), ho, (c + 1) % 3, 1, lane,
                               SplitStore32<K, V>{o0, y, c + 1, slice, lane});
    }
    if (c < nc)
        out_step32<K, V, 0, 2>(fa, u.at(c + 2, lane, slice), ho, c % 3, 0, lane,
                               SplitStore32<K, V>{o0, y, c, slice, lane});
}

}  // namespace

}  // namespace kda
