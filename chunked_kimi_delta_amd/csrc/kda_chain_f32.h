// kda_chain_f32.h -- the chunk-sequential state pass in fp32 on the matrix cores, for the fp32
// forward and for both chains of the backward.
//
// Per chunk of a (sequence, value head), with S the state at the chunk start and the chunk
// record of the prepare kernel ("手撕KDA" section 1, the chunk loop of naive_chunk_kda):
//   forward: delta = u - w S;  o = qd S + Mqk delta;  S <- diag(E) S + kr^T delta
//   states:  the same without o, S recorded at every chunk start (for the backward)
//   grads:   dDelta = Mqk^T dO + kr Lam;  Lam <- diag(E) Lam + qd^T dO - w^T dDelta, newest
//            chunk first from Lam = dht (Lam = d loss / d S), recorded at every chunk end
// Every V column of S and of Lam evolves on its own, so one workgroup owns one 16-column slice
// of one (sequence, value head). Its 4 waves split the K rows: wave w keeps the K/64 tiles of
// 16 rows x 16 columns it owns in fp32 registers (C-layout, which is also the B operand layout
// of the fp32 16x16x4 MFMA, so a tile feeds the products with no data movement between
// lanes). The 16 x 16 products that contract over K (w S, qd S, kr Lam) are summed over the
// waves through LDS, double-buffered by chunk parity so that one barrier per chunk suffices;
// the barrier orders LDS only, so the next chunk's record loads and this chunk's stores stay
// in flight across it.
// S and Lam are recorded per chunk in tile order ([V/16 slice][K/16 tile][64 lanes][4 fp32],
// the C-layout registers as they are), one 1 KB contiguous block per tile and wave, with
// non-temporal stores.
// The chunk records are read as they are laid out ([16][K] row-major w, qd, kr; [16][V] u;
// [16][16] Mqk; [K] E; the backward's copy of dO in C-layout): A-operand rows of w, qd, kr and
// Mqk and the dO tile are contiguous 16-byte loads, the transposes four 4-byte loads. Records
// of the next chunk are loaded before the current chunk's products.
#pragma once

#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ float ldx(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldx(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

enum ChainMode { CHAIN_STATES = 0, CHAIN_GRADS = 1, CHAIN_FORWARD = 2 };
constexpr int CHAIN_WAVES = 4;
constexpr int CK_AUX = 2;          // state-record stores: the non-temporal (nt) cache policy

template <int K>
struct ChainOps {
    static constexpr int TPW = K / 16 / CHAIN_WAVES;   // row tiles per wave
    f32x4 a[TPW];     // states, forward: w rows;  grads: kr rows     (A operand, 16 x 16)
    f32x4 at[TPW];    // states, forward: kr^T;    grads: qd^T        (A operand)
    f32x4 bt[TPW];    // grads: w^T;  forward: qd rows                (A operand)
    f32x4 e[TPW];     // exp(gam) of the tile rows this lane holds (staged from e1)
    float e1;         // exp(gam) of row 16 TPW wave + lane % (16 TPW), as loaded
    f32x4 x;          // states, forward: u (C-layout);  grads: dO (C-layout)
    f32x4 m;          // grads: Mqk^T;  forward: Mqk rows             (A operand; wave 0 uses it)
};

template <int K, int V, int MODE>
__device__ __forceinline__ void chain_load(ChainOps<K> &o, const float *ch, int n0, int wave,
                                           int lane)
{
    using WS = WsF32<K, V>;
    constexpr bool GRAD = MODE == CHAIN_GRADS, FWD = MODE == CHAIN_FORWARD;
    constexpr int TPW = ChainOps<K>::TPW;
    const int r = lane & 15, g = lane >> 4;
    const float *W = ch + WS::W / 4, *QD = ch + WS::QD / 4, *KR = ch + WS::KR / 4;
    o.e1 = ch[WS::EG / 4 + wave * TPW * 16 + lane % (TPW * 16)];
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int k0 = (wave * TPW + x) * 16;
        const float *ra = (GRAD ? KR : W) + r * K + k0 + 4 * g;
        o.a[x] = *(const f32x4 *)ra;
        if (FWD) o.bt[x] = *(const f32x4 *)(QD + r * K + k0 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            o.at[x][i] = (GRAD ? QD : KR)[t * K + k0 + r];
            if (GRAD) o.bt[x][i] = W[t * K + k0 + r];
        }
    }
    // Loads are unconditional and their values are used as loaded (rows past the sequence end
    // read its last row and are zeroed at use): any arithmetic on a value here, or a load under
    // a branch, would make the compiler wait for the load on the spot.
    if (FWD) o.m = *(const f32x4 *)(ch + WS::MQK / 4 + r * 16 + 4 * g);
    // dO (grads) from the backward record, where the prepare kernel put it in this order: an
    // input read straight from HBM arrived too late for a load one chunk ahead
    if (GRAD) o.x = *(const f32x4 *)(ch + WsF32B<K, V>::DO / 4 + ((n0 / 16) * 64 + lane) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        if (GRAD) {
            o.m[i] = ch[WS::MQK / 4 + t * 16 + r];
        } else {
            o.x[i] = ch[WS::U / 4 + t * V + n0 + r];
        }
    }
}

// One chain of one 16-column slice (columns n0 ..) of one unit (sequence * HV + value head).
// init: S (states, forward) or Lam (grads) at the start, [N][HV][K][V] or null (zero); ck: the
// per-chunk records (states, grads); fin: where the last S / Lam goes (final state, dh0) or
// null; o: the forward's output (fp32 io); rec_bytes: the chunk record's size.
template <int K, int V, int MODE>
__device__ __forceinline__ void chain_run(const FwdParams &p, int unit, int n0, int wave,
                                          int lane, const float *init, float *ck, float *fin,
                                          float *o, int rec_bytes)
{
    constexpr bool GRAD = MODE == CHAIN_GRADS, FWD = MODE == CHAIN_FORWARD;
    constexpr int TPW = ChainOps<K>::TPW;
    __shared__ f32x4 part[2][CHAIN_WAVES][FWD ? 2 : 1][64];
    __shared__ float estage[CHAIN_WAVES][64];
    const int r = lane & 15, g = lane >> 4;
    const int j = unit % p.HV, s = unit / p.HV;
    const int64_t bos = seq_bos(p.seq, s), eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CHUNK - 1) / CHUNK);
    const size_t slot0 = (size_t)j * p.seq.n_slots + (size_t)(bos / CHUNK + s);
    const size_t unit_off = ((size_t)s * p.HV + j) * (size_t)K * V;
    // element (k0 + 4g + i, n0 + r) of a row-major K x V matrix, k0 the first row of tile x
    auto at = [&](int x, int i) {
        return (size_t)((wave * TPW + x) * 16 + 4 * g + i) * V + n0 + r;
    };
    auto rec = [&](int c) { return (const float *)(p.ws + (slot0 + c) * (size_t)rec_bytes); };

    f32x4 X[TPW];                     // S (states, forward) or Lam (grads), C-layout tiles
#pragma unroll
    for (int x = 0; x < TPW; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[x][i] = init ? init[unit_off + at(x, i)] : 0.f;
    // exp(gam) of `op` from one value per lane to the C-layout rows of its tiles, through this
    // wave's own LDS stage (its write and reads are ordered by the wave's LDS queue). A 16-byte
    // load per tile fetched each value 16 times through the CU's vector-memory path (backward
    // at 16 heads x 4096 tokens 0.62 -> 0.595 ms, fp32 forward state pass 257 -> 251 us).
    auto stage_e = [&](ChainOps<K> &op) {
        estage[wave][lane] = op.e1;
#pragma unroll
        for (int x = 0; x < TPW; ++x) op.e[x] = *(const f32x4 *)&estage[wave][16 * x + 4 * g];
    };
    // one chunk with the operands in `o` (loaded one chunk earlier)
    auto step = [&](ChainOps<K> &op, int it) {
        stage_e(op);
        const int c = GRAD ? nc - 1 - it : it;
        if (!FWD) {
            // the record of this chunk, tile order: [V/16 slice][K/16 tile][64 lanes][4], as
            // two 8-byte buffer stores per tile (bstore8: plain 8-byte stores to adjacent
            // addresses are merged into one 16-byte store by the compiler, see bstore16 for why
            // that matters)
            const __amdgpu_buffer_rsrc_t cr =
                buffer_rsrc(ck + (slot0 + c) * (size_t)K * V, K * V * 4);
            const int cbase = (((n0 / 16) * (K / 16) + wave * TPW) * 256 + lane * 4) * 4;
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                bstore8<CK_AUX>(cr, cbase + x * 1024, 0, f32v2{X[x][0], X[x][1]});
                bstore8<CK_AUX>(cr, cbase + x * 1024 + 8, 0, f32v2{X[x][2], X[x][3]});
            }
        }
        f32x4 ox = op.x;
        if (GRAD) {                   // dO rows past the sequence end are zero
#pragma unroll
            for (int i = 0; i < 4; ++i) ox[i] = bos + 16 * c + 4 * g + i < eos ? ox[i] : 0.f;
        }
        // this wave's share of the K contractions: w S (states, forward) or kr Lam
        // (+ Mqk^T dO, once), and qd S (forward)
        f32x4 acc = zero4(), accq = zero4();
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            acc = mm16_f32(op.a[x], X[x], acc);
            if (FWD) accq = mm16_f32(op.bt[x], X[x], accq);
        }
        if (GRAD && wave == 0) acc = mm16_f32(op.m, ox, acc);
        const int par = it & 1;
        part[par][wave][0][lane] = acc;
        if (FWD) part[par][wave][FWD ? 1 : 0][lane] = accq;
        lds_barrier();
        f32x4 d = zero4(), oq = zero4();
#pragma unroll
        for (int w = 0; w < CHAIN_WAVES; ++w) {
            const f32x4 pw = part[par][w][0][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] += pw[i];
            if (FWD && wave == 0) {
                const f32x4 qw = part[par][w][FWD ? 1 : 0][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) oq[i] += qw[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)   // states, forward: delta = u - w S;  grads: -dDelta
            d[i] = GRAD ? -d[i] : op.x[i] - d[i];
        if (FWD && wave == 0) {       // o = qd S + Mqk delta, rows past the end not stored
            const f32x4 ov = mm16_f32(op.m, d, oq);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = bos + 16 * c + 4 * g + i;
                if (tok < eos) o[(tok * p.HV + j) * V + n0 + r] = ov[i];
            }
        }
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            f32x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = op.e[x][i] * X[x][i];
            if (GRAD) {
                y = mm16_f32(op.at[x], ox, y);                        // + qd^T dO
                y = mm16_f32(op.bt[x], d, y);                         // - w^T dDelta
            } else {
                y = mm16_f32(op.at[x], d, y);                         // + kr^T delta
            }
            X[x] = y;
        }
    };
    auto load = [&](ChainOps<K> &op, int it) {
        const int c = GRAD ? nc - 1 - it : it;
        chain_load<K, V, MODE>(op, rec(c), n0, wave, lane);
    };
    // two operand sets used alternately (a copy from one to the other would wait for the loads)
    if (nc > 0) {
        ChainOps<K> o0, o1;
        load(o0, 0);
        for (int it = 0; it < nc; it += 2) {
            load(o1, it + 1 < nc ? it + 1 : it);
            step(o0, it);
            if (it + 1 >= nc) break;
            load(o0, it + 2 < nc ? it + 2 : it + 1);
            step(o1, it + 1);
        }
    }
    if (fin) {
#pragma unroll
        for (int x = 0; x < TPW; ++x)
#pragma unroll
            for (int i = 0; i < 4; ++i) fin[unit_off + at(x, i)] = X[x][i];
    }
}

}  // namespace

}  // namespace kda
