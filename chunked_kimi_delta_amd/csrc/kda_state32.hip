// kda_state32.hip -- stage 2 with 32-token chunks: the chunk-sequential state pass, one serial
// step per 32 tokens.
//
// Per chunk, with S the K x V state at the chunk start ("手撕KDA" section 1, chunk loop of
// naive_chunk_kda, here with chunk 32):
//     delta = U - W S                      (32 x V)
//     o     = QD S + Mqk delta             (32 x V), rows past the sequence end not stored
//     S    <- diag(e^{gam}) S + KR^T delta
//
// Same structure as the 16-token kernel (kda_state.hip): one workgroup = a chain wave and an
// output wave on two SIMDs for one (sequence, value head, 16-column slice), S in fp32 registers,
// fp16 operands, a double-buffered LDS hand-off and one barrier per chunk. Chunk operands are
// read through buffer resources (scalar addressing). The 32-token step is
// what makes the chain cheaper per token: W S is two independent 16-row products (8 MFMAs), the
// state update contracts all 32 tokens in one full-rate 16x16x32 MFMA per 16-row tile of S
// (8 MFMAs, against 8 half-rate 16x16x16 MFMAs per 16 tokens), and the per-step VALU work
// (fp16 copy of S, decay, hand-off, barrier) is paid once per 32 tokens.
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

__device__ __forceinline__ void release_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}
__device__ __forceinline__ void acquire_lds() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int K, int V>
struct ChainFrag32 {
    f16x8 w[2][K / 32];                      // W rows of blocks a and b
    f16x8 kr[K / 16];                        // KR^T tiles over the 32 tokens
    f32x4 nu[2];                             // -U of blocks a and b, this lane's slice (fp32)
};

template <int K, int V>
struct OutFrag32 {
    static constexpr int EGPL = K / 64;      // exp(gam) values loaded per lane
    f16x8 qd[2][K / 32];
    f16x4 mqa;
    f16x8 mqb;
    float eg[EGPL];                          // exp(gam) of the chunk two ahead of this one
};

// One chunk record seen through a buffer resource (scalar base = the record); every field
// offset is a scalar constant and the per-lane part is lane * size, so no load needs vector
// address arithmetic.
template <int K, int V>
struct Chunk32 {
    using WS = WsBf16x32<K, V>;
    static constexpr int NS = K / 32, NV = V / 16, EGPL = K / 64;
    __amdgpu_buffer_rsrc_t rs;
    int lane, slice;
    __device__ __forceinline__ void load_w(ChainFrag32<K, V> &f) const {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int st = 0; st < NS; ++st)
                f.w[b][st] = __builtin_bit_cast(f16x8, bload16(rs, lane * 16,
                                                               WS::W + (b * NS + st) * 1024));
#pragma unroll
        for (int b = 0; b < 2; ++b)
            f.nu[b] = __builtin_bit_cast(f32x4, bload16(rs, lane * 16,
                                                        WS::NU + (b * NV + slice) * 1024));
    }
    __device__ __forceinline__ void load_kreg(ChainFrag32<K, V> &f) const {
#pragma unroll
        for (int t = 0; t < K / 16; ++t)
            f.kr[t] = __builtin_bit_cast(f16x8, bload16(rs, lane * 16, WS::KR + t * 1024));
    }
    __device__ __forceinline__ void load_eg(float (&eg)[EGPL]) const {
        if constexpr (EGPL == 2) {
            const u32x2 e = bload8(rs, lane * 8, WS::EG);
            eg[0] = __uint_as_float(e[0]);
            eg[1] = __uint_as_float(e[1]);
        } else {
            eg[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, WS::EG, 0));
        }
    }
    // output operands of this chunk and exp(gam) of chunk `ahead` (two chunks later)
    __device__ __forceinline__ void load_out(OutFrag32<K, V> &f, const Chunk32 &ahead) const {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int st = 0; st < NS; ++st)
                f.qd[b][st] = __builtin_bit_cast(f16x8, bload16(rs, lane * 16,
                                                                WS::QD + (b * NS + st) * 1024));
        f.mqa = __builtin_bit_cast(f16x4, bload8(rs, lane * 8, WS::MQKA));
        f.mqb = __builtin_bit_cast(f16x8, bload16(rs, lane * 16, WS::MQKB));
        ahead.load_eg(f.eg);
    }
};

template <int K>
struct Handoff32 {
    f16x8 sh[2][K / 32][64];     // S (fp16) by chunk parity
    f16x4 dh[2][2][64];          // delta of blocks a and b by chunk parity
    float eg[2][K];              // exp(gam) by chunk parity, staged by the output wave
};

// exp(gam) arrives as K/64 values per lane, but every chain lane needs the four values of the
// S rows 16t + 4g + i it holds: the output wave stages the row in LDS two chunks ahead and the
// chain wave reads it back as broadcast vector loads.
template <int K>
__device__ __forceinline__ void stage_eg(const float (&eg)[K / 64], Handoff32<K> &ho, int par,
                                         int lane)
{
#pragma unroll
    for (int e = 0; e < K / 64; ++e) ho.eg[par][lane * (K / 64) + e] = eg[e];
}

// Chain wave, one 32-token chunk with S at the chunk start.
//   1. exp(gam) of the chunk is read from LDS (latency covered by the products below);
//   2. the fp16 copy of S goes to the hand-off and into the W S products, which start from -U
//      so that delta is the negated accumulator; delta goes to the hand-off;
//   3. S is decayed tile by tile, each tile followed by its update MFMA (KR^T delta); the
//      update is issued before the hand-off barrier, so the barrier wait overlaps it.
// The W and -U groups of `f` are refilled from `nxt` (two chunks ahead, clamped to the last
// chunk) once the products are issued, the KR^T group once the update is issued.
template <int K, int V>
__device__ __forceinline__ void chain_step32(ChainFrag32<K, V> &f, const Chunk32<K, V> &nxt,
                                             f32x4 (&S)[K / 16], Handoff32<K> &ho, int par,
                                             int lane, int grp)
{
    constexpr int NS = K / 32, NK = K / 16;
    f32x4 e4[NK];
#pragma unroll
    for (int t = 0; t < NK; ++t) e4[t] = *(const f32x4 *)&ho.eg[par][16 * t + 4 * grp];
    f32x4 X0 = f.nu[0], X1 = f.nu[1];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const f16x8 Sh = cat(to_f16x4(S[2 * st]), to_f16x4(S[2 * st + 1]));
        ho.sh[par][st][lane] = Sh;
        X0 = mfma32(f.w[0][st], Sh, X0);
        X1 = mfma32(f.w[1][st], Sh, X1);
    }
    nxt.load_w(f);
    f16x4 dh0, dh1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dh0[i] = (_Float16)(-X0[i]);
        dh1[i] = (_Float16)(-X1[i]);
    }
    ho.dh[par][0][lane] = dh0;
    ho.dh[par][1][lane] = dh1;
    const f16x8 d32 = cat(dh0, dh1);
#pragma unroll
    for (int t = 0; t < NK; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] *= e4[t][i];
        S[t] = mfma32(f.kr[t], d32, S[t]);
    }
    release_lds();
    __builtin_amdgcn_s_barrier();
    acquire_lds();
    nxt.load_kreg(f);
}

// Output wave, one 32-token chunk: o = QD S + Mqk delta from the hand-off, stored as bf16;
// exp(gam) of the chunk two ahead is staged for the chain wave. `nxt` is the record two
// chunks ahead (output operands) and `nxt2` the one four ahead (its exp(gam)).
template <int K, int V>
__device__ __forceinline__ void out_step32(OutFrag32<K, V> &f, const Chunk32<K, V> &nxt,
                                           const Chunk32<K, V> &nxt2, Handoff32<K> &ho, int par,
                                           int lane, __amdgpu_buffer_rsrc_t orows,
                                           const int (&ooff)[8])
{
    constexpr int NS = K / 32;
    release_lds();
    __builtin_amdgcn_s_barrier();
    acquire_lds();
    f16x8 Sh[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) Sh[st] = ho.sh[par][st][lane];
    const f16x4 dh0 = ho.dh[par][0][lane], dh1 = ho.dh[par][1][lane];
    stage_eg<K>(f.eg, ho, par, lane);
    f32x4 Y0 = zero4(), Y1 = zero4();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        Y0 = mfma32(f.qd[0][st], Sh[st], Y0);
        Y1 = mfma32(f.qd[1][st], Sh[st], Y1);
    }
    const f32x4 O0 = mfma16(f.mqa, dh0, Y0);
    const f32x4 O1 = mfma32(f.mqb, cat(dh0, dh1), Y1);
    nxt.load_out(f, nxt2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 b0 = (__bf16)O0[i], b1 = (__bf16)O1[i];
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b0), orows, ooff[i],
                                              0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b1), orows,
                                              ooff[4 + i], 0, 0);
    }
}

}  // namespace

// Barrier schedule (nc chunks, both waves pass nc + 1 barriers): an initial one after the
// output wave has staged exp(gam) of chunks 0 and 1, then one per chunk c after the chain wave
// has written the hand-off of chunk c. Between barriers c and c+1 the output wave reads the
// hand-off slot c % 2 and overwrites the exp(gam) slot c % 2 with chunk c+2, while the chain
// wave reads exp(gam) slot (c+1) % 2 and writes the hand-off slot (c+1) % 2.
template <int K, int V>
__global__ __launch_bounds__(128) void state32_bf16_kernel(FwdParams p)
{
    constexpr int NK = K / 16, NV = V / 16, CT = 32;
    using WS = WsBf16x32<K, V>;
    __shared__ Handoff32<K> ho;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = lane >> 4, n = lane & 15;
    int unit, slice;
    if (!state_unit32(blockIdx.x, NV, p.seq.N * p.HV, &unit, &slice)) return;
    const int j = unit % p.HV;
    const int s = unit / p.HV;
    const int64_t bos = seq_bos(p.seq, s);
    const int64_t eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CT - 1) / CT);
    const int col = 16 * slice + n;
    const uint8_t *base =
        p.ws + ((size_t)j * p.seq.n_slots + (size_t)(bos / CT + s)) * (size_t)WS::BYTES;
    auto at = [&](int c) {
        return Chunk32<K, V>{buffer_rsrc(base + (size_t)min(c, nc - 1) * WS::BYTES, WS::BYTES),
                             lane, slice};
    };

    if (wave == 0) {
        f32x4 S[NK];
        if (p.h0) {
            const float *h0 = p.h0 + ((size_t)s * p.HV + j) * (size_t)K * V + col;
#pragma unroll
            for (int t = 0; t < NK; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[t][i] = h0[(size_t)(16 * t + 4 * grp + i) * V];
        } else {
#pragma unroll
            for (int t = 0; t < NK; ++t) S[t] = zero4();
        }
        if (nc > 0) {
            ChainFrag32<K, V> fa, fb;
            at(0).load_w(fa); at(0).load_kreg(fa);
            at(1).load_w(fb); at(1).load_kreg(fb);
            // drain the prologue loads: the loop header then carries only the loop's own
            // pending loads, and the waits inside the loop count back to the right group
            vm_drain();
            __builtin_amdgcn_s_barrier();     // exp(gam) of chunks 0 and 1 staged
            acquire_lds();
            // no exit between the loop body's two steps: an exit there would merge a
            // half-step state into the loop header and make every iteration wait for the
            // loads just issued
            int c = 0;
            for (; c + 2 <= nc; c += 2) {
                chain_step32<K, V>(fa, at(c + 2), S, ho, 0, lane, grp);
                chain_step32<K, V>(fb, at(c + 3), S, ho, 1, lane, grp);
            }
            if (c < nc) chain_step32<K, V>(fa, at(c + 2), S, ho, 0, lane, grp);
        }
        if (p.ht) {
            float *ht = p.ht + ((size_t)s * p.HV + j) * (size_t)K * V + col;
#pragma unroll
            for (int t = 0; t < NK; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) ht[(size_t)(16 * t + 4 * grp + i) * V] = S[t][i];
        }
    } else if (nc > 0) {
        const int64_t row_bytes = (int64_t)p.HV * V * 2, head_bytes = (int64_t)j * V * 2;
        int ooff[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ooff[i] = (int)((4 * grp + i) * row_bytes + col * 2);
            ooff[4 + i] = (int)((16 + 4 * grp + i) * row_bytes + col * 2);
        }
        auto rows = [&](int c) {
            const int64_t r0 = bos + CT * c;
            const int64_t nv = eos - r0;
            return rows_rsrc(p.o, r0, (int)(nv < CT ? nv : CT), row_bytes, head_bytes);
        };
        OutFrag32<K, V> fa, fb;
        float eg0[K / 64], eg1[K / 64];
        at(0).load_eg(eg0);
        at(1).load_eg(eg1);
        at(0).load_out(fa, at(2));
        at(1).load_out(fb, at(3));
        vm_drain();
        stage_eg<K>(eg0, ho, 0, lane);
        stage_eg<K>(eg1, ho, 1, lane);
        release_lds();
        __builtin_amdgcn_s_barrier();         // initial barrier: exp(gam) of chunks 0 and 1
        int c = 0;
        for (; c + 2 <= nc; c += 2) {
            out_step32<K, V>(fa, at(c + 2), at(c + 4), ho, 0, lane, rows(c), ooff);
            out_step32<K, V>(fb, at(c + 3), at(c + 5), ho, 1, lane, rows(c + 1), ooff);
        }
        if (c < nc) out_step32<K, V>(fa, at(c + 2), at(c + 4), ho, 0, lane, rows(c), ooff);
    }
}

template <int K, int V>
hipError_t launch_state32_bf16(const FwdParams &p, hipStream_t st)
{
    const int64_t units = (int64_t)p.seq.N * p.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * (V / 16);
    if (nblk == 0) return hipSuccess;
    state32_bf16_kernel<K, V><<<dim3((unsigned)nblk), dim3(128), 0, st>>>(p);
    return hipGetLastError();
}

#define KDA_INST(K, V) \
    template hipError_t launch_state32_bf16<K, V>(const FwdParams &, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
