// kda_state.hip -- stage 2 of the chunked KDA forward: the chunk-sequential state pass.
//
// For each sequence s and value head j, with S the K x V state at the start of the chunk
// (initial_state[s, j] or 0), every chunk in order does ("手撕KDA" section 1, the chunk loop
// of naive_chunk_kda; section 5 describes the same loop as the v8 recurrence kernel):
//     delta = u - w S                       (16 x V)
//     o     = qd S + Mqk delta              (16 x V), rows past the sequence end not stored
//     S    <- diag(exp(gam)) S + kr^T delta
// and final_state[s, j] = S after the last chunk.
//
// gfx950 design (bf16 io). The V columns of S evolve independently, so each workgroup owns one
// 16-column slice of one (sequence, value head); its chain wave keeps the K x 16 slice of S in
// fp32 registers as K/16 C-layout tiles for the whole sequence and its output wave, on another
// SIMD, forms o from what the chain wave hands over each chunk. Per chunk:
//   * S is rounded to fp16 in place: C-layout == B-layout, so the accumulators feed
//     w S and qd S (16x16x32 f16 MFMAs) with no data movement between lanes (qd S runs on
//     the output wave from the same fragments, passed through LDS);
//   * delta = u - w S comes out in C-layout == the B-layout of both Mqk delta and
//     kr^T delta (16x16x16 f16 MFMAs), and the state update accumulates onto the decayed
//     fp32 S tiles, so the S -> S chain never leaves the register file;
//   * the chunk's fragments (w, qd, kr, u, Mqk, exp(gam)) are read from the workspace in the
//     exact lane order stage 1 wrote them, as contiguous vector loads, two chunks ahead;
//   * the workgroups of one (sequence, value head) share an XCD, hence an L2.
#include "kda_chain_f32.h"

namespace kda {

// Output rows of one chunk for one wave: a buffer resource whose range ends after the last
// valid token of the chunk, so stores to rows past the end of the sequence are dropped by the
// hardware range check instead of a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rows(void *o, int64_t row0, int nvalid,
                                                           int64_t row_bytes,
                                                           int64_t head_bytes) {
    uint8_t *base = (uint8_t *)o + row0 * row_bytes + head_bytes;
    const int num = (int)(nvalid * row_bytes - head_bytes);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, num, 0x00020000);
}

// The chain wave's operands of one chunk (fp16 fragments in MFMA operand order).
template <int K, int V>
struct ChainFrag {
    f16x8 w[K / 32], kr[K / 32];
    f16x4 u;
    f32x4 eg[K / 16];    // exp(gam) of the S rows 16t + 4g + i this lane holds
};

// The output wave's operands of one chunk.
template <int K, int V>
struct OutFrag {
    f16x8 qd[K / 32];
    f16x4 mq;
};

template <int K, int V>
struct ChunkPtr {
    using WS = WsBf16<K, V>;
    const uint8_t *ch;
    int lane, grp, slice;
    __device__ __forceinline__ void load_w(ChainFrag<K, V> &f) const {
#pragma unroll
        for (int st = 0; st < K / 32; ++st)
            f.w[st] = *(const f16x8 *)(ch + WS::W + (st * 64 + lane) * 16);
    }
    __device__ __forceinline__ void load_u(ChainFrag<K, V> &f) const {
        f.u = *(const f16x4 *)(ch + WS::U + (slice * 64 + lane) * 8);
    }
    __device__ __forceinline__ void load_kreg(ChainFrag<K, V> &f) const {
#pragma unroll
        for (int st = 0; st < K / 32; ++st)
            f.kr[st] = *(const f16x8 *)(ch + WS::KR + (st * 64 + lane) * 16);
#pragma unroll
        for (int t = 0; t < K / 16; ++t)
            f.eg[t] = *(const f32x4 *)(ch + WS::EG + (16 * t + 4 * grp) * 4);
    }
    __device__ __forceinline__ void load_out(OutFrag<K, V> &f) const {
#pragma unroll
        for (int st = 0; st < K / 32; ++st)
            f.qd[st] = *(const f16x8 *)(ch + WS::QD + (st * 64 + lane) * 16);
        f.mq = *(const f16x4 *)(ch + WS::MQK + lane * 8);
    }
};

// Per-chunk hand-off from the chain wave to the output wave: S (rounded to fp16, in the B
// operand order of qd S) and delta, double-buffered by chunk parity.
template <int K>
struct Handoff {
    f16x8 sh[2][K / 32][64];
    f16x4 dh[2][64];
};

// Chain wave, one chunk: delta = u - w S, hand (S, delta) to the output wave, then
// S <- diag(exp(gam)) S + kr^T delta. Each operand group of `f` is refilled from `nxt` (two
// chunks ahead, clamped to the last chunk, so the loads are unconditional and the compiler's
// wait counts stay exact) right after its last use.
template <int K, int V>
__device__ __forceinline__ void chain_step(ChainFrag<K, V> &f, const ChunkPtr<K, V> &nxt,
                                           f32x4 (&S)[K / 16], Handoff<K> &ho, int par,
                                           int lane)
{
    constexpr int NS = K / 32, NK = K / 16;
    f16x8 Sh[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        Sh[st] = cat(to_f16x4(S[2 * st]), to_f16x4(S[2 * st + 1]));
        ho.sh[par][st][lane] = Sh[st];
    }
    // decay in place now: S is needed only as the update's accumulator from here on, and the
    // multiplies overlap the w S products instead of delaying the update
#pragma unroll
    for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] *= f.eg[t][i];
    f32x4 X0 = zero4(), X1 = zero4();
#pragma unroll
    for (int st = 0; st < NS; st += 2) {
        X0 = mfma32(f.w[st], Sh[st], X0);
        if (st + 1 < NS) X1 = mfma32(f.w[st + 1], Sh[st + 1], X1);
    }
    nxt.load_w(f);
    float d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = (float)f.u[i] - (X0[i] + X1[i]);
    const f16x4 dh = to_f16x4(d);
    ho.dh[par][lane] = dh;
    nxt.load_u(f);
    lds_release();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int t = 0; t < NK; ++t) {
        const f16x8 &kp = f.kr[t >> 1];
        const f16x4 ka = (t & 1) ? __builtin_shufflevector(kp, kp, 4, 5, 6, 7)
                                 : __builtin_shufflevector(kp, kp, 0, 1, 2, 3);
        S[t] = mfma16(ka, dh, S[t]);
    }
    nxt.load_kreg(f);
}

// Output wave, one chunk: o = qd S + Mqk delta from the hand-off, stored as bf16.
template <int K, int V>
__device__ __forceinline__ void out_step(OutFrag<K, V> &f, const ChunkPtr<K, V> &nxt,
                                         const Handoff<K> &ho, int par, int lane,
                                         __amdgpu_buffer_rsrc_t orows, const int (&ooff)[4])
{
    constexpr int NS = K / 32;
    __builtin_amdgcn_s_barrier();
    lds_acquire();
    f16x8 Sh[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) Sh[st] = ho.sh[par][st][lane];
    const f16x4 dh = ho.dh[par][lane];
    f32x4 Y0 = zero4(), Y1 = zero4();
#pragma unroll
    for (int st = 0; st < NS; st += 2) {
        Y0 = mfma32(f.qd[st], Sh[st], Y0);
        if (st + 1 < NS) Y1 = mfma32(f.qd[st + 1], Sh[st + 1], Y1);
    }
    f32x4 Y;
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[i] = Y0[i] + Y1[i];
    const f32x4 O = mfma16(f.mq, dh, Y);
    nxt.load_out(f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 b = (__bf16)O[i];
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b), orows, ooff[i],
                                              0, 0);
    }
}

// One workgroup = two waves on two SIMDs for one (sequence, value head, 16-column slice):
// wave 0 carries the S -> S chain and keeps the K x 16 slice of S in fp32 registers for the
// whole sequence; wave 1 forms the outputs. One workgroup barrier per chunk (LDS-only fences,
// so outstanding global prefetches stay in flight across it).
template <int K, int V>
__global__ __launch_bounds__(128) void state_bf16_kernel(FwdParams p)
{
    constexpr int NK = K / 16, NV = V / 16;
    using WS = WsBf16<K, V>;
    __shared__ Handoff<K> ho;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = lane >> 4, n = lane & 15;
    int unit, slice;
    if (!state_unit(blockIdx.x, NV, p.seq.N * p.HV, &unit, &slice)) return;
    unit = longest_first(p.seq, p.HV, unit);
    const int j = unit % p.HV;
    const int s = unit / p.HV;
    const int64_t bos = seq_bos(p.seq, s);
    const int64_t eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CHUNK - 1) / CHUNK);
    const int col = 16 * slice + n;
    const uint8_t *base =
        p.ws + ((size_t)j * p.seq.n_slots + (size_t)(bos / CHUNK + s)) * (size_t)WS::BYTES;
    auto at = [&](int c) {
        return ChunkPtr<K, V>{base + (size_t)min(c, nc - 1) * WS::BYTES, lane, grp, slice};
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
            ChainFrag<K, V> fa, fb;
            at(0).load_w(fa); at(0).load_u(fa); at(0).load_kreg(fa);
            at(1).load_w(fb); at(1).load_u(fb); at(1).load_kreg(fb);
            // prologue loads drained and no exit between the loop body's two steps: the loop
            // header then carries only the loop's own pending loads, so each wait counts back
            // to the group it needs instead of the loads just issued
            vm_drain();
            int c = 0;
            for (; c + 2 <= nc; c += 2) {
                chain_step<K, V>(fa, at(c + 2), S, ho, 0, lane);
                chain_step<K, V>(fb, at(c + 3), S, ho, 1, lane);
            }
            if (c < nc) chain_step<K, V>(fa, at(c + 2), S, ho, 0, lane);
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
        int ooff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ooff[i] = (int)((4 * grp + i) * row_bytes + col * 2);
        auto rows = [&](int c) {
            const int64_t r0 = bos + CHUNK * c;
            const int64_t nv = eos - r0;
            return out_rows(p.o, r0, (int)(nv < CHUNK ? nv : CHUNK), row_bytes, head_bytes);
        };
        OutFrag<K, V> fa, fb;
        at(0).load_out(fa);
        at(1).load_out(fb);
        vm_drain();
        int c = 0;
        for (; c + 2 <= nc; c += 2) {
            out_step<K, V>(fa, at(c + 2), ho, 0, lane, rows(c), ooff);
            out_step<K, V>(fb, at(c + 3), ho, 1, lane, rows(c + 1), ooff);
        }
        if (c < nc) out_step<K, V>(fa, at(c + 2), ho, 0, lane, rows(c), ooff);
    }
}

// =============================================================================== fp32 io
// The state pass in fp32 on the fp32 matrix cores (kda_chain_f32.h, forward mode): one
// workgroup of 4 waves per (sequence, value head, 16-column slice), the K rows split over the
// waves, o formed by wave 0 from the waves' qd S partials and Mqk delta.
template <int K, int V>
__global__ __launch_bounds__(64 * CHAIN_WAVES) void state_f32_kernel(FwdParams p)
{
    int unit, slice;
    if (!state_unit(blockIdx.x, V / 16, p.seq.N * p.HV, &unit, &slice)) return;
    unit = longest_first(p.seq, p.HV, unit);
    chain_run<K, V, CHAIN_FORWARD>(p, unit, slice * 16, threadIdx.x >> 6, threadIdx.x & 63,
                                   p.h0, nullptr, p.ht, (float *)p.o, WsF32<K, V>::BYTES);
}

template <int K, int V>
hipError_t launch_state_bf16(const FwdParams &p, hipStream_t st)
{
    const int64_t units = (int64_t)p.seq.N * p.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * (V / 16);
    if (nblk == 0) return hipSuccess;
    state_bf16_kernel<K, V><<<dim3((unsigned)nblk), dim3(128), 0, st>>>(p);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_state_f32(const FwdParams &p, hipStream_t st)
{
    const int64_t units = (int64_t)p.seq.N * p.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * (V / 16);
    if (nblk == 0) return hipSuccess;
    state_f32_kernel<K, V><<<dim3((unsigned)nblk), dim3(64 * CHAIN_WAVES), 0, st>>>(p);
    return hipGetLastError();
}

#define KDA_INST(K, V)                                                             \
    template hipError_t launch_state_bf16<K, V>(const FwdParams &, hipStream_t);  \
    template hipError_t launch_state_f32<K, V>(const FwdParams &, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
