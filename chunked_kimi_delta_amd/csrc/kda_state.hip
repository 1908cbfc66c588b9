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
// gfx950 design (bf16 io). The V columns of S evolve independently, so each wave64 owns one
// 16-column slice of one (sequence, value head) and keeps its K x 16 slice of S in fp32
// registers as K/16 C-layout tiles for the whole sequence. Per chunk:
//   * S is rounded to fp16 in place: C-layout == B-layout, so the accumulators feed
//     w S and qd S (16x16x32 f16 MFMAs) with no data movement between lanes;
//   * delta = u - w S comes out in C-layout == the B-layout of both Mqk delta and
//     kr^T delta (16x16x16 f16 MFMAs), and the state update accumulates onto the decayed
//     fp32 S tiles, so the S -> S chain never leaves the register file;
//   * the chunk's fragments (w, qd, kr, u, Mqk, exp(gam)) are read from the workspace in the
//     exact lane order stage 1 wrote them, as contiguous vector loads, one chunk ahead.
#include "kda_internal.h"

namespace kda {

template <int K, int V>
struct ChunkFrag {
    static constexpr int NS = K / 32, NK = K / 16;
    f16x8 w[NS], qd[NS], kr[NS];
    f16x4 u, mq;
    f32x4 eg[NK];
};

template <int K, int V>
__device__ __forceinline__ void load_frag(ChunkFrag<K, V> &f, const uint8_t *ch, int lane,
                                          int grp, int slice)
{
    using WS = WsBf16<K, V>;
#pragma unroll
    for (int st = 0; st < K / 32; ++st) {
        f.w[st] = *(const f16x8 *)(ch + WS::W + (st * 64 + lane) * 16);
        f.qd[st] = *(const f16x8 *)(ch + WS::QD + (st * 64 + lane) * 16);
        f.kr[st] = *(const f16x8 *)(ch + WS::KR + (st * 64 + lane) * 16);
    }
    f.u = *(const f16x4 *)(ch + WS::U + (slice * 64 + lane) * 8);
    f.mq = *(const f16x4 *)(ch + WS::MQK + lane * 8);
#pragma unroll
    for (int t = 0; t < K / 16; ++t) f.eg[t] = *(const f32x4 *)(ch + WS::EG + (16 * t + 4 * grp) * 4);
}

template <int K, int V>
__device__ __forceinline__ void state_step(const ChunkFrag<K, V> &f, f32x4 (&S)[K / 16],
                                           uint16_t *orow, int64_t row0, int64_t eos,
                                           int64_t ostride)
{
    constexpr int NS = K / 32, NK = K / 16;
    f16x8 Sh[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) Sh[st] = cat(to_f16x4(S[2 * st]), to_f16x4(S[2 * st + 1]));
    f32x4 X0 = zero4(), X1 = zero4(), Y0 = zero4(), Y1 = zero4();
#pragma unroll
    for (int st = 0; st < NS; st += 2) {
        X0 = mfma32(f.w[st], Sh[st], X0);
        Y0 = mfma32(f.qd[st], Sh[st], Y0);
        if (st + 1 < NS) {
            X1 = mfma32(f.w[st + 1], Sh[st + 1], X1);
            Y1 = mfma32(f.qd[st + 1], Sh[st + 1], Y1);
        }
    }
    float d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = (float)f.u[i] - (X0[i] + X1[i]);
    const f16x4 dh = to_f16x4(d);
    f32x4 Y;
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[i] = Y0[i] + Y1[i];
    const f32x4 O = mfma16(f.mq, dh, Y);
#pragma unroll
    for (int t = 0; t < NK; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] *= f.eg[t][i];
        const f16x8 &kp = f.kr[t >> 1];
        const f16x4 ka = (t & 1) ? __builtin_shufflevector(kp, kp, 4, 5, 6, 7)
                                 : __builtin_shufflevector(kp, kp, 0, 1, 2, 3);
        S[t] = mfma16(ka, dh, S[t]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (row0 + i < eos) {
            const __bf16 b = (__bf16)O[i];
            orow[(row0 + i) * ostride] = __builtin_bit_cast(uint16_t, b);
        }
    }
}

template <int K, int V>
__global__ __launch_bounds__(64) void state_bf16_kernel(FwdParams p)
{
    constexpr int NK = K / 16, NV = V / 16;
    using WS = WsBf16<K, V>;
    const int lane = threadIdx.x, grp = lane >> 4, n = lane & 15;
    const int wg = blockIdx.x;
    const int slice = wg % NV;
    const int j = (wg / NV) % p.HV;
    const int s = wg / (NV * p.HV);
    const int64_t bos = seq_bos(p.seq, s);
    const int64_t eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CHUNK - 1) / CHUNK);
    const int col = 16 * slice + n;

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

    const uint8_t *base =
        p.ws + ((size_t)j * p.seq.n_slots + (size_t)(bos / CHUNK + s)) * (size_t)WS::BYTES;
    const int64_t ostride = (int64_t)p.HV * V;
    uint16_t *orow = (uint16_t *)p.o + (size_t)j * V + col;

    ChunkFrag<K, V> fa, fb;
    if (nc > 0) load_frag(fa, base, lane, grp, slice);
    for (int c = 0; c < nc; c += 2) {
        if (c + 1 < nc) load_frag(fb, base + (size_t)(c + 1) * WS::BYTES, lane, grp, slice);
        state_step<K, V>(fa, S, orow, bos + CHUNK * c + 4 * grp, eos, ostride);
        if (c + 1 >= nc) break;
        if (c + 2 < nc) load_frag(fa, base + (size_t)(c + 2) * WS::BYTES, lane, grp, slice);
        state_step<K, V>(fb, S, orow, bos + CHUNK * (c + 1) + 4 * grp, eos, ostride);
    }

    if (p.ht) {
        float *ht = p.ht + ((size_t)s * p.HV + j) * (size_t)K * V + col;
#pragma unroll
        for (int t = 0; t < NK; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) ht[(size_t)(16 * t + 4 * grp + i) * V] = S[t][i];
    }
}

// =============================================================================== fp32 io
// Correctness mode: one block per (sequence, value head), one thread per value column, the
// column of S held in registers, chunk operands staged in LDS.
template <int K, int V>
__global__ __launch_bounds__(V) void state_f32_kernel(FwdParams p)
{
    using WS = WsF32<K, V>;
    __shared__ float sw[16][K], sqd[16][K], skr[16][K], smq[16][16], seg[K];
    const int n = threadIdx.x;
    const int j = blockIdx.x % p.HV, s = blockIdx.x / p.HV;
    const int64_t bos = seq_bos(p.seq, s);
    const int64_t eos = seq_eos(p.seq, s, bos);
    const int nc = (int)((eos - bos + CHUNK - 1) / CHUNK);

    float S[K];
    if (p.h0) {
        const float *h0 = p.h0 + ((size_t)s * p.HV + j) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) S[d] = h0[(size_t)d * V];
    } else {
#pragma unroll
        for (int d = 0; d < K; ++d) S[d] = 0.f;
    }
    const float *base = (const float *)(p.ws + ((size_t)j * p.seq.n_slots +
                                                (size_t)(bos / CHUNK + s)) * (size_t)WS::BYTES);
    float *o = (float *)p.o;
    for (int c = 0; c < nc; ++c) {
        const float *ch = base + (size_t)c * (WS::BYTES / 4);
        for (int idx = n; idx < 16 * K; idx += V) {
            sw[idx / K][idx % K] = ch[WS::W / 4 + idx];
            sqd[idx / K][idx % K] = ch[WS::QD / 4 + idx];
            skr[idx / K][idx % K] = ch[WS::KR / 4 + idx];
        }
        for (int idx = n; idx < 256; idx += V) smq[idx / 16][idx % 16] = ch[WS::MQK / 4 + idx];
        for (int idx = n; idx < K; idx += V) seg[idx] = ch[WS::EG / 4 + idx];
        __syncthreads();
        float d[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = ch[WS::U / 4 + t * V + n];
#pragma unroll
            for (int kk = 0; kk < K; ++kk) acc -= sw[t][kk] * S[kk];
            d[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < K; ++kk) acc += sqd[t][kk] * S[kk];
#pragma unroll
            for (int m = 0; m < 16; ++m) acc += smq[t][m] * d[m];
            const int64_t tok = bos + 16 * c + t;
            if (tok < eos) o[(tok * p.HV + j) * V + n] = acc;
        }
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            float acc = seg[kk] * S[kk];
#pragma unroll
            for (int t = 0; t < 16; ++t) acc += skr[t][kk] * d[t];
            S[kk] = acc;
        }
        __syncthreads();
    }
    if (p.ht) {
        float *ht = p.ht + ((size_t)s * p.HV + j) * (size_t)K * V + n;
#pragma unroll
        for (int d = 0; d < K; ++d) ht[(size_t)d * V] = S[d];
    }
}

template <int K, int V>
hipError_t launch_state_bf16(const FwdParams &p, hipStream_t st)
{
    const int64_t nblk = (int64_t)p.seq.N * p.HV * (V / 16);
    if (nblk == 0) return hipSuccess;
    state_bf16_kernel<K, V><<<dim3((unsigned)nblk), dim3(64), 0, st>>>(p);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_state_f32(const FwdParams &p, hipStream_t st)
{
    const int64_t nblk = (int64_t)p.seq.N * p.HV;
    if (nblk == 0) return hipSuccess;
    state_f32_kernel<K, V><<<dim3((unsigned)nblk), dim3(V), 0, st>>>(p);
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
