// kda_state32.hip -- the stand-alone state kernel for 32-token chunks (the per-slice work
// itself is in kda_state32.h).
#include "kda_state32.h"

namespace kda {

// SPW V-slices of one (sequence, value head) per workgroup. Each slice has two chain halves
// (the two halves of its key rows) and an output wave; the slices of a unit share every operand
// but -U, so once a workgroup holds several, one output wave serves two slices (QD / Mqk loaded
// once: 0.431 -> 0.388 ms at 4 x 8192 tokens x 32 value heads, 0.487 -> 0.440 ms for 8 packed
// sequences x 32 heads) and, with four, one chain wave serves the same half of two slices (W,
// KR, e^gam loaded once: 0.392 -> 0.330 ms at 4 x 8192 x 32; with two slices per workgroup it
// lengthened each step of the packed sequences' longest units, 0.440 -> 0.484 ms). With several
// slices per workgroup the slices pass their barriers together and read each chunk record at
// the same time, so a record is fetched once per workgroup instead of once per slice; with one
// slice per workgroup small launches spread over more CUs.
template <int SPW> constexpr int out_slices32() { return SPW == 1 ? 1 : 2; }     // per output wave
template <int SPW> constexpr int chain_slices32() { return SPW == 4 ? 2 : 1; }   // per chain wave
template <int SPW> constexpr int group_waves32() {
    return 2 * (out_slices32<SPW>() / chain_slices32<SPW>()) + 1;
}
template <int SPW> constexpr int waves32() {
    return SPW / out_slices32<SPW>() * group_waves32<SPW>();
}

template <int K, int V, int SPW>
__global__ __launch_bounds__(64 * waves32<SPW>()) void state32_bf16_kernel(FwdParams p)
{
    constexpr int NV = V / 16, NG = NV / SPW, OPW = out_slices32<SPW>(),
                  CS = chain_slices32<SPW>(), GW = group_waves32<SPW>();
    __shared__ Handoff32<K> hos[SPW];
    // the wave index is uniform per wave; readfirstlane makes that visible to the compiler,
    // so field offsets derived from it stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    int unit, group;
    if (!state_unit32(blockIdx.x, NG, p.seq.N * p.HV, &unit, &group)) return;
    unit = longest_first(p.seq, p.HV, unit);
    const Unit32<K, V, 0> u(p, unit);
    // waves in groups of GW per OPW slices: the two chain halves of each CS of them, then the
    // group's output wave
    const int gi = wave / GW, r = wave % GW;
    if (r < GW - 1) {
        const int sw = gi * OPW + (r >> 1) * CS;
        state32_chain<K, V, 0, CS>(p, &hos[sw], u, group * SPW + sw, r & 1, lane);
    } else {
        state32_out<K, V, 0, OPW>(p, &hos[gi * OPW], u, group * SPW + gi * OPW, lane);
    }
}

template <int K, int V, int SPW>
static hipError_t launch_state32_spw(const FwdParams &p, hipStream_t st)
{
    const int64_t units = (int64_t)p.seq.N * p.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * (V / 16 / SPW);
    if (nblk == 0) return hipSuccess;
    state32_bf16_kernel<K, V, SPW><<<dim3((unsigned)nblk), dim3(64 * waves32<SPW>()), 0, st>>>(p);
    return hipGetLastError();
}

// Two-segment pass (Split32), one launch: the first nA workgroups are segment A (one value
// slice each: two chain waves and an output wave; waves 3 and 4 only pass the barriers), the
// next nA segment B (a value slice and the same-numbered slice of the transition: two chain
// waves each and one output wave for both). Both halves use the XCD map of the one-segment
// kernel. The launch reserves enough LDS that no CU holds two of these workgroups: the grid is
// sized to the CU count, and two on one CU would share its SIMDs while another CU idles.
template <int K, int V>
__global__ __launch_bounds__(320) void state32_split_kernel(FwdParams p)
{
    static_assert(K == V, "the transition slices pair with the value slices");
    constexpr int NV = V / 16;
    using WS = WsBf16x32<K, V>;
    __shared__ Handoff32<K> hos[2];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int units = p.seq.N * p.HV;
    const int nA = (units + 7) / 8 * 8 * NV;
    const bool seg_b = (int)blockIdx.x >= nA;
    int unit, slice;
    if (!state_unit32((int)blockIdx.x - (seg_b ? nA : 0), NV, units, &unit, &slice)) return;
    Unit32<K, V, 0> u(p, unit);
    const size_t st = ((size_t)u.s * p.HV + u.j) * (size_t)K * V;
    if (!seg_b) {
        u.nc = p.split.c0;
        const float *h0u = p.h0 ? p.h0 + st : nullptr;
        if (wave == 0)
            chain_wave<K, V, 0, 0, 1, false, FIN_BFRAG>(&hos[0], u.base, u.nc, h0u,
                                                        p.split.smf + st, slice, lane);
        else if (wave == 1)
            chain_wave<K, V, 1, 0, 1, false, FIN_BFRAG>(&hos[0], u.base, u.nc, h0u,
                                                        p.split.smf + st, slice, lane);
        else if (wave == 2)
            state32_out<K, V, 0, 1>(p, &hos[0], u, slice, lane);
        else
            for (int c = 0; c <= u.nc; ++c) lds_barrier();   // the same barriers as the others
        return;
    }
    const int c0 = p.split.c0;
    u.base += (size_t)c0 * WS::BYTES;
    u.bos += 32 * (int64_t)c0;
    u.nc = p.split.nb;
    float *s0 = p.ht ? p.split.s0 + st : nullptr;
    _Float16 *phi = p.ht ? p.split.phf + st : nullptr;
    switch (wave) {
    case 0: chain_wave<K, V, 0, 0, 1>(&hos[0], u.base, u.nc, nullptr, s0, slice, lane); break;
    case 1: chain_wave<K, V, 1, 0, 1>(&hos[0], u.base, u.nc, nullptr, s0, slice, lane); break;
    case 2:
        chain_wave<K, V, 0, 0, 1, true, FIN_TTILE>(&hos[1], u.base, u.nc, nullptr, phi, slice,
                                                   lane);
        break;
    case 3:
        chain_wave<K, V, 1, 0, 1, true, FIN_TTILE>(&hos[1], u.base, u.nc, nullptr, phi, slice,
                                                   lane);
        break;
    default: state32_out_split<K, V>(p, hos, u, (size_t)unit, slice, lane);
    }
}

// Chunks of segment B per correction workgroup.
constexpr int SPLIT_FIX_CHUNKS = 1;

// The correction after the two-segment pass: for every token of segment B, o = o0 + y S_A
// (stored as bf16), and the final state S0_end + phi S_A (S0_end from the scratch: this kernel
// is the only writer of final_state, after every read of initial_state). Workgroups of V/32
// waves, per unit first one per SPLIT_FIX_CHUNKS chunks of B, then one per 16-row tile of the
// final state; wave w owns the output columns [32 w, 32 w + 32). Every product is a 16x16x32
// MFMA: C(O^T) = S_A^T Y^T takes the S_A fragment (the B operand of S_A) as the A operand of
// S_A^T, and phi S_A takes it as the B operand it is.
template <int K, int V>
__global__ __launch_bounds__(64 * (V / 32)) void split32_fix_kernel(FwdParams p)
{
    static_assert(K == V, "square transition");
    constexpr int NS = K / 32, NK = K / 16, NV = V / 16;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, n = lane & 15;
    const int nb = p.split.nb;
    const int ngrp = (nb + SPLIT_FIX_CHUNKS - 1) / SPLIT_FIX_CHUNKS;
    // unit u's workgroups on XCD u % 8 (dispatch is round-robin over the 8 XCDs), the XCD
    // whose L2 last held the unit's scratch: the pass ran all of the unit's slices there
    const int xcd = (int)blockIdx.x & 7, r = (int)blockIdx.x >> 3;
    const int unit = r / (ngrp + NK) * 8 + xcd, gi = r % (ngrp + NK);
    if (unit >= p.seq.N * p.HV) return;
    const int j = unit % p.HV, s = unit / p.HV;
    const size_t st = ((size_t)s * p.HV + j) * (size_t)K * V;
    if (gi >= ngrp && !p.ht) return;
    const f16x8 *smf = (const f16x8 *)(p.split.smf + st);
    f16x8 SA[2][NS];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int t = 0; t < NS; ++t) SA[vt][t] = smf[((2 * wave + vt) * NS + t) * 64 + lane];
    if (gi >= ngrp) {
        // final-state rows [16 rt, 16 rt + 16): A operand of phi from two transposed tiles
        const int rt = gi - ngrp;
        const f16x4 *phf = (const f16x4 *)(p.split.phf + st);
        f16x8 PA[NS];
#pragma unroll
        for (int t = 0; t < NS; ++t)
            PA[t] = cat(phf[(rt * NK + 2 * t) * 64 + lane], phf[(rt * NK + 2 * t + 1) * 64 + lane]);
        const float *s0 = p.split.s0 + st;
        float *ht = p.ht + st;
        f32x4 acc[2];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[vt][i] = s0[(size_t)(16 * rt + 4 * grp + i) * V + 16 * (2 * wave + vt) + n];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
#pragma unroll
            for (int t = 0; t < NS; ++t) acc[vt] = mfma32(PA[t], SA[vt][t], acc[vt]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ht[(size_t)(16 * rt + 4 * grp + i) * V + 16 * (2 * wave + vt) + n] = acc[vt][i];
        }
        return;
    }
    const int64_t bos = seq_bos(p.seq, s), eos = seq_eos(p.seq, s, bos);
    const int64_t row_bytes = (int64_t)p.HV * V * 2, head_bytes = (int64_t)j * V * 2;
    const size_t o0_bytes = (size_t)nb * 2 * NV * 64 * 8, y_bytes = (size_t)nb * 2 * NK * 64 * 8;
    const __amdgpu_buffer_rsrc_t o0 =
        buffer_rsrc((uint8_t *)p.split.o0 + (size_t)unit * o0_bytes, (uint32_t)o0_bytes);
    const __amdgpu_buffer_rsrc_t yr =
        buffer_rsrc((uint8_t *)p.split.y + (size_t)unit * y_bytes, (uint32_t)y_bytes);
    // every operand of the workgroup's chunks is requested before the first product (a chunk
    // index past the last chunk of B is clamped for the loads, and its stores are dropped)
    f16x8 yb[SPLIT_FIX_CHUNKS][2][NS];
    f16x4 oc[SPLIT_FIX_CHUNKS][2][2];
#pragma unroll
    for (int k = 0; k < SPLIT_FIX_CHUNKS; ++k) {
        const int c = min(gi * SPLIT_FIX_CHUNKS + k, nb - 1);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int at = ((2 * c + b) * NK + 2 * t) * 64 + lane;
                const f16x4 lo = __builtin_bit_cast(f16x4, bload8(yr, at * 8, 0));
                const f16x4 hi = __builtin_bit_cast(f16x4, bload8(yr, (at + 64) * 8, 0));
                yb[k][b][t] = cat(lo, hi);
            }
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
                oc[k][b][vt] = __builtin_bit_cast(
                    f16x4, bload8(o0, (((2 * c + b) * NV + 2 * wave + vt) * 64 + lane) * 8, 0));
        }
    }
#pragma unroll
    for (int k = 0; k < SPLIT_FIX_CHUNKS; ++k) {
        const int c = gi * SPLIT_FIX_CHUNKS + k;
        // the chunk's rows (nv >= 1 for every chunk of B; rows past eos are dropped, and so is
        // every store of a chunk index past B)
        const int64_t r0 = bos + 32 * ((int64_t)p.split.c0 + c);
        const int64_t nv = eos - r0;
        const __amdgpu_buffer_rsrc_t orows =
            c < nb ? rows_rsrc(p.o, r0, (int)(nv < 32 ? nv : 32), row_bytes, head_bytes)
                   : buffer_rsrc(p.o, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = (float)oc[k][b][vt][i];
#pragma unroll
                for (int t = 0; t < NS; ++t) acc = mfma32(SA[vt][t], yb[k][b][t], acc);
                const int col = 16 * (2 * wave + vt) + 4 * grp;
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(u32x2, to_bf16x4(acc)), orows,
                    (int)((16 * b + n) * row_bytes + col * 2), 0, 0);
            }
    }
}

template <int K, int V>
static hipError_t launch_state32_split(const FwdParams &p, hipStream_t st)
{
    if constexpr (K != V) {
        return hipErrorInvalidValue;
    } else {
        const int64_t units = (int64_t)p.seq.N * p.HV;
        const int64_t nA = (units + 7) / 8 * 8 * (V / 16);
        // more than half of the CU's LDS per workgroup: one workgroup per CU
        const size_t pad = 82 * 1024 - 2 * sizeof(Handoff32<K>);
        state32_split_kernel<K, V><<<dim3((unsigned)(2 * nA)), dim3(320), pad, st>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t ngrp = (p.split.nb + SPLIT_FIX_CHUNKS - 1) / SPLIT_FIX_CHUNKS;
        split32_fix_kernel<K, V><<<dim3((unsigned)((units + 7) / 8 * 8 * (ngrp + K / 16))),
                                   dim3(64 * (V / 32)), 0, st>>>(p);
        return hipGetLastError();
    }
}

// Slices per workgroup: 4 (2) once there are at least 4 (2) slice workgroups per CU to fill,
// else 1. A workgroup of four slices holds a CU alone (12 waves); packed sequences of uneven
// lengths pay for it only with the longest-first unit order (longest_first), which starts the
// long chains before the short ones fill in (8 packed sequences of 944 to 7424 tokens x 32
// heads: state pass 0.439 ms with 2 slices in input order, 0.418 with 2 longest first, 0.420
// with 4 in input order, 0.345 with 4 longest first).
template <int K, int V>
hipError_t launch_state32_bf16(const FwdParams &p, hipStream_t st)
{
    if (p.split.c0 > 0) return launch_state32_split<K, V>(p, st);
    const int cus = current_device_cus();
    const int64_t slice_wgs = (int64_t)p.seq.N * p.HV * (V / 16);
    if (slice_wgs >= 4LL * cus) return launch_state32_spw<K, V, 4>(p, st);
    if (slice_wgs >= 2LL * cus) return launch_state32_spw<K, V, 2>(p, st);
    return launch_state32_spw<K, V, 1>(p, st);
}

#define KDA_INST(K, V) \
    template hipError_t launch_state32_bf16<K, V>(const FwdParams &, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
