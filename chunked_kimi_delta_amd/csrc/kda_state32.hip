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

// Slices per workgroup: 4 (2) once there are at least 4 (2) slice workgroups per CU to fill,
// else 1. Packed sequences of different lengths take at most 2: a workgroup of four slices
// holds a CU alone (12 waves), and with uneven units the last long ones then run on few CUs
// (8 packed sequences of 256 to 8192 tokens x 32 heads: 0.640 ms with 4, 0.526 with 2; equal
// dense sequences, 4 x 8192 x 32 heads: 0.477 with 4, 0.503 with 2).
template <int K, int V>
hipError_t launch_state32_bf16(const FwdParams &p, hipStream_t st)
{
    const int cus = current_device_cus();
    const int64_t slice_wgs = (int64_t)p.seq.N * p.HV * (V / 16);
    if (!p.seq.cu && slice_wgs >= 4LL * cus) return launch_state32_spw<K, V, 4>(p, st);
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
