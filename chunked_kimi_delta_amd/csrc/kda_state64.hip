// kda_state64.hip -- the stand-alone state kernel with 64-token steps over pairs of 32-token
// chunk records (the per-slice work itself is in kda_state64.h).
#include "kda_state64.h"

namespace kda {

// SPW V-slices of one (sequence, value head) per workgroup, four waves each (two chain halves
// and two output waves).
template <int K, int V, int SPW, bool TWOK>
__global__ __launch_bounds__(256 * SPW) void state64_bf16_kernel(FwdParams p)
{
    constexpr int NV = V / 16, NG = NV / SPW;
    __shared__ Handoff64<K> hos[SPW];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sw = wave / 4, role = wave % 4;
    const int lane = threadIdx.x & 63;
    int unit, group;
    if (!state_unit64(blockIdx.x, NG, p.seq.N * p.HV, &unit, &group)) return;
    unit = longest_first(p.seq, p.HV, unit);
    const int slice = group * SPW + sw;
    state64_slice<K, V, 0, TWOK>(p, hos[sw], unit, slice, role, lane);
}

template <int K, int V, int SPW, bool TWOK>
static hipError_t launch_state64_spw(const FwdParams &p, hipStream_t st)
{
    const int64_t units = (int64_t)p.seq.N * p.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * (V / 16 / SPW);
    if (nblk == 0) return hipSuccess;
    state64_bf16_kernel<K, V, SPW, TWOK><<<dim3((unsigned)nblk), dim3(256 * SPW), 0, st>>>(p);
    return hipGetLastError();
}

// One slice per workgroup (with two, a chain wave's operand groups spill to scratch). Two
// register sets of every operand group (one wave per SIMD) while the launch fits on the chip
// at that occupancy; beyond, one set of the post-exchange group (two waves per SIMD).
template <int K, int V>
hipError_t launch_state64_bf16(const FwdParams &p, hipStream_t st)
{
    const int cus = current_device_cus();
    const int64_t waves = (int64_t)p.seq.N * p.HV * (V / 16) * 4;
    if (waves <= 4LL * cus) return launch_state64_spw<K, V, 1, true>(p, st);
    return launch_state64_spw<K, V, 1, false>(p, st);
}

#define KDA_INST(K, V) \
    template hipError_t launch_state64_bf16<K, V>(const FwdParams &, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
