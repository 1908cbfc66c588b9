// kda_prepare32.hip -- the stand-alone prepare kernel for 32-token chunks (the per-chunk
// work itself is in kda_prep32.h).
#include "kda_prep32.h"

namespace kda {

// Two chunk slots per workgroup: the second slot's inputs are loaded before the first slot is
// processed, so their memory latency is covered by the first slot's work.
template <int K, int V, bool NORM>
__global__ __launch_bounds__(128) void prepare32_bf16_kernel(FwdParams p)
{
    using WS = WsBf16x32<K, V>;
    __shared__ Prep32Share<K, V> sh;
    const int wave = threadIdx.x >> 6;      // row block: 0 = a, 1 = b
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.y;
    const int slot0 = 2 * blockIdx.x, slot1 = slot0 + 1;
    int s0 = 0, s1 = 0, nv0 = 0, nv1 = 0;
    int64_t bos0 = 0, bos1 = 0;
    // workgroup-uniform: every wave takes the same branches and barriers
    const bool ok0 = slot0 < p.seq.n_slots && locate_slot<32>(p.seq, slot0, &s0, &bos0, &nv0);
    const bool ok1 = slot1 < p.seq.n_slots && locate_slot<32>(p.seq, slot1, &s1, &bos1, &nv1);
    Prep32In<K, V> in0, in1;
    if (ok0) prep32_load<K, V>(p, bos0, nv0, j, wave, lane, in0);
    if (ok1) prep32_load<K, V>(p, bos1, nv1, j, wave, lane, in1);
    const uint8_t *ws = p.ws + (size_t)j * p.seq.n_slots * (size_t)WS::BYTES;
    if (ok0)
        prep32_chunk<K, V, NORM>(p, sh, in0,
                                 buffer_rsrc(ws + (size_t)slot0 * WS::BYTES, WS::BYTES), j, wave,
                                 lane);
    if (ok0 && ok1) __syncthreads();         // the shared block is reused by the second slot
    if (ok1)
        prep32_chunk<K, V, NORM>(p, sh, in1,
                                 buffer_rsrc(ws + (size_t)slot1 * WS::BYTES, WS::BYTES), j, wave,
                                 lane);
}

template <int K, int V>
hipError_t launch_prepare32_bf16(const FwdParams &p, hipStream_t st)
{
    dim3 grid((p.seq.n_slots + 1) / 2, p.HV);
    if (p.pre.qk_l2norm)
        prepare32_bf16_kernel<K, V, true><<<grid, dim3(128), 0, st>>>(p);
    else
        prepare32_bf16_kernel<K, V, false><<<grid, dim3(128), 0, st>>>(p);
    return hipGetLastError();
}

#define KDA_INST(K, V) \
    template hipError_t launch_prepare32_bf16<K, V>(const FwdParams &, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
