// kda_prepare32.hip -- the stand-alone prepare kernels for 32-token chunks (the per-chunk work
// itself is in kda_prep32.h): one record per 32-token chunk (chunk 32), or the two records of
// each 64-token pair of chunks (chunk 64).
#include "kda_prep32.h"

namespace kda {

// Two chunk slots per workgroup: the second slot's inputs are requested as soon as the first
// slot's have arrived, so they stream in while the first slot is processed (requested at the
// kernel start they had competed with every workgroup's first-slot loads, and every wave
// waited for the whole input read before computing).
//
// Grid: x enumerates (slot pair, member of the value-head group), y the q/k head. The G value
// heads of a group read the same q and k rows; blockIdx.x -> (pair, member) is the XCD map of
// state_unit (workgroups go to the 8 XCDs round-robin), so the G workgroups of one slot pair
// run on one XCD, eight dispatches apart, and the later ones find q and k in that XCD's L2.
template <int K, int V, bool NORM>
__global__ __launch_bounds__(128) void prepare32_bf16_kernel(FwdParams p)
{
    using WS = WsBf16x32<K, V>;
    __shared__ Prep32Share<K, V> sh;
    const int wave = threadIdx.x >> 6;      // row block: 0 = a, 1 = b
    const int lane = threadIdx.x & 63;
    int pair = 0, member = 0;
    if (!state_unit(blockIdx.x, p.G, (p.seq.n_slots + 1) / 2, &pair, &member)) return;
    const int j = blockIdx.y * p.G + member;
    const int slot0 = 2 * pair, slot1 = slot0 + 1;
    int s0 = 0, s1 = 0, nv0 = 0, nv1 = 0;
    int64_t bos0 = 0, bos1 = 0;
    // workgroup-uniform: every wave takes the same branches and barriers
    const bool ok0 = slot0 < p.seq.n_slots && locate_slot<32>(p.seq, slot0, &s0, &bos0, &nv0);
    const bool ok1 = slot1 < p.seq.n_slots && locate_slot<32>(p.seq, slot1, &s1, &bos1, &nv1);
    Prep32In<K, V> in0, in1;
    if (ok0) prep32_load<K, V>(p, bos0, nv0, j, wave, lane, in0);
    const uint8_t *ws = p.ws + (size_t)j * p.seq.n_slots * (size_t)WS::BYTES;
    auto load1 = [&]() {
        if (ok1) prep32_load<K, V>(p, bos1, nv1, j, wave, lane, in1);
    };
    if (ok0)
        prep32_chunk<K, V, NORM, 0, 0>(p, sh, nullptr, in0,
                                       buffer_rsrc(ws + (size_t)slot0 * WS::BYTES, WS::BYTES), j,
                                       wave, lane, load1);
    else
        load1();
    if (ok0 && ok1) __syncthreads();         // the shared block is reused by the second slot
    if (ok1)
        prep32_chunk<K, V, NORM>(p, sh, nullptr, in1,
                                 buffer_rsrc(ws + (size_t)slot1 * WS::BYTES, WS::BYTES), j, wave,
                                 lane);
}

// One workgroup per 64-token pair slot: sequence s's pair m (tokens bos + 64 m ..) lives in pair
// slot floor(bos / 64) + s + m, and its two records (chunks 2m and 2m + 1, WsPair layout) at
// record index 2 * slot and 2 * slot + 1 of the value head. The second chunk may be empty (a
// sequence whose length ends in the first half): its rows are zero, which makes its record the
// identity step (W = U = KR = P = 0, e^{gam} = 1).
template <int K, int V, bool NORM>
__global__ __launch_bounds__(128) void prepare64_bf16_kernel(FwdParams p)
{
    using WP = WsPair<K, V>;
    __shared__ Prep32Share<K, V> sh;
    __shared__ PairStash<K> ps;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.y;
    const int slot = blockIdx.x;
    int s = 0, nv = 0;
    int64_t bos = 0;
    if (!locate_slot<64>(p.seq, slot, &s, &bos, &nv)) return;   // workgroup-uniform
    Prep32In<K, V> in0, in1;
    prep32_load<K, V>(p, bos, nv < 32 ? nv : 32, j, wave, lane, in0);
    const uint8_t *rec =
        p.ws + ((size_t)j * 2 * p.seq.n_slots + 2 * (size_t)slot) * (size_t)WP::BYTES;
    prep32_chunk<K, V, NORM, 0, 1>(p, sh, &ps, in0, buffer_rsrc(rec, WP::BYTES), j, wave, lane,
                                   [&]() { prep32_load<K, V>(p, bos + 32, nv - 32, j, wave, lane,
                                                             in1); });
    __syncthreads();                         // the shared block is reused; the stash is read
    prep32_chunk<K, V, NORM, 0, 2>(p, sh, &ps, in1, buffer_rsrc(rec + WP::BYTES, WP::BYTES), j,
                                   wave, lane);
}

template <int K, int V>
hipError_t launch_prepare32_bf16(const FwdParams &p, hipStream_t st)
{
    const int pairs = (p.seq.n_slots + 1) / 2;
    dim3 grid((pairs + 7) / 8 * 8 * p.G, p.H);
    if (p.pre.qk_l2norm)
        prepare32_bf16_kernel<K, V, true><<<grid, dim3(128), 0, st>>>(p);
    else
        prepare32_bf16_kernel<K, V, false><<<grid, dim3(128), 0, st>>>(p);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_prepare64_bf16(const FwdParams &p, hipStream_t st)
{
    dim3 grid(p.seq.n_slots, p.HV);          // pair slots
    if (p.pre.qk_l2norm)
        prepare64_bf16_kernel<K, V, true><<<grid, dim3(128), 0, st>>>(p);
    else
        prepare64_bf16_kernel<K, V, false><<<grid, dim3(128), 0, st>>>(p);
    return hipGetLastError();
}

#define KDA_INST(K, V)                                                                     \
    template hipError_t launch_prepare32_bf16<K, V>(const FwdParams &, hipStream_t);     \
    template hipError_t launch_prepare64_bf16<K, V>(const FwdParams &, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
