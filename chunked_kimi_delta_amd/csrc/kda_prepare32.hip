// kda_prepare32.hip -- the stand-alone prepare kernels for 32-token chunks (the per-chunk work
// itself is in kda_prep32.h): one record per 32-token chunk (chunk 32), or the two records of
// each 64-token pair of chunks (chunk 64).
#include "kda_prep32.h"

namespace kda {

// SLOTS (1 or 2) chunk slots per workgroup. With two, the second slot's inputs are requested
// as soon as the first slot's have arrived, so they stream in while the first slot is
// processed (requested at the kernel start they had competed with every workgroup's first-slot
// loads, and every wave waited for the whole input read before computing). Two slots pay when
// the whole grid is resident at once (every wave would otherwise wait for its inputs at the
// same moment); with several rounds of workgroups one slot each is faster, because the rounds
// overlap one workgroup's loads with others' arithmetic by themselves.
//
// Grid: x enumerates (slot group, member of the value-head group), y the q/k head. The G value
// heads of a group read the same q and k rows; blockIdx.x -> (group, member) is the XCD map of
// state_unit (workgroups go to the 8 XCDs round-robin), so the G workgroups of one slot group
// run on one XCD, eight dispatches apart, and the later ones find q and k in that XCD's L2.
template <int K, int V, bool NORM, int SLOTS>
__global__ __launch_bounds__(128) void prepare32_bf16_kernel(FwdParams p)
{
    static_assert(SLOTS == 1 || SLOTS == 2, "one or two chunk slots per workgroup");
    using WS = WsBf16x32<K, V>;
    __shared__ Prep32Share<K, V> sh;
    const int wave = threadIdx.x >> 6;      // row block: 0 = a, 1 = b
    const int lane = threadIdx.x & 63;
    int grp = 0, member = 0;
    if (!state_unit(blockIdx.x, p.G, (p.seq.n_slots + SLOTS - 1) / SLOTS, &grp, &member))
        return;
    const int j = blockIdx.y * p.G + member;
    const int slot0 = SLOTS * grp;
    const int slot1 = SLOTS == 2 ? slot0 + 1 : p.seq.n_slots;    // one slot: no second
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

template <int K, int V, int SLOTS>
static hipError_t launch_prepare32_slots(const FwdParams &p, hipStream_t st)
{
    const int groups = (p.seq.n_slots + SLOTS - 1) / SLOTS;
    dim3 grid((groups + 7) / 8 * 8 * p.G, p.H);
    if (p.pre.qk_l2norm)
        prepare32_bf16_kernel<K, V, true, SLOTS><<<grid, dim3(128), 0, st>>>(p);
    else
        prepare32_bf16_kernel<K, V, false, SLOTS><<<grid, dim3(128), 0, st>>>(p);
    return hipGetLastError();
}

// Two slots per workgroup while the two-slot workgroups that hold chunks fit on the chip in
// one round (four two-wave workgroups per CU: the kernel's register use allows two waves per
// SIMD), else one. Workgroups of empty slots exit at once and are not counted: a dense batch
// has ceil(ceil(T / 32) / 2) two-slot groups per sequence; packed sequences at most
// T_total / 64 + N. Measured with the 16 x 4096 grid (1,024 two-slot workgroups, one round):
// 37.5 us with two slots, 39.4 with one; at 4 x 8192 tokens x 32 heads (16 rounds): 488 us
// with two, 464 with one.
template <int K, int V>
hipError_t launch_prepare32_bf16(const FwdParams &p, hipStream_t st)
{
    const int64_t groups = p.seq.cu ? (p.seq.T_total + 63) / 64 + p.seq.N
                                    : p.seq.N * (((p.seq.T + 31) / 32 + 1) / 2);
    if (groups * p.HV <= 4LL * current_device_cus()) return launch_prepare32_slots<K, V, 2>(p, st);
    return launch_prepare32_slots<K, V, 1>(p, st);
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
