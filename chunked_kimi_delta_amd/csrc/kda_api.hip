// kda_api.hip -- the extern "C" boundary of libkda_fwd (declared in include/kda_fwd.h).
//
// Host side only: argument validation, workspace sizing and the two launches on the
// caller's stream. Launch arguments follow the pages' statement of the problem: shapes and
// grouping of naive_chunk_kda ("手撕KDA" section 1) and the packed-sequence arguments of the
// FlashKDA prepare launch ("KDA源码剖析之FlashKDA（上）" parts 3 and 4: scale, total tokens,
// heads, number of sequences, cu_seqlens, an upper bound on the number of chunk tiles).
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "kda_fwd.h"
#include "kda_internal.h"

namespace kda {

// The compute-unit count only changes with the device, so it is queried once per device
// ordinal; hipGetDevice is a thread-local read.
int current_device_cus()
{
    constexpr int MAX_DEV = 64, FALLBACK = 256;
    static std::atomic<int> cached[MAX_DEV];   // 0: not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FALLBACK;
    int c = dev < MAX_DEV ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (c > 0) return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c <= 0)
        c = FALLBACK;
    if (dev < MAX_DEV) cached[dev].store(c, std::memory_order_relaxed);
    return c;
}

}  // namespace kda

namespace {

using namespace kda;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <template <int, int> class WS>
size_t record_bytes(int K, int V)
{
    return K == 64 ? (V == 64 ? WS<64, 64>::BYTES : WS<64, 128>::BYTES)
                   : (V == 64 ? WS<128, 64>::BYTES : WS<128, 128>::BYTES);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Share of a sequence's chunks given to segment A of the two-segment state pass, in parts per
// thousand. Segment A's workgroups hold one value slice, segment B's two (a value slice and a
// transition slice sharing every chunk operand). Measured at 16 heads x 4096 tokens with each
// segment alone, a workgroup takes about 2 us plus 355 ns per chunk in A and 2 us plus 478 ns
// per chunk in B, so both end together with A at 478 / (355 + 478) = 0.57 of the chunks;
// 0.58 measured best (the split kernel took 30.8 us at 0.56, 30.1 at 0.58, 31.3 at 0.60, 33.0
// at 0.65 and 34.8 at 0.70).
#ifndef KDA_SPLIT_A_PERMILLE
#define KDA_SPLIT_A_PERMILLE 580
#endif

// The two-segment state pass (Split32) and its scratch after the chunk records: bf16 io,
// 32-token chunks, dense sequences of at least 16 chunks, K == V, and a batch whose value
// slices (N HV V / 16 workgroups of the one-segment pass) fill at most half of the compute
// units, so that both segments' workgroups run at once, one per CU.
struct SplitPlan {
    int c0 = 0, nb = 0;
    size_t smf = 0, phf = 0, s0 = 0, o0 = 0, y = 0, end = 0;   // byte offsets in the workspace
};

SplitPlan split_plan(const kda_fwd_args *a, int ct, size_t records)
{
    SplitPlan sp;
    if (ct != 32 || a->io != KDA_BF16 || a->cu_seqlens || a->K != a->V || a->T < 512)
        return sp;
    const int64_t units = (int64_t)a->N * a->HV;
    if (2 * units * (a->V / 16) > (int64_t)current_device_cus()) return sp;
    const int64_t nc = ((int64_t)a->T + 31) / 32;
    int64_t c0 = (nc * KDA_SPLIT_A_PERMILLE + 500) / 1000;
    c0 = c0 < 1 ? 1 : (c0 > nc - 1 ? nc - 1 : c0);
    const int64_t nb = nc - c0;
    const size_t o0_unit = (size_t)nb * 32 * a->V * 2, y_unit = (size_t)nb * 32 * a->K * 2;
    if (o0_unit >= (1u << 31)) return sp;      // per-unit buffer resources stay 32-bit
    sp.c0 = (int)c0;
    sp.nb = (int)nb;
    sp.smf = align256(records);
    sp.phf = sp.smf + align256((size_t)units * a->K * a->V * 2);
    sp.s0 = sp.phf + align256((size_t)units * a->K * a->K * 2);
    sp.o0 = sp.s0 + align256((size_t)units * a->K * a->V * 4);
    sp.y = sp.o0 + align256((size_t)units * o0_unit);
    sp.end = sp.y + align256((size_t)units * y_unit);
    return sp;
}

// Returns KDA_OK and fills the derived sizes (`need`: workspace bytes), or the status kda_fwd
// must return.
kda_status check_shapes(const kda_fwd_args *a, int64_t *T_total, int64_t *n_slots,
                        size_t *need, int *chunk, SplitPlan *split = nullptr)
{
    if (!a) return KDA_ERR_INVALID_ARG;
    if (a->B < 1 || a->T < 0 || a->N < 0 || a->H < 1 || a->HV < 1 || a->HV % a->H)
        return KDA_ERR_INVALID_ARG;
    if (a->cu_seqlens) {
        if (a->B != 1 || a->N < 1) return KDA_ERR_INVALID_ARG;
    } else if (a->N != a->B) {
        return KDA_ERR_INVALID_ARG;
    }
    const bool k_ok = a->K == 64 || a->K == 128, v_ok = a->V == 64 || a->V == 128;
    if (!k_ok || !v_ok) return KDA_ERR_UNSUPPORTED;
    if (a->io != KDA_BF16 && a->io != KDA_FP32) return KDA_ERR_UNSUPPORTED;
    int ct = a->chunk;
    if (ct == 0)            // default: the token recurrence for short dense batches (decode)
        ct = (!a->cu_seqlens && a->T <= 16) ? 1 : (a->io == KDA_BF16 ? 32 : 16);
    if (ct != 1 && ct != 16 && !((ct == 32 || ct == 64) && a->io == KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    const int64_t tt = (int64_t)a->B * a->T;
    const int64_t ns = tt / ct + a->N;    // chunk slots (for chunk 64: pairs of 32-token chunks)
    if (2 * ns > INT32_MAX || (int64_t)a->HV > 65535) return KDA_ERR_UNSUPPORTED;
    // the 32-token prepare grid is up to (ns rounded up to 8) x (HV / H) workgroups wide
    if (ct == 32 && (ns + 8) * (int64_t)(a->HV / a->H) > INT32_MAX)
        return KDA_ERR_UNSUPPORTED;
    size_t cb;
    if (ct == 1)
        cb = 0;                      // the token-recurrent kernel needs no workspace
    else if (a->io == KDA_BF16 && ct == 64)
        cb = 2 * record_bytes<WsPair>(a->K, a->V);      // two 32-token records per slot
    else if (a->io == KDA_BF16)
        cb = ct == 32 ? record_bytes<WsBf16x32>(a->K, a->V) : record_bytes<WsBf16>(a->K, a->V);
    else
        cb = record_bytes<WsF32>(a->K, a->V);
    *T_total = tt;
    *n_slots = ns;
    *need = (size_t)ns * (size_t)a->HV * cb;
    *chunk = ct;
    const SplitPlan sp = split_plan(a, ct, *need);
    if (sp.c0 > 0) *need = sp.end;
    if (split) *split = sp;
    return KDA_OK;
}

// The pre-stage fields of the arguments (shared by the forward and the backward).
kda_status check_prestage(const kda_fwd_args *a)
{
    if (a->gate != KDA_GATE_NONE && a->gate != KDA_GATE_SOFTPLUS && a->gate != KDA_GATE_BOUNDED)
        return KDA_ERR_UNSUPPORTED;
    if (a->gate != KDA_GATE_NONE) {
        if (!a->A_log || ((uintptr_t)a->A_log & 3u)) return KDA_ERR_INVALID_ARG;
        if (a->dt_bias && !aligned16(a->dt_bias)) return KDA_ERR_INVALID_ARG;
        if (a->gate == KDA_GATE_BOUNDED &&
            !(a->gate_lower_bound < 0.f && a->gate_lower_bound > -INFINITY))
            return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

enum Stage { STAGE_PREPARE = 1, STAGE_STATE = 2, STAGE_BOTH = 3 };

template <int K, int V>
hipError_t dispatch(const FwdParams &p, int io, int chunk, int stages, hipStream_t st)
{
    hipError_t e;
    if (chunk == 1)     // token-recurrent: no prepare stage
        return (stages & STAGE_STATE) ? launch_recurrent<K, V>(p, io, st) : hipSuccess;
    const bool prep = (stages & STAGE_PREPARE) && p.seq.T_total > 0;
    if (io == KDA_BF16 && chunk == 64) {
        if (prep && (e = launch_prepare64_bf16<K, V>(p, st)) != hipSuccess) return e;
        return (stages & STAGE_STATE) ? launch_state64_bf16<K, V>(p, st) : hipSuccess;
    }
    if (io == KDA_BF16 && chunk == 32) {
        if (prep && (e = launch_prepare32_bf16<K, V>(p, st)) != hipSuccess) return e;
        return (stages & STAGE_STATE) ? launch_state32_bf16<K, V>(p, st) : hipSuccess;
    }
    if (io == KDA_BF16) {
        if (prep && (e = launch_prepare_bf16<K, V>(p, st)) != hipSuccess) return e;
        return (stages & STAGE_STATE) ? launch_state_bf16<K, V>(p, st) : hipSuccess;
    }
    if (prep && (e = launch_prepare_f32<K, V>(p, st)) != hipSuccess) return e;
    return (stages & STAGE_STATE) ? launch_state_f32<K, V>(p, st) : hipSuccess;
}

kda_status run_stages(const kda_fwd_args *a, void *workspace, size_t ws_bytes, void *stream,
                      int stages)
{
    int64_t tt, ns;
    size_t need;
    int ct;
    SplitPlan sp;
    const kda_status st = check_shapes(a, &tt, &ns, &need, &ct, &sp);
    if (st != KDA_OK) return st;
    if (a->N > 0 || tt > 0) {
        const void *ptrs[] = {a->q, a->k, a->v, a->g, a->beta, a->o};
        for (const void *ptr : ptrs)
            if (tt > 0 && (!ptr || !aligned16(ptr))) return KDA_ERR_INVALID_ARG;
    }
    if (a->initial_state && !aligned16(a->initial_state)) return KDA_ERR_INVALID_ARG;
    if (a->final_state && !aligned16(a->final_state)) return KDA_ERR_INVALID_ARG;
    if (a->cu_seqlens && !aligned16(a->cu_seqlens)) return KDA_ERR_INVALID_ARG;
    const kda_status ps = check_prestage(a);
    if (ps != KDA_OK) return ps;
    if (tt > 0 && need > 0 && (!workspace || ws_bytes < need || ((uintptr_t)workspace & 255u)))
        return KDA_ERR_WORKSPACE;
    if (a->N == 0) return KDA_OK;

    FwdParams p;
    p.seq.cu = a->cu_seqlens;
    p.seq.T = a->T;
    p.seq.T_total = tt;
    p.seq.N = a->N;
    p.seq.n_slots = (int32_t)ns;
    p.H = a->H;
    p.HV = a->HV;
    p.G = a->HV / a->H;
    p.scale = (a->scale > 0.f && !isnan(a->scale)) ? a->scale : 1.0f / sqrtf((float)a->K);
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.g = a->g;
    p.beta = a->beta;
    p.h0 = a->initial_state;
    p.o = a->o;
    p.ht = a->final_state;
    p.ws = (uint8_t *)workspace;
    p.pre.qk_l2norm = a->qk_l2norm != 0;
    p.pre.beta_sigmoid = a->beta_sigmoid != 0;
    p.pre.gate = a->gate;
    p.pre.lower_bound = a->gate_lower_bound;
    p.pre.A_log = a->A_log;
    p.pre.dt_bias = a->dt_bias;
    if (sp.c0 > 0) {
        uint8_t *w = (uint8_t *)workspace;
        p.split.c0 = sp.c0;
        p.split.nb = sp.nb;
        p.split.smf = (_Float16 *)(w + sp.smf);
        p.split.phf = (_Float16 *)(w + sp.phf);
        p.split.s0 = (float *)(w + sp.s0);
        p.split.o0 = (_Float16 *)(w + sp.o0);
        p.split.y = (_Float16 *)(w + sp.y);
    }

    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (a->K == 64)
        e = a->V == 64 ? dispatch<64, 64>(p, a->io, ct, stages, s)
                       : dispatch<64, 128>(p, a->io, ct, stages, s);
    else
        e = a->V == 64 ? dispatch<128, 64>(p, a->io, ct, stages, s)
                       : dispatch<128, 128>(p, a->io, ct, stages, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Backward workspace: the fp32 chunk records, then S at the start and Lam at the end of every
// chunk slot, then (G > 1 or q/k L2 norm) per-value-head dq and dk, then (gate on) per-chunk
// partials of dA_log and dt_bias. Offsets in bytes, each 256-aligned.
struct BwdLayout {
    size_t rec, ck_S, ck_L, part_q, part_k, part_A, part_dt, total;
};

// Shape checks of the backward (the forward's, at chunk 16) and its workspace layout.
kda_status check_bwd(const kda_fwd_args *a, int64_t *T_total, int64_t *n_slots, BwdLayout *L)
{
    if (!a) return KDA_ERR_INVALID_ARG;
    if (a->chunk != 0 && a->chunk != 16) return KDA_ERR_UNSUPPORTED;
    kda_fwd_args c = *a;
    c.chunk = 16;
    size_t rec;
    int ct;
    const kda_status st = check_shapes(&c, T_total, n_slots, &rec, &ct);
    if (st != KDA_OK) return st;
    rec = (size_t)*n_slots * (size_t)a->HV * record_bytes<WsF32B>(a->K, a->V);  // fp32 records
    const size_t slots = (size_t)*n_slots * (size_t)a->HV;
    const size_t state = slots * (size_t)a->K * (size_t)a->V * 4;
    const bool qk_part = a->HV > a->H || a->qk_l2norm;
    const size_t part = qk_part ? (size_t)*T_total * (size_t)a->HV * (size_t)a->K * 4 : 0;
    const bool gated = a->gate != KDA_GATE_NONE;
    L->rec = 0;
    L->ck_S = align256(rec);
    L->ck_L = L->ck_S + align256(state);
    L->part_q = L->ck_L + align256(state);
    L->part_k = L->part_q + align256(part);
    L->part_A = L->part_k + align256(part);
    L->part_dt = L->part_A + (gated ? align256(slots * 4) : 0);
    L->total = L->part_dt + (gated ? align256(slots * (size_t)a->K * 4) : 0);
    return KDA_OK;
}

template <int K, int V>
hipError_t dispatch_bwd(const BwdParams &b, int io, hipStream_t st)
{
    return launch_backward<K, V>(b, io == KDA_BF16, st);
}

}  // namespace

extern "C" {

size_t kda_bwd_workspace_bytes(const kda_fwd_args *a)
{
    int64_t tt, ns;
    BwdLayout L;
    if (check_bwd(a, &tt, &ns, &L) != KDA_OK) return 0;
    return L.total;
}

kda_status kda_bwd(const kda_fwd_args *a, const void *d_o, const float *dht, void *workspace,
                   size_t ws_bytes, float *dq, float *dk, float *dv, float *dg, float *dbeta,
                   float *dh0, float *dA_log, float *ddt_bias, void *stream)
{
    int64_t tt, ns;
    BwdLayout L;
    kda_status st = check_bwd(a, &tt, &ns, &L);
    if (st != KDA_OK) return st;
    if ((st = check_prestage(a)) != KDA_OK) return st;
    if (a->gate != KDA_GATE_NONE &&
        (!dA_log || ((uintptr_t)dA_log & 3u) || (ddt_bias && !aligned16(ddt_bias))))
        return KDA_ERR_INVALID_ARG;
    if (tt > 0) {
        const void *ptrs[] = {a->q, a->k, a->v, a->g, a->beta, d_o, dq, dk, dv, dg, dbeta};
        for (const void *ptr : ptrs)
            if (!ptr || !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    }
    const void *opt[] = {a->initial_state, a->cu_seqlens, dht, dh0};
    for (const void *ptr : opt)
        if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    if (tt > 0 && (!workspace || ws_bytes < L.total || ((uintptr_t)workspace & 255u)))
        return KDA_ERR_WORKSPACE;
    if (a->N == 0) return KDA_OK;

    BwdParams b = {};
    FwdParams &p = b.f;
    p.seq.cu = a->cu_seqlens;
    p.seq.T = a->T;
    p.seq.T_total = tt;
    p.seq.N = a->N;
    p.seq.n_slots = (int32_t)ns;
    p.H = a->H;
    p.HV = a->HV;
    p.G = a->HV / a->H;
    p.scale = (a->scale > 0.f && !isnan(a->scale)) ? a->scale : 1.0f / sqrtf((float)a->K);
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.g = a->g;
    p.beta = a->beta;
    p.h0 = a->initial_state;
    p.o = nullptr;
    p.ht = nullptr;
    p.d_o = d_o;
    uint8_t *ws = (uint8_t *)workspace;
    p.ws = ws;
    p.pre.qk_l2norm = a->qk_l2norm != 0;
    p.pre.beta_sigmoid = a->beta_sigmoid != 0;
    p.pre.gate = a->gate;
    p.pre.lower_bound = a->gate_lower_bound;
    p.pre.A_log = a->A_log;
    p.pre.dt_bias = a->dt_bias;
    b.d_o = d_o;
    b.dht = dht;
    b.ck_S = ws ? (float *)(ws + L.ck_S) : nullptr;
    b.ck_L = ws ? (float *)(ws + L.ck_L) : nullptr;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.dg = dg;
    b.dbeta = dbeta;
    b.dh0 = dh0;
    const bool qk_part = p.G > 1 || p.pre.qk_l2norm;
    b.part_q = ws && qk_part ? (float *)(ws + L.part_q) : nullptr;
    b.part_k = ws && qk_part ? (float *)(ws + L.part_k) : nullptr;
    b.dA_log = dA_log;
    b.ddt_bias = ddt_bias;
    b.part_A = ws && p.pre.gate ? (float *)(ws + L.part_A) : nullptr;
    b.part_dt = ws && p.pre.gate ? (float *)(ws + L.part_dt) : nullptr;

    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (a->K == 64)
        e = a->V == 64 ? dispatch_bwd<64, 64>(b, a->io, s) : dispatch_bwd<64, 128>(b, a->io, s);
    else
        e = a->V == 64 ? dispatch_bwd<128, 64>(b, a->io, s)
                       : dispatch_bwd<128, 128>(b, a->io, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_fwd_workspace_bytes(const kda_fwd_args *a)
{
    int64_t tt, ns;
    size_t need;
    int ct;
    if (check_shapes(a, &tt, &ns, &need, &ct) != KDA_OK) return 0;
    return need;
}

kda_status kda_fwd(const kda_fwd_args *a, void *workspace, size_t ws_bytes, void *stream)
{
    return run_stages(a, workspace, ws_bytes, stream, STAGE_BOTH);
}

kda_status kda_fwd_prepare(const kda_fwd_args *a, void *workspace, size_t ws_bytes,
                           void *stream)
{
    return run_stages(a, workspace, ws_bytes, stream, STAGE_PREPARE);
}

kda_status kda_fwd_state(const kda_fwd_args *a, void *workspace, size_t ws_bytes, void *stream)
{
    return run_stages(a, workspace, ws_bytes, stream, STAGE_STATE);
}

const char *kda_strerror(int status)
{
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED:
        return "unsupported configuration (K, V in {64, 128}; chunk 1, 16, or 32 / 64 with bf16 "
               "io; gate 0, 1 or 2; the backward: chunk 16)";
    case KDA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case KDA_ERR_HIP: return "HIP kernel launch failed";
    case KDA_ERR_NOALLOC_TOO_LARGE:
        return "shapes need more workspace than kda_fwd_noalloc's static device array "
               "(KDA_NOALLOC_WORKSPACE_BYTES = 128 MiB)";
    default: return "unknown status";
    }
}

int kda_version(void) { return 105; }

}  // extern "C"
