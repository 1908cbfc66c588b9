// kda_recurrent.hip -- the token-recurrent forward (chunk = 1): the KDA recurrence itself, one
// token after another, for decoding and other short sequences where a chunk's fixed cost
// (a 16- or 32-token WY block and a workspace round trip) would dominate.
//
// Per token t of a sequence, for value head j and q/k head h ("手撕KDA" section 1: the
// recurrence that a one-token chunk of naive_chunk_kda reduces to; "手撕KDA" section 5 names
// this form, fused_recurrent_kda, as the cross-check of the chunked kernels):
//     S <- diag(exp g_t) S;   r = v_t - S^T k_t;   S <- S + beta_t k_t r^T;   o_t = scale S^T q_t
//
// One wave per (sequence, value head, 64 value columns); lane c keeps column c of S (K fp32
// values) in registers for the whole sequence, so every product is a per-lane loop over the key
// dimension with no cross-lane reduction. Per token the wave first stages q, k, exp(g) (and
// beta k) of the token in LDS — one coalesced load per lane per tensor — and then every lane
// reads them back as broadcast vector loads. The state is read once at the start and written
// once at the end, column-contiguous across lanes (coalesced 256-byte rows).
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ void st_io(uint16_t *p, int64_t i, float x) {
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ void st_io(float *p, int64_t i, float x) { p[i] = x; }

template <int K>
struct TokenRow {
    f32x4 qkeb[K];               // per key dim: q, k, exp(g), beta * k
};

// What one token contributes, as stored (raw io values), for lane l: key dims l, l + 64, ...
// and its value column.
template <int KL, typename T>
struct TokenIn {
    T q[KL], k[KL], g[KL], b, v;
};

}  // namespace

template <int K, int V, typename T>
__global__ __launch_bounds__(64) void recurrent_kernel(FwdParams p)
{
    static_assert(V % 64 == 0, "one lane per value column, 64 columns per wave");
    constexpr int NW = V / 64;                       // waves per (sequence, value head)
    __shared__ TokenRow<K> row;
    const int lane = threadIdx.x;
    const int unit = blockIdx.x / NW, part = blockIdx.x % NW;
    const int j = unit % p.HV, s = unit / p.HV;
    if (s >= p.seq.N) return;
    const int h = j / p.G;
    const int col = part * 64 + lane;
    const int64_t bos = seq_bos(p.seq, s), eos = seq_eos(p.seq, s, bos);
    const T *q = (const T *)p.q, *k = (const T *)p.k, *v = (const T *)p.v;
    const T *g = (const T *)p.g, *beta = (const T *)p.beta;
    T *o = (T *)p.o;
    // this wave's 64 columns of S[s, j] through a buffer resource: per key dim the offset is
    // the scalar kk * V * 4 plus the lane's 4 * lane, so no per-load address arithmetic
    const size_t st_off = ((size_t)s * p.HV + j) * (size_t)K * V + part * 64;
    const uint32_t st_bytes = (uint32_t)(((K - 1) * V + 64) * 4);

    // pre-stage gate parameters of this lane's key dims (lane, lane + 64, ...)
    constexpr int KL = K / 64;
    const bool gated = p.pre.gate != 0;
    const float aexp = gated ? __builtin_amdgcn_exp2f(p.pre.A_log[j] * LOG2E) : 0.f;
    float dtl[KL];
#pragma unroll
    for (int u = 0; u < KL; ++u)
        dtl[u] = gated && p.pre.dt_bias ? p.pre.dt_bias[(size_t)j * K + lane + 64 * u] : 0.f;

    // the inputs of token t of this sequence, through resources over its rows only (a token
    // past the sequence end reads zeros and is never used): no load sits under a branch
    constexpr int SZ = (int)sizeof(T);
    auto load_token = [&](TokenIn<KL, T> &x, int64_t t) {
        const bool in = t < eos;
        const int64_t tc = in ? t : 0;
        const auto rq = buffer_rsrc(q + (tc * p.H + h) * K, in ? K * SZ : 0);
        const auto rk = buffer_rsrc(k + (tc * p.H + h) * K, in ? K * SZ : 0);
        const auto rg = buffer_rsrc(g + (tc * p.HV + j) * K, in ? K * SZ : 0);
        const auto rb = buffer_rsrc(beta + tc * p.HV + j, in ? SZ : 0);
        const auto rv = buffer_rsrc(v + (tc * p.HV + j) * V, in ? V * SZ : 0);
#pragma unroll
        for (int u = 0; u < KL; ++u) {
            bload_elem(rq, (lane + 64 * u) * SZ, x.q[u]);
            bload_elem(rk, (lane + 64 * u) * SZ, x.k[u]);
            bload_elem(rg, (lane + 64 * u) * SZ, x.g[u]);
        }
        bload_elem(rb, 0, x.b);
        bload_elem(rv, col * SZ, x.v);
    };
    // the first token's inputs go out before the state, so their latency is covered by it;
    // every later token's go out one token ahead
    TokenIn<KL, T> x;
    load_token(x, bos);

    float S[K];
    if (p.h0) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.h0 + st_off, st_bytes);
#pragma unroll
        for (int kk = 0; kk < K; ++kk)
            S[kk] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4,
                                                                         kk * V * 4, 0));
    } else {
#pragma unroll
        for (int kk = 0; kk < K; ++kk) S[kk] = 0.f;
    }

    for (int64_t t = bos; t < eos; ++t) {
        // this token's inputs (loaded one token earlier), then the next token's loads into the
        // same registers
        float b = to_f32(x.b), vt = to_f32(x.v);
        float qv[KL], kv[KL], gv[KL];
#pragma unroll
        for (int u = 0; u < KL; ++u) {
            qv[u] = to_f32(x.q[u]);
            kv[u] = to_f32(x.k[u]);
            gv[u] = to_f32(x.g[u]);
        }
        load_token(x, t + 1);
        if (p.pre.beta_sigmoid) b = sigmoid_f(b);
        // stage this token's q, k, exp(g), beta k: lane l takes key dims l, l + 64, ...
        if (gated) {
#pragma unroll
            for (int u = 0; u < KL; ++u) gv[u] = gate_activation(p.pre, gv[u] + dtl[u], aexp);
        }
        if (p.pre.qk_l2norm) {          // pre-stage: the token's q and k over all K dims
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int u = 0; u < KL; ++u) {
                sq += qv[u] * qv[u];
                sk += kv[u] * kv[u];
            }
            const float rq = l2norm_factor(wave_sum(sq)), rk = l2norm_factor(wave_sum(sk));
#pragma unroll
            for (int u = 0; u < KL; ++u) {
                qv[u] *= rq;
                kv[u] *= rk;
            }
        }
#pragma unroll
        for (int u = 0; u < KL; ++u)
            row.qkeb[lane + 64 * u] =
                f32x4{qv[u], kv[u], __builtin_amdgcn_exp2f(gv[u] * LOG2E), b * kv[u]};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();        // one wave: orders the stage before the reads
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        // (the loops are unrolled so that S stays in registers; the scheduling barriers every
        // 8 key dims keep the broadcast reads from being hoisted all at once)
        float kS = 0.f;
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            const f32x4 e = row.qkeb[kk];
            S[kk] *= e[2];
            kS += e[1] * S[kk];
            if (kk % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
        const float r = vt - kS;
        float os = 0.f;
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            const f32x4 e = row.qkeb[kk];
            S[kk] += e[3] * r;
            os += e[0] * S[kk];
            if (kk % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
        st_io(o, (t * p.HV + j) * V + col, p.scale * os);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();        // reads done before the next token's stage
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    if (p.ht) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.ht + st_off, st_bytes);
#pragma unroll
        for (int kk = 0; kk < K; ++kk)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[kk]), rs, lane * 4,
                                                  kk * V * 4, 0);
    }
}

template <int K, int V>
hipError_t launch_recurrent(const FwdParams &p, int io, hipStream_t st)
{
    constexpr int NW = V / 64;
    const int64_t nblk = (int64_t)p.seq.N * p.HV * NW;
    if (nblk == 0) return hipSuccess;
    if (io == 0)
        recurrent_kernel<K, V, uint16_t><<<dim3((unsigned)nblk), dim3(64), 0, st>>>(p);
    else
        recurrent_kernel<K, V, float><<<dim3((unsigned)nblk), dim3(64), 0, st>>>(p);
    return hipGetLastError();
}

#define KDA_INST(K, V) \
    template hipError_t launch_recurrent<K, V>(const FwdParams &, int, hipStream_t);
KDA_INST(64, 64)
KDA_INST(64, 128)
KDA_INST(128, 64)
KDA_INST(128, 128)
#undef KDA_INST

}  // namespace kda
