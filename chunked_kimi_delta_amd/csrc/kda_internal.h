// kda_internal.h -- device-side building blocks of libkda_fwd (gfx950 / CDNA4 only).
//
// Layout vocabulary used by every kernel (wave64, 16x16 MFMA tiles; g = lane / 16 is the
// lane group, r or n = lane % 16 the lane within its 16-lane row):
//   C-layout    of a 16x16 fp32 tile X: lane (g, n) holds X[4g + i][n], i = 0..3. This is
//               the accumulator layout of v_mfma_f32_16x16x{16,32}_{bf16,f16}.
//   A16-layout  (16x16x16 A operand): lane (g, m) holds X[m][4g + i], i = 0..3.
//   B16-layout  (16x16x16 B operand): lane (g, n) holds X[4g + i][n] == C-layout.
//   A32/B32     (16x16x32): lane (g, m) holds X[m][kappa = 8g .. 8g + 7] (A) and
//               X[kappa = 8g .. 8g + 7][n] (B).
//   Two identities follow and are used throughout: the registers of C(X) ARE the A16-layout
//   of X^T, so an MFMA with A = C(X) and B = I produces C(X^T) (a register transpose on the
//   matrix core); and C-layout == B16-layout, so a product's accumulator feeds the next
//   product as B without moving data between lanes.
//   TPL         "token per lane": lane (g, r) holds row (token) r, columns 16c + 4g + i for
//               every 16-column tile c. It is the A16-layout of every tile, and step s of a
//               16x16x32 product over the column axis pairs tiles (2s, 2s+1):
//               kappa = 8g + e  <->  column 16(2s + e/4) + 4g + e%4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int CHUNK = 16;
constexpr float LOG2E = 1.4426950408889634f;

// ----------------------------------------------------------------------------- parameters

// Sequence geometry shared by both kernels. Sequence s covers tokens [bos_s, eos_s) of the
// packed token axis; with chunks of CT tokens its chunk c lives in workspace slot
// floor(bos_s / CT) + s + c. The map is injective and every slot is < T_total / CT + N (so the
// prepare grid is that bound).
struct SeqGeom {
    const int64_t *cu;   // device [N + 1] or nullptr (dense: bos_s = s * T)
    int64_t T;           // dense per-sequence length
    int64_t T_total;     // tokens on the packed axis (B * T)
    int32_t N;           // sequences
    int32_t n_slots;     // T_total / CT + N
};

// Pre-stage of the raw inputs (q/k L2 norm, beta sigmoid, gate activation), applied by every
// kernel that reads q, k, g or beta.
struct Prestage {
    int32_t qk_l2norm, beta_sigmoid, gate;   // gate: 0 none, 1 softplus, 2 bounded sigmoid
    float lower_bound;
    const float *A_log;                      // [HV]
    const float *dt_bias;                    // [HV, K] or nullptr
};

// Two-segment state pass of the 32-token path, for dense batches whose state slices would
// leave at least half of the compute units idle: segment A (chunks [0, c0)) runs from the
// initial state as usual and leaves its end state S_A in s_mid; at the same time segment B
// (chunks [c0, c0 + nb)) runs from a zero state, and next to it its transition from the
// identity (the K x K state of the same recurrence with U = 0). The state is affine in the
// state at a segment's start ("手撕KDA" section 1: S_c = diag(e^gam) S + KR^T (U - W S) per
// chunk), so for every token of B the output is o0 + y S_A and the final state is
// S0_end + phi S_A, which a third kernel forms. S_A and phi are kept as the fp16 operand
// fragments of those products (the precision of the chain's own S operand).
struct Split32 {
    int32_t c0 = 0;             // chunks of segment A; 0: one segment
    int32_t nb = 0;             // chunks of segment B (the same for every sequence)
    _Float16 *smf = nullptr;    // [N][HV][V/16][K/32][64 lanes][8]: S_A as 16x16x32 B operands
                                // (lane (g, n): rows 32 t + 16 (e / 4) + 4g + e % 4, column n)
    _Float16 *phf = nullptr;    // [N][HV][K/16 row tiles][K/16 column slices][64][4]: phi tile
                                // transposed (lane (g, m): row m, columns 4g .. 4g + 3)
    float *s0 = nullptr;        // [N][HV][K][V] segment B's end state from zero (final_state
                                // is written only by the correction, after every read of
                                // initial_state, so the two may be one buffer)
    _Float16 *o0 = nullptr;     // [N][HV][nb][2 blocks][V/16][64 lanes][4] C(O^T) from zero
    _Float16 *y = nullptr;      // [N][HV][nb][2][K/16][64][4] C(Y^T): the transition's output
};

struct FwdParams {
    SeqGeom seq;
    int32_t H, HV, G;
    float scale;
    const void *q, *k, *v, *g, *beta;
    const float *h0;
    void *o;
    float *ht;
    uint8_t *ws;
    Prestage pre;
    const void *d_o = nullptr;   // backward only: d loss / d o, copied into the chunk records
    Split32 split;
};

// Arguments of the backward: the forward's (f.ws holds the fp32 chunk records), the incoming
// gradients, the per-chunk state records and the gradient outputs (all fp32).
struct BwdParams {
    FwdParams f;
    const void *d_o;          // d loss / d o, [T_total][HV][V] in the input storage type
    const float *dht;         // d loss / d final_state, [N][HV][K][V] or null (zero)
    float *ck_S, *ck_L;       // [HV][n_slots][K][V]: S at the start / Lam at the end of a chunk
    float *dq, *dk;           // [T_total][H][K]
    float *dv;                // [T_total][HV][V]
    float *dg;                // [T_total][HV][K]
    float *dbeta;             // [T_total][HV]
    float *dh0;               // [N][HV][K][V] or null
    float *part_q, *part_k;   // [T_total][HV][K] per-value-head dq, dk of the activated q, k
                              // (G > 1 or q/k L2 norm; else null and dq, dk are written
                              // directly)
    float *dA_log;            // [HV] gradient of A_log (gate on)
    float *ddt_bias;          // [HV][K] gradient of dt_bias (gate on), or null
    float *part_A, *part_dt;  // [HV][n_slots], [HV][n_slots][K]: per-chunk parameter partials
};

// Workspace of one (value head, slot) chunk, bf16 io. All fragments are stored in the exact
// per-lane order the state kernel's MFMAs consume, so every state-kernel load is a contiguous
// 64-lane vector load:
//   W   [K/32][64 lanes][8] fp16   w in TPL; step s holds tiles (2s, 2s+1)
//   QD  [K/32][64][8]       fp16   scale * q * exp(Gam), same order
//   KR  [K/32][64][8]       fp16   k * exp(gam - Gam) in C-layout of each 16-key-dim tile
//                                  (= A16-layout of KR^T); pair s holds tiles (2s, 2s+1)
//   U   [V/16][64][4]       fp16   u = A v in C-layout (rows = tokens), one 16-column slice
//   MQK [64][4]             fp16   Mqk in A16-layout
//   EG  [K]                 fp32   exp(gam), natural key-dim order
template <int K, int V>
struct WsBf16 {
    static constexpr int W = 0;
    static constexpr int QD = W + 32 * K;
    static constexpr int KR = QD + 32 * K;
    static constexpr int U = KR + 32 * K;
    static constexpr int MQK = U + 32 * V;
    static constexpr int EG = MQK + 512;
    static constexpr int END = EG + 4 * K;
    static constexpr int BYTES = (END + 255) / 256 * 256;
};

// Workspace of one (value head, slot) 32-token chunk, bf16 io. The chunk is two 16-token row
// blocks a (tokens 0..15) and b (16..31). Products over the 32 tokens use 16x16x32 MFMAs whose
// reduction index pairs the blocks: kappa = 8g + e is token 4g + e of block a for e < 4 and
// token 4g + e - 4 of block b for e >= 4.
//   W    [2 blocks][K/32][64][8] fp16   W rows of each block in TPL (as WsBf16::W)
//   QD   [2][K/32][64][8]        fp16
//   KR   [K/16][64][8]           fp16   KR^T tile t as a 16x16x32 A operand over the 32 tokens
//   NU   [V/16][64][8]           fp16   -U in C-layout per 16-column slice, block a in
//                                       elements 0..3 and block b in 4..7 of each lane's 16
//                                       bytes (negated: the state kernel starts its W S
//                                       accumulator from it, so delta = -(W S - U) needs no
//                                       subtraction)
//   MQKA [64][4]                 fp16   Mqk_aa in A16-layout
//   MQKB [64][8]                 fp16   [Mqk_ba | Mqk_bb] as a 16x16x32 A operand
//   EG   [K]                     fp32   exp(gamma) of the whole 32-token chunk
template <int K, int V>
struct WsBf16x32 {
    static constexpr int W = 0;
    static constexpr int QD = W + 64 * K;
    static constexpr int KR = QD + 64 * K;
    static constexpr int NU = KR + 64 * K;
    static constexpr int MQKA = NU + 64 * V;
    static constexpr int MQKB = MQKA + 512;
    static constexpr int EG = MQKB + 1024;
    static constexpr int END = EG + 4 * K;
    static constexpr int BYTES = (END + 255) / 256 * 256;
};

// The 64-token step of the state kernel reads the records of two consecutive 32-token chunks
// (c, c + 1) of one sequence, stored side by side, each a WsBf16x32 record followed by
//   PT   [2 blocks][64][8] fp16   (second chunk only) P = W_{c+1} KR_c^T (32 x 32) as the
//                                 16x16x32 A operand of each row block, the reduction pairing
//                                 chunk c's blocks as in WsBf16x32
// and the second chunk's W is stored scaled by e^{gam_c} per key dim, so that
//     delta_{c+1} = U_{c+1} - (W_{c+1} diag(e^{gam_c})) S_c - P delta_c
// needs only the state at the start of the pair.
template <int K, int V>
struct WsPair {
    static constexpr int PT = WsBf16x32<K, V>::END;
    static constexpr int END = PT + 2048;
    static constexpr int BYTES = (END + 255) / 256 * 256;
};

// Workspace of one chunk, fp32 io: plain row-major fp32 arrays.
//   W [16][K], QD [16][K], KR [16][K], U [16][V], MQK [16][16], EG [K]
template <int K, int V>
struct WsF32 {
    static constexpr int W = 0;
    static constexpr int QD = W + 64 * K;
    static constexpr int KR = QD + 64 * K;
    static constexpr int U = KR + 64 * K;
    static constexpr int MQK = U + 64 * V;
    static constexpr int EG = MQK + 1024;
    static constexpr int END = EG + 4 * K;
    static constexpr int BYTES = (END + 255) / 256 * 256;
};

// The backward's fp32 chunk record: WsF32 followed by the inverse X = (I + L)^{-1} and the
// strictly lower Gram G (L = diag(beta) G), both [16][16] fp32 row-major, and the chunk's dO.
template <int K, int V>
struct WsF32B : WsF32<K, V> {
    static constexpr int XM = WsF32<K, V>::END;
    static constexpr int GM = XM + 1024;
    // dO of the chunk's 16 rows in fp32, C-layout per 16-column slice ([V/16][64 lanes][4]:
    // lane (g, r) holds rows 4g .. 4g + 3 of column 16 n + r), rows past the sequence end zero
    static constexpr int DO = GM + 1024;
    static constexpr int END = DO + 16 * V * 4;
    static constexpr int BYTES = (END + 255) / 256 * 256;
};

// ----------------------------------------------------------------------------- sequences

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ int64_t seq_bos(const SeqGeom &sg, int s) {
    const int64_t b = sg.cu ? sg.cu[s] : (int64_t)s * sg.T;
    return clamp64(b, 0, sg.T_total);
}

__device__ __forceinline__ int64_t seq_eos(const SeqGeom &sg, int s, int64_t bos) {
    const int64_t e = sg.cu ? sg.cu[s + 1] : (int64_t)(s + 1) * sg.T;
    return clamp64(e, bos, sg.T_total);
}

template <int CT = CHUNK>
__device__ __forceinline__ int64_t slot_base(const SeqGeom &sg, int s) {
    return seq_bos(sg, s) / CT + s;
}

// Slot -> (sequence, chunk start, valid rows) for chunks of CT tokens. Binary search for the
// last sequence whose first slot is <= slot (the first-slot map is nondecreasing for valid
// offsets; for invalid ones the search still ends inside [0, N)). Returns false for slots that
// hold no chunk. Every lane computes the same values (uniform addresses).
template <int CT = CHUNK>
__device__ __forceinline__ bool locate_slot(const SeqGeom &sg, int slot, int *s_out,
                                            int64_t *bos_out, int *nvalid_out) {
    if (sg.N <= 0) return false;
    int lo = 0, hi = sg.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_base<CT>(sg, mid) <= slot) lo = mid; else hi = mid - 1;
    }
    const int64_t bos_s = seq_bos(sg, lo);
    const int64_t eos_s = seq_eos(sg, lo, bos_s);
    const int64_t c = (int64_t)slot - (bos_s / CT + lo);
    const int64_t nc = (eos_s - bos_s + CT - 1) / CT;
    if (c < 0 || c >= nc) return false;
    *s_out = lo;
    *bos_out = bos_s + CT * c;
    const int64_t nv = eos_s - *bos_out;
    *nvalid_out = (int)(nv < CT ? nv : CT);
    return true;
}

// Workgroup -> (unit = sequence * HV + value head, sub-slice in [0, NV)). Workgroups are
// dispatched to the 8 XCDs round-robin (workgroup w runs on XCD w % 8), and each XCD has its
// own L2. The map keeps all NV workgroups of one unit on one XCD so the chunk operands they
// share are fetched into that L2 once. The grid is padded to a multiple of 8 units; units
// beyond N*HV return false.
__device__ __forceinline__ bool state_unit(int wg, int NV, int units, int *unit, int *slice) {
    const int xcd = wg & 7, idx = wg >> 3;
    *unit = (idx / NV) * 8 + xcd;
    *slice = idx % NV;
    return *unit < units;
}

// ----------------------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
    return __uint_as_float((uint32_t)x << 16);
}
// an io element as fp32 (fp32 io, or bf16 bits)
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }

// four consecutive bf16 (8 bytes) -> fp32
__device__ __forceinline__ void unpack_bf16x4(uint2 raw, float out[4]) {
    out[0] = bf16lo(raw.x); out[1] = bf16hi(raw.x);
    out[2] = bf16lo(raw.y); out[3] = bf16hi(raw.y);
}

__device__ __forceinline__ bf16x4 to_bf16x4(const float x[4]) {
    bf16x4 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    return r;
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    bf16x4 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    return r;
}
__device__ __forceinline__ f16x4 to_f16x4(const float x[4]) {
    f16x4 r;
    r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
    return r;
}
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) {
    f16x4 r;
    r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
    return r;
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 cat(f16x4 a, f16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ----------------------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Vector loads through a buffer resource: the address is resource base (scalar) + soffset
// (scalar) + voffset (per lane), so per-chunk address arithmetic stays on the scalar unit.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef float f32v2 __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
template <int AUX = 0>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
}
// One io element (fp32, or bf16 bits) through a buffer resource: loads past its range read 0.
__device__ __forceinline__ void bload_elem(__amdgpu_buffer_rsrc_t r, int voff, float &x) {
    x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
__device__ __forceinline__ void bload_elem(__amdgpu_buffer_rsrc_t r, int voff, uint16_t &x) {
    x = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}
// A resource over the first `rows` rows (of `row_elems` elements, `row_stride` elements apart)
// from `base`: the rows after them read as zero.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_in(const T *base, int rows,
                                                          int64_t row_stride, int row_elems) {
    return buffer_rsrc(base, rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * row_stride + row_elems) *
                                                   (int64_t)sizeof(T))
                                      : 0u);
}
// Stores through a buffer resource with cache policy AUX; stores past the resource's size are
// dropped. A 16-byte store goes out as two 8-byte stores: behind a store with 128-bit data the
// compiler has scheduled a VALU write of one of its data registers, and the store then wrote
// the new value for some lanes (stores of at most 64 bits of data have shown no such loss).
template <int AUX, class T>
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, int voff, int soff, T v) {
    static_assert(sizeof(T) == 16, "16-byte store");
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, r, voff, soff, AUX);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[2], w[3]}, r, voff, soff + 8, AUX);
}
template <int AUX, class T>
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, int voff, int soff, T v) {
    static_assert(sizeof(T) == 8, "8-byte store");
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, AUX);
}

// 16x16x16 product on the fp32 matrix core: D = A B + C with A in A16-layout and B in
// B16-layout (fp32, one value per i), as four v_mfma_f32_16x16x4_f32. Instruction i contracts
// the columns 4g + i of A with the rows 4g + i of B (its k index is the lane group g), so the
// A16/B16/C register roles of the 16-bit products carry over unchanged.
__device__ __forceinline__ f32x4 mm16_f32(f32x4 a, f32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// ----------------------------------------------------------------------------- lanes

// Inclusive prefix sum over the 16 lanes of each DPP row (lane % 16 = token index). Lanes
// shifted in from outside the row contribute 0.
__device__ __forceinline__ float row_inclusive_scan(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    return x;
}

// Sum of x over the four lanes of a wave that share lane % 16 (the four lane groups).
__device__ __forceinline__ float sum_lane_groups(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Sum of x over the 64 lanes of a wave (every lane gets the sum).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// value of x held by lane `src` (0..63)
__device__ __forceinline__ float lane_read(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// ----------------------------------------------------------------------------- pre-stage

constexpr float LN2 = 0.6931471805599453f;
constexpr float L2NORM_EPS = 1e-6f;

// 1 / (1 + e^-x) from the base-2 exponential; 0 and 1 at the extremes, never NaN.
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * LOG2E));
}

// log(1 + e^x) as max(x, 0) + log(1 + e^-|x|): no overflow; absolute error about 1e-7, which
// is what a log decay needs (exp(g) then has relative error about 1e-7).
__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.f) +
           LN2 * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * LOG2E));
}

// The gate activation on x = g + dt_bias with a = exp(A_log) of the value head (pre.gate != 0).
__device__ __forceinline__ float gate_activation(const Prestage &pre, float x, float a) {
    return pre.gate == 1 ? -a * softplus_f(x) : pre.lower_bound * sigmoid_f(a * x);
}

// 1 / sqrt(sum of squares + eps): the L2-norm factor of a q or k row.
__device__ __forceinline__ float l2norm_factor(float sumsq) {
    return __builtin_amdgcn_rsqf(sumsq + L2NORM_EPS);
}

// ----------------------------------------------------------------------------- exact Gram

// The bf16 prepare kernels factor e^{Gam_i - Gam_j} = e^{Gam_i - ref} e^{ref - Gam_j} around a
// reference token of the chunk. The factors of a block's diagonal Gram products then span
// 2^{+-span}, span the decay (log2 units) between the reference and the block's far end; the
// kept products (j <= i) are at most 1 and the discarded upper triangle at most 2^span. Up to
// span 100 every factor, the low bf16 part of its hi + lo split (about 2^-9 of it, so at least
// about 2^-119 |k|) and every sum stay in the normal fp32 / bf16 range; beyond it the small
// factors' low parts would turn subnormal, and the block's diagonal products are formed by
// exact_block_gram instead.
constexpr float FACTOR_SPAN_MAX = 100.f;

// Lane I of each 16-lane DPP row, broadcast to the whole row (row_newbcast).
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_amdgcn_update_dpp(0.f, x, 0x150 + I, 0xf, 0xf, false);
}

// e^{gam} of the state rows a lane holds, for NT 16-row tiles: `raw` is one 16-byte load in
// which lane (g, n) read the four values of tile n % NT for its lane group g (rows
// 16 t + 4 g .. + 3); tile t's values are then broadcast from lane (g, t) to the row. One
// load of 256 distinct bytes per NT tiles instead of NT loads that each fetch 64 lanes x 16 B
// for 64 distinct bytes.
template <int... T>
__device__ __forceinline__ void expand_rows_impl(u32x4 raw, f32x4 (&eg)[sizeof...(T)],
                                                 std::integer_sequence<int, T...>) {
    const f32x4 x = __builtin_bit_cast(f32x4, raw);
    ((eg[T] = f32x4{row_bcast<T>(x[0]), row_bcast<T>(x[1]), row_bcast<T>(x[2]),
                    row_bcast<T>(x[3])}), ...);
}
template <int NT>
__device__ __forceinline__ void expand_rows(u32x4 raw, f32x4 (&eg)[NT]) {
    expand_rows_impl(raw, eg, std::make_integer_sequence<int, NT>{});
}

// One 16-token block's rows of q, k, g as stored in the inputs.
struct BlockRows {
    const uint16_t *q, *k, *g;    // element 0 of the block's first token (this head)
    int64_t qk_stride, g_stride;  // elements between consecutive tokens
    int nrows;                    // valid rows; later rows read as zero (k = q = 0, g = 0)
};

// Column step I of exact_block_gram: this lane is column r (its own token) of the block; E
// carries e^{Gam_I - Gam_r} for I >= r (0 above the diagonal) along the lane's key dims, as the
// running product of the per-token decays e^{g} of tokens r+1 .. I, broadcast from lane I.
template <int I>
__device__ __forceinline__ void exact_gram_step(float (&E)[4], const float (&a)[4],
                                                const float (&kk)[4], const float (&qq)[4],
                                                int r, float (&Lp)[16], float (&Mp)[16]) {
    const float ind = r == I ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        E[e] = fmaf(E[e], row_bcast<I>(a[e]), ind);
        const float t = E[e] * kk[e];
        Lp[I] = fmaf(t, row_bcast<I>(kk[e]), Lp[I]);
        Mp[I] = fmaf(t, row_bcast<I>(qq[e]), Mp[I]);
    }
}

template <int... I>
__device__ __forceinline__ void exact_gram_steps(float (&E)[4], const float (&a)[4],
                                                 const float (&kk)[4], const float (&qq)[4],
                                                 int r, float (&Lp)[16], float (&Mp)[16],
                                                 std::integer_sequence<int, I...>) {
    (exact_gram_step<I>(E, a, kk, qq, r, Lp, Mp), ...);
}

// Sums x[4g + i] over the four lane groups g' of a lane's column, keeping rows 4g .. 4g + 3 on
// lane group g: a reduce-scatter whose result is the C-layout of the 16 x 16 matrix whose
// column n lane (g', n) holds partial sums of in x[0..15].
__device__ __forceinline__ f32x4 reduce_scatter_rows(const float (&x)[16], int grp) {
    const bool hi = grp >= 2, lo = grp & 1;
    float kept[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float mine = hi ? x[8 + k] : x[k];
        const float send = hi ? x[k] : x[8 + k];
        kept[k] = mine + __shfl_xor(send, 32);
    }
    f32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float mine = lo ? kept[4 + i] : kept[i];
        const float send = lo ? kept[i] : kept[4 + i];
        out[i] = mine + __shfl_xor(send, 16);
    }
    return out;
}

// The diagonal Gram products of one 16-token block, with every decay an exact product of
// per-token decays (no factorisation, so no exponent range limit): in C-layout,
//     Lc  = [ sum_d k_i k_j e^{Gam_i - Gam_j} ]_{i >= j}      (the caller keeps i > j, scales by
//                                                            beta_i)
//     Mc  = [ sum_d sq_i q_i k_j e^{Gam_i - Gam_j} ]_{i >= j}
// with i the row (token of the block), j the column, k and q of each token multiplied by rk
// and sq of that token (the L2-norm factor and, for q, the output scale), and g the activated
// per-token log decay (the pre-stage gate, when on, applied as in the kernels). Entries above
// the diagonal are zero. Each lane reloads its own token's q, k, g (TPL, rows past nrows read
// as zero) one 16-dim tile at a time, so nothing the caller keeps in registers is needed.
// "手撕KDA" section 1 (naive_chunk_kda) forms the same products with exponents of differences.
template <int K>
__device__ __forceinline__ void exact_block_gram(const BlockRows &br, const Prestage &pre, int j,
                                                 float aexp, float rk, float sq, int lane,
                                                 f32x4 &Lc, f32x4 &Mc) {
    const int grp = lane >> 4, r = lane & 15;
    float Lp[16], Mp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { Lp[i] = 0.f; Mp[i] = 0.f; }
    auto rows = [&](const uint16_t *base, int64_t stride) {
        return buffer_rsrc(base, br.nrows > 0 ? (uint32_t)(((int64_t)(br.nrows - 1) * stride +
                                                             K) * 2)
                                              : 0u);
    };
    const __amdgpu_buffer_rsrc_t rq = rows(br.q, br.qk_stride), rkk = rows(br.k, br.qk_stride),
                                 rg = rows(br.g, br.g_stride);
    const bool live = r < br.nrows;
    const bool gated = pre.gate != 0;
    // this lane's q, k, g (bf16 pairs) and dt_bias of one 16-dim tile; the next tile's are
    // loaded while the current one is consumed (the index is clamped to the last tile, so every
    // load stays inside its row and dt_bias stays inside its array)
    struct Tile { u32x2 q, k, g; f32x4 dt; };
    auto load = [&](int c) {
        const int col = 16 * c + 4 * grp;
        Tile t;
        t.q = bload8(rq, (int)((r * br.qk_stride + col) * 2), 0);
        t.k = bload8(rkk, (int)((r * br.qk_stride + col) * 2), 0);
        t.g = bload8(rg, (int)((r * br.g_stride + col) * 2), 0);
        t.dt = gated && pre.dt_bias ? *(const f32x4 *)(pre.dt_bias + (size_t)j * K + col)
                                    : zero4();
        return t;
    };
    Tile cur = load(0);
#pragma unroll 1
    for (int c = 0; c < K / 16; ++c) {
        const Tile nxt = load(c + 1 < K / 16 ? c + 1 : c);
        float kk[4], qq[4], gv[4], a[4];
        unpack_bf16x4(make_uint2(cur.k[0], cur.k[1]), kk);
        unpack_bf16x4(make_uint2(cur.q[0], cur.q[1]), qq);
        unpack_bf16x4(make_uint2(cur.g[0], cur.g[1]), gv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kk[e] *= rk;
            qq[e] *= sq;
            float g = gv[e];
            if (gated) g = live ? gate_activation(pre, g + cur.dt[e], aexp) : 0.f;
            a[e] = __builtin_amdgcn_exp2f(g * LOG2E);
        }
        float E[4] = {0.f, 0.f, 0.f, 0.f};
        exact_gram_steps(E, a, kk, qq, r, Lp, Mp, std::make_integer_sequence<int, 16>{});
        cur = nxt;
    }
    Lc = reduce_scatter_rows(Lp, grp);
    Mc = reduce_scatter_rows(Mp, grp);
}

// Workgroup fences that order LDS accesses only. Around s_barrier they make LDS writes visible
// to the other waves without waiting for this wave's outstanding global loads and stores (a
// full __syncthreads() waits for those too, which would drain every prefetch in flight).
__device__ __forceinline__ void lds_release() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}
__device__ __forceinline__ void lds_acquire() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void lds_barrier() {
    lds_release();
    __builtin_amdgcn_s_barrier();
    lds_acquire();
}

// Wait for every outstanding vector memory load of this wave (vmcnt 0; the LDS/scalar counter
// left unconstrained: simm16 = lgkmcnt 15 << 8 | expcnt 6 << 4). The kernels export nothing, so
// expcnt 6 constrains nothing either; it makes a deliberate drain read
// "s_waitcnt vmcnt(0) expcnt(6)" in the assembly, which tests/test_codegen.py tells apart from
// a wait the compiler put behind a load.
__device__ __forceinline__ void vm_drain() {
    __builtin_amdgcn_s_waitcnt(0x0f60);
}

// Packed sequences, longest first: the unit of ordinal u is value head u % HV of the sequence
// whose length ranks u / HV (ties by index). Workgroups start in blockIdx order, so the longest
// chains, which set the end of a launch of several rounds, start first and the short ones fill
// in behind them. The bounds are read with wave-uniform loads (the scalar memory path), lane n
// keeps sequence n's length, and each lane ranks its length against the other lanes' through
// readlane; each wave computes the same answer, so no workgroup barrier is needed. More than 64
// sequences keep the input order. The map only reorders whole units: every workgroup of a
// unit computes the same unit.
__device__ __forceinline__ int longest_first(const SeqGeom &sg, int HV, int u) {
    const int N = sg.N;
    if (sg.cu == nullptr || N <= 1 || N > 64) return u;
    const int lane = threadIdx.x & 63;
    int64_t len = -1;
    for (int k = 0; k < N; ++k) {
        const int64_t bk = seq_bos(sg, k);
        const int64_t lk = seq_eos(sg, k, bk) - bk;
        len = lane == k ? lk : len;
    }
    const int lo = (int)(uint32_t)len, hi = (int)(len >> 32);
    int rank = 0;
    for (int k = 0; k < N; ++k) {
        const int64_t lk = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, k) << 32) |
                                     (uint32_t)__builtin_amdgcn_readlane(lo, k));
        rank += (lk > len || (lk == len && k < lane)) ? 1 : 0;
    }
    // ranks of lanes < N are a permutation of 0 .. N - 1: exactly one lane matches
    const uint64_t m = __builtin_amdgcn_ballot_w64(lane < N && rank == u / HV);
    return m ? __builtin_ctzll(m) * HV + u % HV : u;
}

}  // namespace kda

// Host-side launchers (defined next to their kernels).
namespace kda {
// Compute units of the calling thread's current device, read once per device and cached
// (kda_api.hip).
int current_device_cus();
template <int K, int V> hipError_t launch_prepare_bf16(const FwdParams &p, hipStream_t st);
template <int K, int V> hipError_t launch_state_bf16(const FwdParams &p, hipStream_t st);
// fp32 chunk records from fp32 or (in_bf16) bf16 inputs: WsF32, or WsF32B for the backward
template <int K, int V>
hipError_t launch_prepare_f32(const FwdParams &p, hipStream_t st, bool in_bf16 = false,
                              bool for_backward = false);
template <int K, int V> hipError_t launch_state_f32(const FwdParams &p, hipStream_t st);
template <int K, int V> hipError_t launch_prepare32_bf16(const FwdParams &p, hipStream_t st);
template <int K, int V> hipError_t launch_state32_bf16(const FwdParams &p, hipStream_t st);
template <int K, int V> hipError_t launch_prepare64_bf16(const FwdParams &p, hipStream_t st);
template <int K, int V> hipError_t launch_state64_bf16(const FwdParams &p, hipStream_t st);
template <int K, int V> hipError_t launch_recurrent(const FwdParams &p, int io, hipStream_t st);
template <int K, int V>
hipError_t launch_backward(const BwdParams &b, bool in_bf16, hipStream_t st);
}  // namespace kda
