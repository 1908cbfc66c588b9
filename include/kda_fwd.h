/*
 * kda_fwd.h -- C ABI of libkda_fwd: the chunked Kimi Delta Attention (KDA) forward on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (the KDA definition, read off the chunked listing of "手撕KDA" ("KDA by
 * hand"), section 1, naive_chunk_kda): for every sequence s and value head j, with q/k head
 * h = j / (HV / H) and a state S in R^{K x V} that starts at initial_state[s, j] (or zero),
 * each token t of the sequence does
 *
 *     S <- diag(exp(g[t, j, :])) S;   r = v[t, j, :] - S^T k[t, h, :];
 *     S <- S + beta[t, j] k[t, h, :] r^T;   o[t, j, :] = scale * S^T q[t, h, :]
 *
 * and final_state[s, j] is S after the last token. The library evaluates it in the chunked
 * form of the same section with chunks of 16, 32 or 64 tokens: a token-parallel prepare kernel
 * (in-chunk cumsum of g, decayed q/k, the strictly lower triangular L and the masked Mqk, the
 * inverse of (I + L) by the Neumann doubling product of "KDA源码剖析之FlashKDA（上）" part 12,
 * and w = A (exp(G) k), u = A v) followed by a chunk-sequential state kernel; or token by token
 * (chunk 1, for decoding). Optionally the kernels first apply the pre-stage that turns raw
 * projections into q, k, g, beta (q/k L2 norm, beta sigmoid, a gate activation). kda_bwd
 * computes the gradients of all inputs of that forward (declared at the end of this file).
 *
 * Conventions
 *  - All tensor pointers are DEVICE pointers, caller-owned, contiguous (row-major), and
 *    16-byte aligned. The library allocates nothing (kda_fwd_noalloc's workspace is a static
 *    device array of the library, see there); its only host-side state is a per-device cache
 *    of the compute-unit count, read once and thread-safe. Calls are re-entrant: concurrent
 *    calls must use distinct workspaces and outputs, and kda_fwd_noalloc calls that overlap on
 *    one device race on its array.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default stream). Nothing
 *    synchronises; the caller owns synchronisation. Results are deterministic (no atomics).
 *  - Errors are reported only through the return value; nothing aborts or throws.
 */
#ifndef KDA_FWD_H
#define KDA_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,  /* null required pointer, bad shape, misalignment, B != 1 with
                                 cu_seqlens, N != B without cu_seqlens, HV % H != 0, a gate
                                 without A_log, a bounded gate's lower bound not < 0         */
    KDA_ERR_UNSUPPORTED = 2,  /* K or V outside {64, 128}, unknown io dtype, chunk not
                                 offered for this io dtype (the backward: other than 0, 16),
                                 unknown gate                                                */
    KDA_ERR_WORKSPACE = 3,    /* workspace NULL, misaligned, or smaller than
                                 kda_fwd_workspace_bytes() / kda_bwd_workspace_bytes()       */
    KDA_ERR_HIP = 4,          /* a kernel launch failed (hipGetLastError)                    */
    KDA_ERR_NOALLOC_TOO_LARGE = 5  /* kda_fwd_noalloc: these shapes need more workspace than
                                      KDA_NOALLOC_WORKSPACE_BYTES                             */
} kda_status;

typedef enum {
    KDA_BF16 = 0,             /* q, k, v, g, beta, o in bf16; states fp32; fp32 accumulation */
    KDA_FP32 = 1              /* everything fp32                                             */
} kda_dtype;

/* Gate activation applied to g before use (kda_fwd_args.gate). With value head j and key dim
   d, x = g[t, j, d] + dt_bias[j, d]:
     KDA_GATE_NONE      g is the log decay as given
     KDA_GATE_SOFTPLUS  g <- -exp(A_log[j]) * log(1 + exp(x))       ("手撕KDA" section 2.1,
                                                                      the C++ pre-stage)
     KDA_GATE_BOUNDED   g <- lower_bound / (1 + exp(-exp(A_log[j]) * x))
                        ("KDA源码剖析之FlashKDA（上）" part 7, gate activation; lower_bound < 0,
                        so the log decay lies in (lower_bound, 0))                          */
typedef enum {
    KDA_GATE_NONE = 0,
    KDA_GATE_SOFTPLUS = 1,
    KDA_GATE_BOUNDED = 2
} kda_gate;

typedef struct {
    /* Shapes. Dense batch: q is [B, T, H, K] and sequence b spans tokens [b*T, (b+1)*T) of
       the packed token axis (N must equal B). Varlen: B == 1, T = total tokens, and sequence
       s spans [cu_seqlens[s], cu_seqlens[s+1]) ("KDA源码剖析之FlashKDA（上）", part 4:
       sequences packed along one token axis). Any length >= 0 is accepted, including 0 and
       lengths that are not multiples of 16.                                                */
    int32_t B, T, N;
    int32_t H, HV;            /* q/k heads and value heads, HV % H == 0 (grouped value heads,
                                 "手撕KDA" section 1: value head j uses q/k head j / (HV/H)) */
    int32_t K, V;             /* head dims, each in {64, 128}                               */
    int32_t io;               /* kda_dtype                                                  */
    const void *q;            /* [B, T, H, K]   io dtype                                    */
    const void *k;            /* [B, T, H, K]   io dtype                                    */
    const void *v;            /* [B, T, HV, V]  io dtype                                    */
    const void *g;            /* [B, T, HV, K]  io dtype; per-key-dim decay in natural-log
                                 units (exp(g) multiplies the state). Any g <= 0 is exact to
                                 rounding at every chunk length: where a chunk's decay is too
                                 strong for the bf16 prepare kernels' factorised decay products
                                 (exponents spanning more than 2^100 between a chunk's
                                 reference token and its far end, e.g. below about -4.3 per
                                 token over the 16 tokens of a 32-token chunk's block), they
                                 form that chunk's diagonal Gram
                                 blocks from exact products of per-token decays instead.
                                 g <= 0 is expected but not enforced.                       */
    const void *beta;         /* [B, T, HV]     io dtype; used as given (no sigmoid)        */
    float scale;              /* output scale; <= 0 or NaN selects K^-0.5                   */
    const int64_t *cu_seqlens;/* device [N + 1] token offsets (cu[0] = 0, nondecreasing,
                                 cu[N] = T), or NULL for a dense batch. Contents cannot be
                                 validated without a synchronisation: invalid offsets give
                                 undefined values but every access stays in bounds.         */
    const float *initial_state; /* [N, HV, K, V] fp32, or NULL for zeros                    */
    void *o;                  /* [B, T, HV, V]  io dtype, written for every token            */
    float *final_state;       /* [N, HV, K, V] fp32, or NULL to skip; may be the same
                                 buffer as initial_state (the state updated in place)       */
    int32_t chunk;            /* tokens per serial step of the state kernel: 16 (the FlashKDA
                                 tile of "KDA源码剖析之FlashKDA（上）"), 32 (two 16-token blocks
                                 joined by block forward substitution; bf16 io only), 64 (pairs
                                 of 32-token chunks per serial step, the second chunk's delta
                                 written in the pair's starting state and the first chunk's
                                 delta; bf16 io only), 1 (the
                                 token recurrence itself, fp32 arithmetic, no workspace: for
                                 decoding and other short sequences, where a chunk's fixed cost
                                 dominates), or 0 for the default: 1 for a dense batch with
                                 T <= 16, else 32 for bf16 io and 16 for fp32 io. Results agree
                                 to rounding.                                                */
    /* Pre-stage, fused into the kernels that read the inputs (all zero: inputs used as given;
       "KDA源码剖析之FlashKDA（上）" parts 6, 7 and 10; "手撕KDA" section 2.1). The activated
       values replace q, k, g, beta everywhere above.                                          */
    int32_t qk_l2norm;        /* nonzero: q and k of every token and q/k head are divided by
                                 sqrt(sum over the K dims of the squares + 1e-6)             */
    int32_t beta_sigmoid;     /* nonzero: beta <- 1 / (1 + exp(-beta))                       */
    int32_t gate;             /* kda_gate                                                    */
    float gate_lower_bound;   /* KDA_GATE_BOUNDED: finite and < 0                            */
    const float *A_log;       /* [HV] fp32 device, one per value head; required for a gate   */
    const float *dt_bias;     /* [HV, K] fp32 device (16-byte aligned), or NULL for zeros    */
} kda_fwd_args;

/* Bytes of device workspace kda_fwd needs for these arguments (only shapes and io are read,
   and the current device's compute-unit count). Returns 0 for arguments kda_fwd would reject.
   The workspace holds the prepare kernel's per-chunk outputs (w, qd, kr, u, Mqk, exp(gamma))
   for ceil-bounded chunk slots of every value head: (B*T/chunk + N) * HV slots of 17,408 B
   (chunk 16), 34,816 B (chunk 32) or 2 x 36,864 B (chunk 64: two 32-token records per slot)
   at bf16 io and K = V = 128. At chunk 32 a dense batch (no cu_seqlens) with K == V, at least
   512 tokens per sequence and at most CUs / 2 sixteen-column state slices (N * HV * V / 16)
   runs the state pass as two segments whose scratch follows the records (about 2 * 2 * K
   bytes per token of the second segment and value head, plus two K x K fp16 states and one
   K x V fp32 state per (sequence, value head)); the size therefore depends on the device the
   call is sized for, and a workspace sized on a device with more compute units than the one
   it runs on may be too small (KDA_ERR_WORKSPACE). Chunk 1 needs none (0; kda_fwd then
   accepts a NULL workspace). */
size_t kda_fwd_workspace_bytes(const kda_fwd_args *args);

/* Enqueue the forward: prepare kernel, then state kernel, on `stream` (hipStream_t or NULL).
   `workspace` is a device buffer of at least kda_fwd_workspace_bytes(args) bytes, 256-byte
   aligned, owned by the caller; its contents on entry do not matter. Returns KDA_OK when both
   launches were enqueued. */
kda_status kda_fwd(const kda_fwd_args *args, void *workspace, size_t ws_bytes, void *stream);

/* The two stages of kda_fwd as separate launches, for callers that schedule or time them
   individually. kda_fwd_prepare enqueues the token-parallel prepare kernel, which writes the
   per-chunk quantities of every (chunk, value head) into `workspace`; kda_fwd_state enqueues
   the chunk-sequential state kernel (for a two-segment state pass, the pass and its
   correction kernel), which reads them and writes o and final_state. Running
   kda_fwd_prepare then kda_fwd_state on one stream with the same arguments and workspace is
   exactly kda_fwd. Same arguments, checks and status codes as kda_fwd. */
kda_status kda_fwd_prepare(const kda_fwd_args *args, void *workspace, size_t ws_bytes,
                           void *stream);
kda_status kda_fwd_state(const kda_fwd_args *args, void *workspace, size_t ws_bytes,
                         void *stream);

/* ---------------------------------------------------------------------------- backward
   Gradients of the forward above with respect to q, k, v, g, beta, initial_state and (with a
   gate) A_log and dt_bias, given the gradients of a loss with respect to o (d_o) and to
   final_state (dht): the reverse sweep of the C++ chunk backward of "手撕KDA" section 2.1,
   which walks the chunks newest first and carries the gradient of the state from the
   final-state gradient back to the initial state, followed by the backward of its pre-stage.
   The library records the state at every chunk start in a forward pass over the chunks, runs
   the state-gradient chain newest first (both chains in one launch), then back-propagates
   every (chunk, value head) independently to its tokens (through the chunk's u, w, Mqk, the
   inverse of (I + L) and the in-chunk cumsum of g) and finally through the pre-stage. fp32
   arithmetic, 16-token chunks.

   Arguments: `args` as for kda_fwd with the same inputs (raw inputs when the pre-stage is on;
   o and final_state are not read; chunk must be 0 or 16). Device buffers, caller-owned,
   16-byte aligned unless stated:
     d_o      [B, T, HV, V]  io dtype   gradient of o (required when B*T > 0)
     dht      [N, HV, K, V]  fp32       gradient of final_state, or NULL for zero
     dq, dk   [B, T, H, K]   fp32       written (summed over the value heads of a q/k head)
     dv       [B, T, HV, V]  fp32       written
     dg       [B, T, HV, K]  fp32       written
     dbeta    [B, T, HV]     fp32       written
     dh0      [N, HV, K, V]  fp32       gradient of initial_state, or NULL to skip
     dA_log   [HV]           fp32       gradient of A_log (4-byte aligned); required with a
                                        gate, ignored without
     ddt_bias [HV, K]        fp32       gradient of dt_bias (also when dt_bias is NULL: the
                                        gradient of a zero bias), or NULL to skip
   dq, dk, dg, dbeta are the gradients of the arguments as passed: with the pre-stage on, of
   the raw q, k, g, beta.
   `workspace`: at least kda_bwd_workspace_bytes(args) bytes, 256-byte aligned, contents on
   entry irrelevant: the fp32 chunk records (each with a copy of its chunk's d_o), the state
   at every chunk start and the state gradient at every chunk end (about
   2 * (B*T/16 + N) * HV * K * V * 4 bytes), plus
   2 * B*T * HV * K * 4 bytes when HV > H or the q/k L2 norm is on, plus (B*T/16 + N) * HV *
   (K + 1) * 4 bytes with a gate. Status codes as for kda_fwd; KDA_ERR_UNSUPPORTED also for a
   chunk other than 0 or 16; KDA_ERR_INVALID_ARG also for a missing or misaligned dA_log with
   a gate. Any g <= 0 is exact to rounding: every exponent the kernels form is a difference
   of in-chunk cumsums with the later one first. Deterministic
   (fixed-order sums, no atomics). With N = 0 nothing is written.                          */
size_t kda_bwd_workspace_bytes(const kda_fwd_args *args);

kda_status kda_bwd(const kda_fwd_args *args, const void *d_o, const float *dht,
                   void *workspace, size_t ws_bytes, float *dq, float *dk, float *dv, float *dg,
                   float *dbeta, float *dh0, float *dA_log, float *ddt_bias, void *stream);

/* ---------------------------------------------------------------------------- no allocation
   For callers that cannot allocate device memory or pass a workspace: code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc. kda_fwd_noalloc is kda_fwd
   with the workspace taken from a static device array of KDA_NOALLOC_WORKSPACE_BYTES that the
   library holds on every device it runs on until the process ends; it calls no allocating
   routine. Same arguments (no workspace), checks, results and status codes as kda_fwd, plus
   KDA_ERR_NOALLOC_TOO_LARGE when kda_fwd_workspace_bytes(args) exceeds the array (128 MiB:
   for example 16 value heads of up to about 6,300 tokens at bf16 io; chunk 1 needs none, so
   decoding steps have no limit). The work runs on the calling thread's current device and
   uses that device's array. Every call on one device shares that array: calls whose work
   overlaps on one device (several streams or threads) race on it, so the caller serialises
   them (one stream, or events between them). The array's contents on entry do not matter. */
#define KDA_NOALLOC_WORKSPACE_BYTES ((size_t)128 << 20)
kda_status kda_fwd_noalloc(const kda_fwd_args *args, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *kda_strerror(int status);

/* Library ABI version (major * 100 + minor). */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_FWD_H */
