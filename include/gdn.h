/*
 * gdn.h -- C ABI of the gated delta rule (GatedDeltaNet) scan for AMD MI355X (gfx950).
 *
 * The operation (one independent recurrence per sequence b and value head h):
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (scale * q_t)
 *
 * with the state S a dv x dk matrix (row = value dimension, column = key
 * dimension). Sources on the pages:
 *   - state orientation, the one-step update and the output taken from the
 *     updated state: tinygrad compare page "27b 935/47", the gated-delta
 *     decode and prefill reference tests (test_llm_quant_cpu.py), where the
 *     state is contracted with k and q over its last index and the core output
 *     equals alpha*S*q + delta*(k.q) with delta = (v - alpha*S*k)*beta;
 *   - prefill from a given state returning (outputs, next state), and a
 *     one-token step as the decode call: the same tests' gated_delta_prefill
 *     and gated_delta_decode signatures, and the commit log of page
 *     "mergable fast RDNA3 Qwen 3.6" (a 1-token chunk is a decode step);
 *   - padded steps with beta = 0 and g = 0 (alpha = exp(0) = 1) are exact
 *     no-ops: commit log of page "mergable fast RDNA3 Qwen 3.6",
 *     symbolic-length prefill entry;
 *   - key heads shared by value heads: the gdn_qkv test on page "27b 935/47"
 *     repeats (tiles) the key heads over the value heads (GDN_HEADS_TILED).
 * The decay is passed as g (log-decay); the library forms alpha = exp(g). g <= 0 is
 * a precondition (alpha in (0, 1]: a decay, as the pages' gates are); g > 0 is not
 * rejected but leaves the range in which the float16 operands below are safe.
 * Callers pass q and k already L2-normalised and q without the scale.
 *
 * Memory: every tensor pointer is a DEVICE pointer to memory the caller owns
 * (the library allocates nothing and keeps no state besides a thread-local
 * error string). Tensors are dense, row-major, in the layouts given per call.
 * q, k, v, o and the states must be 16-byte aligned; g and beta 4-byte aligned.
 *
 * Errors: arguments are validated synchronously on the host before anything
 * is enqueued; on a non-OK status nothing was launched and gdn_last_error()
 * describes the problem. Work is enqueued asynchronously on `stream` (a
 * hipStream_t passed as void*; NULL = the null stream) and the caller
 * synchronises. No C++ exception crosses this interface. Non-finite data is
 * not detected: it propagates into the outputs.
 *
 * Precision: g and beta are float32; o is float32, or float16 when
 * shape->o_dtype says so; the states are float32, or float16 when
 * shape->state_dtype says so (below). q/k/v are float32 or bfloat16. The bfloat16
 * path at head_dim 128 runs its matrix products on float16 MFMA operands with
 * float32 accumulation; the float32 path, and bfloat16 at head_dims below 128,
 * compute in fp32 on the vector ALUs. Results depend on the chunk length through
 * the order of reductions, so different chunk lengths agree within rounding, not
 * bit for bit.
 *
 * Float16 operand range (bfloat16 at head_dim 128, prefill and its segment maps):
 * k and q, the state, the values R = beta (v - gamma K S^T) and U = T R of a chunk,
 * and the chunk matrices T and A_qk are rounded to float16 as MFMA operands.
 * bfloat16 inputs convert exactly while their magnitudes lie in about 6e-5 .. 65504
 * (smaller ones lose at most 3e-8 absolutely). A value beyond +-65504 becomes
 * infinite, and the outputs and final state that depend on it become non-finite
 * (inf or NaN): nothing is clamped and no error is reported. With L2-normalised q, k,
 * g <= 0 and |v|, |state| up to a few thousand every operand stays far inside the
 * range. Decode and the float32 paths have no such limit.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 7

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* malformed shape, NULL or misaligned pointer, overlapping output */
    GDN_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported set below */
    GDN_ERR_HIP = 3          /* the HIP runtime refused a launch; see gdn_last_error() */
} gdn_status;

typedef enum {
    GDN_DTYPE_F32 = 0,  /* q, k, v are float32 */
    GDN_DTYPE_BF16 = 1  /* q, k, v are bfloat16 */
} gdn_dtype;

/*
 * Storage type of the states (prefill initial and final state, decode state). The
 * recurrence always runs in float32; a 16-bit state is widened on load and rounded
 * to nearest-even float16 (or bfloat16) when written, which halves the state traffic
 * of decode. The gated delta decode and prefill tests on page "27b 935/47" hold the
 * recurrent state in float16 (the decode test rounds its expected next state
 * back to float16). float16 covers magnitudes up to 65504 (a state beyond that
 * becomes infinite) with 11 significant bits; bfloat16 covers float32's range with 8
 * (each write rounds by up to 2^-9 of a value, and a decode sequence accumulates one
 * such rounding per step). The prefill carries its state in float32 and rounds once,
 * at the final state.
 */
typedef enum {
    GDN_STATE_F32 = 0,
    GDN_STATE_F16 = 1,
    GDN_STATE_BF16 = 2
} gdn_state_dtype;

/*
 * Storage type of the outputs o (prefill, decode, and the gated RMSNorm's in-place rows).
 * float16 rounds each output to nearest even (at most 2^-11 of its value), which keeps the
 * bfloat16 path inside its 2e-3 accuracy bar while halving the bytes of o, the largest
 * tensor a long prefill writes; bfloat16 outputs (2^-8) would not.
 */
typedef enum {
    GDN_OUT_F32 = 0,
    GDN_OUT_F16 = 1
} gdn_out_dtype;

typedef enum {
    GDN_HEADS_TILED = 0,   /* value head h reads key head h % Hk (the pages' repeat of key heads) */
    GDN_HEADS_GROUPED = 1  /* value head h reads key head h / (Hv / Hk) */
} gdn_head_map;

typedef struct {
    int32_t batch;        /* B >= 1 */
    int32_t seq_len;      /* T: prefill T >= 0 (need not be a multiple of chunk); decode: must be 1 */
    int32_t num_k_heads;  /* Hk >= 1 */
    int32_t num_v_heads;  /* Hv >= 1, a multiple of Hk */
    int32_t head_dim_k;   /* dk */
    int32_t head_dim_v;   /* dv */
    int32_t chunk;        /* prefill chunk length C in {16, 32, 64}; ignored by decode */
    gdn_dtype qkv_dtype;  /* element type of q, k, v */
    gdn_head_map head_map;
    float scale;          /* o_t = S_t (scale * q_t); must be finite */
    gdn_state_dtype state_dtype; /* element type of the states */
    gdn_out_dtype o_dtype;       /* element type of o */
} gdn_shape;

/*
 * Optional output norm of gdn_prefill and gdn_decode: the gated RMSNorm that the gated delta
 * calls on the "27b 935/47" compare page take as arguments (gated_delta's norm_weight and
 * norm_eps, gated_delta_prefill's weight and eps; the q8_gated_rmsnorm test). With it, each
 * output row x of head_dim_v values (one token of one value head) is written as
 *     x / sqrt(mean(x^2) + eps) * weight * silu(gate),  silu(z) = z / (1 + exp(-z))
 * instead of x; the un-normalised x is not written. gdn_gated_rmsnorm gives the same values
 * as a separate pass.
 *   weight  [dv] float32, the same for every head and token; 16-byte aligned
 *   gate    o's shape ([B][Hv][T][dv] for prefill, [B][Hv][dv] for decode) in qkv_dtype, or
 *           NULL for no gate factor; 16-byte aligned
 *   eps     finite, >= 0
 * weight and gate must not overlap any output. Fused into the output store of the segmented
 * bf16 prefill (dk = 128, every C) and of decode when B * Hv >= 256 (a workgroup then
 * owns whole output rows); the other paths apply it as one more pass over o after the scan.
 * In the segmented prefill a row passes through float16 twice: before the norm, each group of
 * 8 values scaled by a power of two taken from its own sum of squares (so one rounding to 11
 * significant bits at any magnitude; the float32 sums of squares are not rounded), and after
 * it (one more rounding of each normalised value, also with float32 o).
 */
typedef struct {
    const float *weight;
    const void *gate;
    float eps;
} gdn_norm;

/*
 * Supported set (GDN_ERR_UNSUPPORTED otherwise):
 *   prefill:  dk = dv in {16, 32, 64, 128}, C in {16, 32, 64}, either dtype.
 *   decode:   dk = dv in {32, 64, 128}, either dtype.
 *   float16 / bfloat16 states and float16 o: every prefill path, decode (and the gated
 *   RMSNorm for o).
 *   (float16 o rounds each output, at most 2^-11 of its value: within the bfloat16 path's
 *   accuracy, beyond the float32 path's.)
 * Paths: bfloat16 with dk = 128 runs the segmented MFMA prefill (below; C = 16 about 1.4 times
 * the time of C = 64 on long sequences, C = 32 about the same); float32 q/k/v, and bfloat16
 * with dk < 128, a float32 VALU kernel.
 *
 * Segmented prefill (bfloat16, dk = 128, C in {16, 32, 64}): the chunks of each sequence are cut
 * into P segments of equal chunk counts that run in parallel: a map pass computes, per
 * segment, the end state of segment 0 and the affine map S -> S M + N of each later segment
 * (the chunk update is affine in the start state), a combine chains the maps into every
 * segment's start state, and an output pass runs every segment from its start (at C = 64 the
 * map pass runs 32-token chunks: results differ from an all-64 run by rounding only). P is as
 * large as needed to give each of the GPU's 256 CUs a workgroup in the output pass
 * (ceil(256 / (B Hv)), at most the chunk count and 64), reduced until its workspace fits the
 * workspace_bytes the caller passes: 3 * B * Hv * P * dk * dk * 4 bytes for P > 1, nothing
 * for P = 1 (one workgroup per (b, value head) runs the whole sequence). Any workspace size,
 * NULL included, is valid; gdn_prefill_segments() tells which P a size gives.
 */

/*
 * Bytes of workspace for the preferred segment count of this shape (0 when the path uses no
 * workspace, or when one segment is preferred, or for an invalid shape). A smaller workspace
 * is accepted and means fewer segments (see above).
 */
size_t gdn_prefill_workspace_bytes(const gdn_shape *shape);

/*
 * The number of segments P that gdn_prefill runs for this shape with workspace_bytes of
 * workspace: 1 for the paths that do not segment, 0 for an invalid shape. Pure host code.
 */
int gdn_prefill_segments(const gdn_shape *shape, size_t workspace_bytes);

/*
 * Chunked prefill of T tokens from a given state; writes every output and the
 * final state.
 *   q, k           [B][Hk][T][dk]   qkv_dtype
 *   v              [B][Hv][T][dv]   qkv_dtype
 *   g, beta        [B][Hv][T]       float32 (log-decay and write strength)
 *   initial_state  [B][Hv][dv][dk]  state_dtype, or NULL for a zero state
 *   o              [B][Hv][T][dv]   o_dtype, output; must not overlap any input
 *   final_state    [B][Hv][dv][dk]  state_dtype, output, or NULL to skip; may be
 *                                   the same pointer as initial_state (in place)
 *   workspace      device scratch of workspace_bytes bytes, 16-byte aligned, or NULL; the
 *                  segmented path uses as much of it as its segment count needs (above),
 *                  the other paths none. It must not overlap any other argument.
 *   norm           the output norm (gdn_norm above), or NULL to write o as computed
 * A ragged batch passes every sequence padded to the common T with beta = 0,
 * g = 0 (and zero q/k/v) on the padded steps, which leave the state unchanged.
 * With initial_state == final_state (in place) every workgroup reads the state it starts
 * from before any workgroup writes the final state (the segmented path's output pass starts
 * segment 0 from the map pass's float32 copy of the initial state).
 */
gdn_status gdn_prefill(const gdn_shape *shape, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const void *initial_state,
                       void *o, void *final_state, void *workspace, size_t workspace_bytes,
                       const gdn_norm *norm, void *stream);

/*
 * gdn_prefill for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, hosts that forbid allocation): the same computation and arguments,
 * except that the workspace is the library's own static scratch on the current GPU, of which
 * the call uses workspace_bytes (the segment count follows it as in gdn_prefill; 0: one
 * segment, no scratch). The call allocates nothing.
 *   workspace_bytes  at most GDN_STATIC_SCRATCH_BYTES (96 MiB, which holds the preferred
 *                    segment count of every shape, gdn_prefill_workspace_bytes);
 *                    GDN_ERR_INVALID_ARG beyond it
 * The scratch is one array per GPU, set aside when the library's code object is loaded on that
 * GPU and held until the process ends; its address is looked up on the first call on each GPU
 * (GDN_ERR_HIP if that fails). The stream must belong to the current device. Every call on a
 * GPU shares its array and leaves its last contents there; no part of it needs to start at
 * zero (every value the kernels read is written earlier in the same call). Calls that overlap
 * in time on one GPU (on different streams, or from different host threads) race on it.
 */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)96 << 20)
gdn_status gdn_prefill_static(const gdn_shape *shape, const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const void *initial_state,
                              void *o, void *final_state, size_t workspace_bytes,
                              const gdn_norm *norm, void *stream);

/*
 * Prefill of B sequences of different lengths packed end to end along one token axis,
 * without padding: sequence i holds tokens cu_seqlens[i] .. cu_seqlens[i + 1] - 1 and runs
 * as its own recurrence from initial state i. The result equals gdn_prefill on each
 * sequence alone, and equals the padded ragged batch (every sequence padded to a common
 * length with beta = 0, g = 0 steps, which leave the state unchanged: the symbolic-length
 * prefill entry in the commit log of page "mergable fast RDNA3 Qwen 3.6") on the real tokens.
 * shape->batch = B (number of sequences), shape->seq_len = T (packed tokens, >= 0).
 *   cu_seqlens     [B + 1]          int32, DEVICE memory: 0 = cu[0] <= cu[1] <= ... <= cu[B] = T
 *   q, k           [Hk][T][dk]      qkv_dtype (bfloat16 only)
 *   v              [Hv][T][dv]      qkv_dtype
 *   g, beta        [Hv][T]          float32
 *   initial_state  [B][Hv][dv][dk]  state_dtype, or NULL for zero states
 *   o              [Hv][T][dv]      o_dtype, output
 *   final_state    [B][Hv][dv][dk]  state_dtype, output, or NULL; may equal initial_state
 *   workspace      device scratch of gdn_prefill_varlen_workspace_bytes(shape) bytes; it
 *                  grows with T (about 16.4 KB per token at Hv = 32) and is not split into
 *                  token segments
 * Supported: bfloat16 q/k/v, dk = dv = 128, chunk 32 or 64. cu_seqlens is read on the GPU
 * only, so its values are not validated on the host: the kernels clamp every bound into
 * [0, T] and every length to >= 0, which keeps all accesses inside the buffers for any
 * contents, but only a valid array gives meaningful results (tokens outside every sequence
 * leave their o rows unwritten; overlapping sequences write the same rows).
 */
size_t gdn_prefill_varlen_workspace_bytes(const gdn_shape *shape);
gdn_status gdn_prefill_varlen(const gdn_shape *shape, const int32_t *cu_seqlens, const void *q,
                              const void *k, const void *v, const float *g, const float *beta,
                              const void *initial_state, void *o, void *final_state, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * One decode step for a batch of single tokens (shape->seq_len must be 1);
 * updates the state in place and writes the output of the updated state.
 *   q, k     [B][Hk][dk]       qkv_dtype
 *   v        [B][Hv][dv]       qkv_dtype
 *   g, beta  [B][Hv]           float32
 *   state    [B][Hv][dv][dk]   state_dtype, read and overwritten
 *   o        [B][Hv][dv]       o_dtype, output; must not overlap any input or the state
 *   norm     the output norm (gdn_norm above), or NULL to write o as computed
 */
gdn_status gdn_decode(const gdn_shape *shape, const void *q, const void *k, const void *v,
                      const float *g, const float *beta, void *state, void *o, const gdn_norm *norm,
                      void *stream);

/*
 * Per-channel decay (the KDA variant): the recurrence with one log-decay per key channel,
 *     S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t (scale q_t),
 * the "channel decay" of the Kimi K3 experiments on the "master..kimi_slop" page, which keeps
 * one decay value per key channel rather than one per head. The pages give no formula; this
 * is the gated delta rule with its scalar decay made diagonal over the key channels (with
 * every channel of g_t equal it is gdn_prefill / gdn_decode). Layouts as gdn_prefill and
 * gdn_decode except g:
 *   gdn_kda_prefill  g [B][Hv][T][dk] float32, 16-byte aligned. bfloat16 q/k/v with chunk
 *                    32 or 64: the chunked (WY) form in 32-token chunks on MFMA, segment-
 *                    parallel within the workspace passed (as gdn_prefill: query
 *                    gdn_prefill_workspace_bytes and gdn_prefill_segments with the same shape
 *                    and chunk 32; any size, NULL included, is valid). It takes every log-decay
 *                    below -10 as -10 (a step keeping less than e^-10 = 4.5e-5 of a state
 *                    channel keeps that much of it), which bounds the factors of its intra-
 *                    chunk products within e^(+-80). float32 q/k/v, or chunk 16: token by
 *                    token, exact for any decay, no workspace used.
 *   gdn_kda_decode   g [B][Hv][dk] float32, 16-byte aligned
 * Supported: dk = dv = 128 for the prefill (32, 64 or 128 for decode), bfloat16 or float32
 * q/k/v, both state and output storage types.
 */
gdn_status gdn_kda_prefill(const gdn_shape *shape, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const void *initial_state,
                           void *o, void *final_state, void *workspace, size_t workspace_bytes,
                           void *stream);
gdn_status gdn_kda_decode(const gdn_shape *shape, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, void *state, void *o, void *stream);

/* Static text for a status code. */
const char *gdn_status_string(gdn_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *gdn_last_error(void);

/*
 * Gated RMSNorm of the output, in place: the output epilogue that the gated
 * delta kernels apply on the "27b 935/47" compare page (its q8_gated_rmsnorm
 * test; the norm_weight and norm_eps arguments of gated_delta). For every row
 * x of head_dim_v values of o:
 *     x <- x / sqrt(mean(x^2) + eps) * weight * silu(gate),  silu(z) = z / (1 + exp(-z))
 *   o       [B][Hv][T][dv] in shape->o_dtype with T = shape->seq_len (a gdn_decode output
 *           [B][Hv][dv] is the case T = 1); read and overwritten
 *   gate    [B][Hv][T][dv] in shape->qkv_dtype, or NULL for no gate factor
 *   weight  [dv] float32, the same for every head and token
 *   eps     finite, >= 0
 * Supported: head_dim_v in {16, 32, 64, 128}. gate and weight must not overlap o.
 * Alignment: o, weight and a float32 gate 16 bytes; a bfloat16 gate 8 bytes with
 * float32 o and 16 bytes with float16 o.
 * The same norm is an optional argument of gdn_prefill and gdn_decode (gdn_norm), fused into
 * their output stores where a workgroup owns whole output rows; this call is one extra
 * streaming pass over o.
 */
gdn_status gdn_gated_rmsnorm(const gdn_shape *shape, void *o, const void *gate, const float *weight,
                             float eps, void *stream);

/*
 * Input prologue of the scan in one pass: the causal depthwise convolution
 * with SiLU and the q | k | v split with per-head L2 normalisation (the
 * causal_conv_silu and gdn_qkv tests on the "27b 935/47" compare page). With
 * window = the 3 conv_state rows before t = 0 followed by the rows of x,
 *     y[b][t][c] = silu(sum_{i<4} window[b][t + i][c] * conv_weight[c][i])
 * channels [0, Hk d) of y are q, [Hk d, 2 Hk d) k and the rest v, in heads of
 * d; each q and k head is scaled by 1 / sqrt(sum of its squares + eps). The
 * outputs are in gdn_prefill's layouts (key heads are not repeated for the
 * value heads and q is not scaled by 1/sqrt(d): gdn_prefill does both).
 *   x            [B][T][(2 Hk + Hv) d]  qkv_dtype (shape->seq_len = T)
 *   conv_weight  [(2 Hk + Hv) d][4]     float32
 *   conv_state   [B][3][(2 Hk + Hv) d]  float32, read and replaced by the last
 *                                       3 window rows (what continues the
 *                                       sequence), or NULL: zero rows, not written
 *   q, k         [B][Hk][T][d]          qkv_dtype, outputs
 *   v            [B][Hv][T][d]          qkv_dtype, output
 *   eps          finite, > 0 (the pages use 1e-6)
 * Supported: d in {16, 32, 64, 128}. Outputs must not overlap each other or
 * any input. With T = 0 nothing is read or written.
 */
gdn_status gdn_qkv_prologue(const gdn_shape *shape, const void *x, const float *conv_weight, float *conv_state,
                            void *q, void *k, void *v, float eps, void *stream);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
