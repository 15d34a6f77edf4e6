// Internal launch interface between the C ABI (gdn_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Arguments of one prefill launch, already validated by the ABI layer.
struct PrefillParams {
    const void *q;             // [B][Hk][T][D] bf16 or f32
    const void *k;             // [B][Hk][T][D]
    const void *v;             // [B][Hv][T][D]
    const float *g;            // [B][Hv][T]
    const float *beta;         // [B][Hv][T]
    const void *init_state;    // [B][Hv][D][D] f32 (f16 when init_f16), or nullptr (zero state)
    void *o;                   // [B][Hv][T][D] f32 (f16 when o_f16)
    void *final_state;         // [B][Hv][D][D] f32 (f16 when final_f16), or nullptr
    int32_t B, T, Hk, Hv, D;   // T: tokens processed by this launch
    int32_t Ts;                // tokens between consecutive (b, head) sequences in q, k, v, g, beta
                               // and o (T, or more when the launch covers a window of a longer
                               // sequence and the pointers are offset to the window's start)
    int32_t head_map;          // 0 tiled (h % Hk), 1 grouped (h / (Hv/Hk))
    float scale;
    bool init_f16 = false, final_f16 = false;  // state storage types: 16-bit ...
    bool state_bf16 = false;                   // ... in bfloat16 rather than float16
    bool o_f16 = false;                        // o stored as f16 (the chunk-32/64 bf16 path)
    // packed sequences (chunk-32/64 bf16 path): B sequences laid end to end in one token axis
    // of T tokens (q, k, v, g, beta, o as for one sequence); nullptr for the padded layout
    const int32_t *seqs = nullptr;    // [B][4]: first token, tokens, first workspace chunk, 0
    const int32_t *chunks = nullptr;  // [nchunks][2]: first token, tokens (0: unused slot)
    int32_t nchunks = 0;              // workspace chunks of the packed layout
    // output norm fused into the o store (the segmented path): o = x / sqrt(mean(x^2) + eps)
    // * w * silu(gate) per output row; norm_w == nullptr: none
    const float *norm_w = nullptr;    // [D]
    const void *norm_gate = nullptr;  // o's shape, q/k/v element type, or nullptr (no gate factor)
    float norm_eps = 0.0f;
};

struct DecodeParams {
    const void *q;             // [B][Hk][D]
    const void *k;             // [B][Hk][D]
    const void *v;             // [B][Hv][D]
    const float *g;            // [B][Hv], or [B][Hv][D] with kda
    const float *beta;         // [B][Hv]
    void *state;               // [B][Hv][D][D] f32 (f16 when state_f16), in place
    void *o;                   // [B][Hv][D] f32 (f16 when o_f16)
    int32_t B, Hk, Hv, D;
    int32_t head_map;
    float scale;
    bool state_f16 = false;
    bool state_bf16 = false;  // the 16-bit state is bfloat16 rather than float16
    bool o_f16 = false;
    bool kda = false;          // one decay per key channel
    // output norm fused into the o store (one workgroup per pair): as PrefillParams
    const float *norm_w = nullptr;
    const void *norm_gate = nullptr;
    float norm_eps = 0.0f;
};

// Packed sequences (bf16 q/k/v, D = 128, chunk in {32, 64}): chunk-parallel kernel (T and
// A_qk per chunk into the workspace), then the sequential state pass reading them.
hipError_t launch_chunk_prep(const PrefillParams &p, int chunk, void *ws, hipStream_t stream);

// Gated RMSNorm of `rows` output rows of D floats, in place.
struct NormParams {
    void *o;                // [rows][D] f32 (f16 when o_f16), in place
    const void *gate;       // [rows][D] bf16 bits or float, or nullptr (no gate factor)
    const float *weight;    // [D]
    int64_t rows;
    int32_t D;
    bool gate_bf16;
    float eps;
    bool o_f16 = false;
};
hipError_t launch_gated_rmsnorm(const NormParams &p, hipStream_t stream);

// Causal conv + SiLU, q | k | v split and q/k L2 normalisation (4-tap kernel).
struct PrologueParams {
    const void *x;            // [B][T][(2 Hk + Hv) D] bf16 bits or float
    const float *conv_weight; // [(2 Hk + Hv) D][4]
    float *conv_state;        // [B][3][(2 Hk + Hv) D] in/out, or nullptr (zero rows, not written)
    void *q, *k, *v;          // [B][Hk][T][D], [B][Hk][T][D], [B][Hv][T][D] in x's type
    int32_t B, T, Hk, Hv, D;
    bool bf16;
    float eps;
};
hipError_t launch_qkv_prologue(const PrologueParams &p, hipStream_t stream);

// Per-channel decay (g [B][Hv][T][D]), D = 128: token-recurrent prefill.
hipError_t launch_kda_prefill(const PrefillParams &p, bool bf16, hipStream_t stream);

// Packed sequences: the workspace of gdn_prefill_varlen (chunk data for `nchunks` chunks, then
// the sequence and chunk tables), and the launch that fills the tables from cu_seqlens.
struct VarlenLayout {
    int64_t nchunks, seq_offset, chunk_offset, bytes;
};
VarlenLayout varlen_layout(int64_t nseq, int64_t Hk, int64_t Hv, int64_t T, int chunk);
hipError_t launch_varlen_tables(const int32_t *cu_seqlens, int32_t nseq, int32_t T, int chunk, int32_t *seqs,
                                int32_t *chunks, int32_t nchunks, hipStream_t stream);

// Segmented bf16 prefill (chunk 32 or 64, D = 128, fixed-length sequences): P segments per
// sequence run in parallel; the workspace holds three float32 D x D matrices per (pair, segment):
// segment start states, the end states from a zero start (N) and the segment maps (M).
struct SegParams {
    PrefillParams p;
    float *ws_start;     // [B * Hv][P][D][D]
    float *ws_n;         // [B * Hv][P][D][D]
    float *ws_m;         // [B * Hv][P][D][D]
    int32_t P;           // segments
    int32_t seg_chunks;  // chunks per segment (the last segment may hold fewer)
};
// Workspace bytes for P segments (0 for P = 1).
int64_t seg_workspace_bytes(int64_t pairs, int P);
// Segments used for this shape: as many as give every CU a workgroup in the output pass
// (at most one per chunk), reduced until their workspace fits workspace_bytes.
int seg_count(int64_t B, int64_t Hv, int64_t T, int chunk, size_t workspace_bytes, bool have_workspace);
// kda: g is [B][Hv][T][dk] (one log-decay per key channel; chunk 32 only)
hipError_t launch_prefill_seg(const PrefillParams &p, int chunk, int P, void *ws, hipStream_t stream,
                              bool kda = false);
// device address of the current GPU's static scratch (GDN_STATIC_SCRATCH_BYTES), looked up on the
// first call on each GPU and kept
hipError_t static_scratch(void **out);

hipError_t launch_prefill_scan(const PrefillParams &p, int chunk, const void *ws, hipStream_t stream);
// fp32 VALU chunked kernel, chunk in {16, 32, 64}: f32 q/k/v with D in {16, 32, 64, 128},
// or bf16 q/k/v (bf16 = true) with D in {16, 32, 64}.
hipError_t launch_prefill_f32(const PrefillParams &p, int chunk, bool bf16, hipStream_t stream);
// one decode step, D in {32, 64, 128}; bf16 selects bf16 q/k/v, else f32.
hipError_t launch_decode(const DecodeParams &p, bool bf16, hipStream_t stream);

}  // namespace gdn
