// C ABI of the gated delta rule library: argument validation (pure host code,
// run before anything is enqueued), variant dispatch and error reporting.
#include "gdn.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdint>

#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Range &a, const Range &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range range(const char *name, const void *p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks common to both calls. Element counts must stay far from int64 overflow.
gdn_status check_common(const gdn_shape *s) {
    if (!s) return fail(GDN_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch < 1) return fail(GDN_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", s->batch);
    if (s->num_k_heads < 1 || s->num_v_heads < 1)
        return fail(GDN_ERR_INVALID_ARG, "head counts must be >= 1 (Hk=%d, Hv=%d)", s->num_k_heads, s->num_v_heads);
    if (s->num_v_heads % s->num_k_heads != 0)
        return fail(GDN_ERR_INVALID_ARG, "num_v_heads (%d) must be a multiple of num_k_heads (%d)",
                    s->num_v_heads, s->num_k_heads);
    if (s->head_dim_k < 1 || s->head_dim_v < 1)
        return fail(GDN_ERR_INVALID_ARG, "head dims must be >= 1 (dk=%d, dv=%d)", s->head_dim_k, s->head_dim_v);
    if (s->qkv_dtype != GDN_DTYPE_F32 && s->qkv_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_INVALID_ARG, "unknown qkv_dtype %d", (int)s->qkv_dtype);
    if (s->head_map != GDN_HEADS_TILED && s->head_map != GDN_HEADS_GROUPED)
        return fail(GDN_ERR_INVALID_ARG, "unknown head_map %d", (int)s->head_map);
    if (s->state_dtype != GDN_STATE_F32 && s->state_dtype != GDN_STATE_F16 && s->state_dtype != GDN_STATE_BF16)
        return fail(GDN_ERR_INVALID_ARG, "unknown state_dtype %d", (int)s->state_dtype);
    if (s->o_dtype != GDN_OUT_F32 && s->o_dtype != GDN_OUT_F16)
        return fail(GDN_ERR_INVALID_ARG, "unknown o_dtype %d", (int)s->o_dtype);
    if (!std::isfinite(s->scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (s->head_dim_k != s->head_dim_v)
        return fail(GDN_ERR_UNSUPPORTED, "dk != dv (%d, %d) is not supported", s->head_dim_k, s->head_dim_v);
    const double pairs = (double)s->batch * s->num_v_heads;
    if (pairs * s->head_dim_v > 2147483647.0)
        return fail(GDN_ERR_UNSUPPORTED, "batch * num_v_heads * head_dim is too large for one launch");
    return GDN_OK;
}

gdn_status check_ptr(const void *p, const char *name, uintptr_t align) {
    if (!p) return fail(GDN_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(GDN_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, (unsigned)align);
    return GDN_OK;
}

gdn_status check_no_overlap(const Range *outs, int nout, const Range *ins, int nin) {
    for (int i = 0; i < nout; ++i)
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(GDN_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, ins[j].name);
    return GDN_OK;
}

#define GDN_TRY(expr)                      \
    do {                                   \
        gdn_status st_ = (expr);           \
        if (st_ != GDN_OK) return st_;     \
    } while (0)

// An output norm over `rows` output rows of d values: its eps, pointers, and that its weight
// and gate overlap none of the call's outputs.
gdn_status check_norm(const gdn_norm *n, int d, int64_t rows, bool bf16, const Range *outs, int nout) {
    if (!n) return GDN_OK;
    if (!std::isfinite(n->eps) || n->eps < 0.0f) return fail(GDN_ERR_INVALID_ARG, "norm eps must be finite and >= 0");
    GDN_TRY(check_ptr(n->weight, "norm weight", 16));
    if (n->gate) GDN_TRY(check_ptr(n->gate, "norm gate", 16));
    const Range nr[] = {range("norm weight", n->weight, (int64_t)d * 4),
                        range("norm gate", n->gate, n->gate ? rows * d * (bf16 ? 2 : 4) : 0)};
    return check_no_overlap(outs, nout, nr, 2);
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(gdn_status st) {
    switch (st) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *gdn_last_error(void) { return g_last_error; }

// the segmented MFMA path: bfloat16 q/k/v, head_dim 128 (every chunk length)
static bool segmented_path(const gdn_shape *s) {
    return s->qkv_dtype == GDN_DTYPE_BF16 && s->head_dim_k == 128 &&
           (s->chunk == 16 || s->chunk == 32 || s->chunk == 64);
}

size_t gdn_prefill_workspace_bytes(const gdn_shape *s) {
    if (check_common(s) != GDN_OK || s->seq_len < 0 || !segmented_path(s)) return 0;
    const int P = gdn::seg_count(s->batch, s->num_v_heads, s->seq_len, s->chunk, SIZE_MAX, true);
    return (size_t)gdn::seg_workspace_bytes((int64_t)s->batch * s->num_v_heads, P);
}

int gdn_prefill_segments(const gdn_shape *s, size_t workspace_bytes) {
    if (check_common(s) != GDN_OK || s->seq_len < 0) return 0;
    if (!segmented_path(s)) return 1;
    return gdn::seg_count(s->batch, s->num_v_heads, s->seq_len, s->chunk, workspace_bytes, true);
}

}  // extern "C"

namespace {
// gdn_prefill and gdn_prefill_static: with use_static, the workspace is the current GPU's static
// scratch (looked up only when the segmented path uses one)
gdn_status prefill_impl(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const void *initial_state, void *o, void *final_state,
                        void *workspace, size_t workspace_bytes, const gdn_norm *norm, void *stream,
                        bool use_static) {
    GDN_TRY(check_common(s));
    if (s->seq_len < 0) return fail(GDN_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", s->seq_len);
    if (s->chunk != 16 && s->chunk != 32 && s->chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "chunk must be 16, 32 or 64 (got %d)", s->chunk);
    const int d = s->head_dim_k;
    const bool bf16 = s->qkv_dtype == GDN_DTYPE_BF16;
    if (d != 16 && d != 32 && d != 64 && d != 128)
        return fail(GDN_ERR_UNSUPPORTED, "prefill supports head_dim 16, 32, 64 or 128 (got %d)", d);
    const double tokens = (double)s->batch * s->num_v_heads * s->seq_len * d;
    if (tokens > 4.0e15) return fail(GDN_ERR_UNSUPPORTED, "tensor sizes overflow");

    const int64_t B = s->batch, T = s->seq_len, Hk = s->num_k_heads, Hv = s->num_v_heads;
    const int64_t esz = bf16 ? 2 : 4;
    const int64_t qk_bytes = B * Hk * T * d * esz, v_bytes = B * Hv * T * d * esz;
    const bool st16 = s->state_dtype != GDN_STATE_F32, o16 = s->o_dtype == GDN_OUT_F16;
    const int64_t gb_bytes = B * Hv * T * 4, o_bytes = B * Hv * T * d * (o16 ? 2 : 4);
    const int64_t st_bytes = B * Hv * d * d * (st16 ? 2 : 4);
    if (T > 0) {
        GDN_TRY(check_ptr(q, "q", 16));
        GDN_TRY(check_ptr(k, "k", 16));
        GDN_TRY(check_ptr(v, "v", 16));
        GDN_TRY(check_ptr(g, "g", 4));
        GDN_TRY(check_ptr(beta, "beta", 4));
        GDN_TRY(check_ptr(o, "o", 16));
    }
    if (initial_state) GDN_TRY(check_ptr(initial_state, "initial_state", 16));
    if (final_state) GDN_TRY(check_ptr(final_state, "final_state", 16));

    const Range ins[] = {range("q", q, T ? qk_bytes : 0), range("k", k, T ? qk_bytes : 0),
                         range("v", v, T ? v_bytes : 0), range("g", g, T ? gb_bytes : 0),
                         range("beta", beta, T ? gb_bytes : 0),
                         range("initial_state", initial_state, initial_state ? st_bytes : 0)};
    const Range out_o[] = {range("o", o, T ? o_bytes : 0)};
    GDN_TRY(check_no_overlap(out_o, 1, ins, 6));
    if (final_state) {
        const Range out_s[] = {range("final_state", final_state, st_bytes)};
        GDN_TRY(check_no_overlap(out_s, 1, ins, 5));  // q, k, v, g, beta
        GDN_TRY(check_no_overlap(out_s, 1, out_o, 1));
        if (initial_state && final_state != initial_state && overlaps(out_s[0], ins[5]))
            return fail(GDN_ERR_INVALID_ARG, "final_state partially overlaps initial_state");
    }
    {
        const Range outs[] = {out_o[0], range("final_state", final_state, final_state ? st_bytes : 0)};
        GDN_TRY(check_norm(norm, d, B * Hv * T, bf16, outs, 2));
    }

    gdn::PrefillParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.init_state = initial_state;
    p.o = o;
    p.final_state = final_state;
    p.B = s->batch;
    p.T = s->seq_len;
    p.Ts = s->seq_len;
    p.Hk = s->num_k_heads;
    p.Hv = s->num_v_heads;
    p.D = d;
    p.head_map = (int32_t)s->head_map;
    p.scale = s->scale;
    p.init_f16 = p.final_f16 = st16;
    p.state_bf16 = s->state_dtype == GDN_STATE_BF16;
    p.o_f16 = o16;
    // the segmented path splits every sequence into as many segments as its preferred count
    // allows within the workspace the caller passes (one segment, no workspace, at the least)
    int P = 1;
    if (segmented_path(s)) {
        P = gdn::seg_count(B, Hv, T, s->chunk, workspace_bytes, use_static || workspace != nullptr);
        if (P > 1) {
            if (use_static) {
                const hipError_t e = gdn::static_scratch(&workspace);
                if (e != hipSuccess) return fail(GDN_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
            }
            const int64_t used = gdn::seg_workspace_bytes(B * Hv, P);
            if (!aligned(workspace, 16)) return fail(GDN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
            const Range wsr[] = {range("workspace", workspace, used)};
            GDN_TRY(check_no_overlap(wsr, 1, ins, 6));
            GDN_TRY(check_norm(norm, d, B * Hv * T, bf16, wsr, 1));
            GDN_TRY(check_no_overlap(wsr, 1, out_o, 1));
            if (final_state) {
                const Range fs[] = {range("final_state", final_state, st_bytes)};
                GDN_TRY(check_no_overlap(wsr, 1, fs, 1));
            }
        }
    }
    if (!final_state && T == 0) return GDN_OK;  // nothing to compute or write
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (segmented_path(s)) {
        if (norm) {  // fused into the output pass
            p.norm_w = norm->weight;
            p.norm_gate = norm->gate;
            p.norm_eps = norm->eps;
        }
        err = gdn::launch_prefill_seg(p, s->chunk, P, workspace, st);
    } else {
        err = gdn::launch_prefill_f32(p, s->chunk, bf16, st);  // float32 q/k/v, or bf16 below d = 128
        if (err == hipSuccess && norm && T > 0) {  // the norm as one more pass over o
            gdn::NormParams np;
            np.o = o;
            np.gate = norm->gate;
            np.weight = norm->weight;
            np.rows = B * Hv * T;
            np.D = d;
            np.gate_bf16 = bf16;
            np.eps = norm->eps;
            np.o_f16 = o16;
            err = gdn::launch_gated_rmsnorm(np, st);
        }
    }
    if (err != hipSuccess) return fail(GDN_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(err));
    return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_prefill(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const void *initial_state, void *o, void *final_state,
                       void *workspace, size_t workspace_bytes, const gdn_norm *norm, void *stream) {
    return prefill_impl(s, q, k, v, g, beta, initial_state, o, final_state, workspace, workspace_bytes, norm,
                        stream, false);
}

gdn_status gdn_prefill_static(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const void *initial_state, void *o, void *final_state,
                              size_t workspace_bytes, const gdn_norm *norm, void *stream) {
    if (workspace_bytes > GDN_STATIC_SCRATCH_BYTES)
        return fail(GDN_ERR_INVALID_ARG, "workspace_bytes %zu exceeds the static scratch of %zu bytes", workspace_bytes,
                    (size_t)GDN_STATIC_SCRATCH_BYTES);
    return prefill_impl(s, q, k, v, g, beta, initial_state, o, final_state, nullptr, workspace_bytes, norm, stream,
                        true);
}

size_t gdn_prefill_varlen_workspace_bytes(const gdn_shape *s) {
    if (check_common(s) != GDN_OK || s->seq_len < 0) return 0;
    if (s->qkv_dtype != GDN_DTYPE_BF16 || s->head_dim_k != 128 || (s->chunk != 32 && s->chunk != 64)) return 0;
    return (size_t)gdn::varlen_layout(s->batch, s->num_k_heads, s->num_v_heads, s->seq_len, s->chunk).bytes;
}

gdn_status gdn_prefill_varlen(const gdn_shape *s, const int32_t *cu_seqlens, const void *q, const void *k,
                              const void *v, const float *g, const float *beta, const void *initial_state, void *o,
                              void *final_state, void *workspace, size_t workspace_bytes, void *stream) {
    GDN_TRY(check_common(s));
    if (s->seq_len < 0) return fail(GDN_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", s->seq_len);
    if (s->qkv_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "packed sequences need bfloat16 q/k/v");
    if (s->chunk != 32 && s->chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "packed sequences need chunk 32 or 64 (got %d)", s->chunk);
    const int d = s->head_dim_k;
    if (d != 128) return fail(GDN_ERR_UNSUPPORTED, "packed sequences need head_dim 128 (got %d)", d);
    const int64_t N = s->batch, T = s->seq_len, Hk = s->num_k_heads, Hv = s->num_v_heads;
    if ((double)Hv * T * d > 4.0e15 || N > (1 << 24)) return fail(GDN_ERR_UNSUPPORTED, "tensor sizes overflow");
    const bool st16 = s->state_dtype != GDN_STATE_F32, o16 = s->o_dtype == GDN_OUT_F16;
    const int64_t qk_bytes = Hk * T * d * 2, v_bytes = Hv * T * d * 2, gb_bytes = Hv * T * 4;
    const int64_t o_bytes = Hv * T * d * (o16 ? 2 : 4);
    const int64_t st_bytes = N * Hv * d * d * (st16 ? 2 : 4);
    GDN_TRY(check_ptr(cu_seqlens, "cu_seqlens", 4));
    if (T > 0) {
        GDN_TRY(check_ptr(q, "q", 16));
        GDN_TRY(check_ptr(k, "k", 16));
        GDN_TRY(check_ptr(v, "v", 16));
        GDN_TRY(check_ptr(g, "g", 4));
        GDN_TRY(check_ptr(beta, "beta", 4));
        GDN_TRY(check_ptr(o, "o", 16));
    }
    if (initial_state) GDN_TRY(check_ptr(initial_state, "initial_state", 16));
    if (final_state) GDN_TRY(check_ptr(final_state, "final_state", 16));
    const gdn::VarlenLayout vl = gdn::varlen_layout(N, Hk, Hv, T, s->chunk);
    if (vl.nchunks > 0x7fffffff / (Hk > Hv ? Hk : Hv))
        return fail(GDN_ERR_UNSUPPORTED, "too many chunks for one launch");
    if (!workspace) return fail(GDN_ERR_INVALID_ARG, "workspace is NULL (%lld bytes needed)", (long long)vl.bytes);
    if ((int64_t)workspace_bytes < vl.bytes)
        return fail(GDN_ERR_INVALID_ARG, "workspace has %zu bytes, %lld needed", workspace_bytes, (long long)vl.bytes);
    if (!aligned(workspace, 16)) return fail(GDN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");

    const Range ins[] = {range("q", q, T ? qk_bytes : 0), range("k", k, T ? qk_bytes : 0),
                         range("v", v, T ? v_bytes : 0), range("g", g, T ? gb_bytes : 0),
                         range("beta", beta, T ? gb_bytes : 0), range("cu_seqlens", cu_seqlens, (N + 1) * 4),
                         range("initial_state", initial_state, initial_state ? st_bytes : 0)};
    const Range outs[] = {range("o", o, T ? o_bytes : 0), range("workspace", workspace, vl.bytes)};
    GDN_TRY(check_no_overlap(outs, 2, ins, 7));
    if (overlaps(outs[0], outs[1])) return fail(GDN_ERR_INVALID_ARG, "o overlaps workspace");
    if (final_state) {
        const Range out_s[] = {range("final_state", final_state, st_bytes)};
        GDN_TRY(check_no_overlap(out_s, 1, ins, 6));  // all but initial_state
        GDN_TRY(check_no_overlap(out_s, 1, outs, 2));
        if (initial_state && final_state != initial_state && overlaps(out_s[0], ins[6]))
            return fail(GDN_ERR_INVALID_ARG, "final_state partially overlaps initial_state");
    }

    gdn::PrefillParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.init_state = initial_state;
    p.o = o;
    p.final_state = final_state;
    p.B = (int32_t)N;
    p.T = (int32_t)T;
    p.Ts = (int32_t)T;
    p.Hk = s->num_k_heads;
    p.Hv = s->num_v_heads;
    p.D = d;
    p.head_map = (int32_t)s->head_map;
    p.scale = s->scale;
    p.init_f16 = p.final_f16 = st16;
    p.state_bf16 = s->state_dtype == GDN_STATE_BF16;
    p.o_f16 = o16;
    char *wsb = static_cast<char *>(workspace);
    p.seqs = reinterpret_cast<const int32_t *>(wsb + vl.seq_offset);
    p.chunks = reinterpret_cast<const int32_t *>(wsb + vl.chunk_offset);
    p.nchunks = (int32_t)vl.nchunks;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t err = gdn::launch_varlen_tables(cu_seqlens, (int32_t)N, (int32_t)T, s->chunk,
                                               reinterpret_cast<int32_t *>(wsb + vl.seq_offset),
                                               reinterpret_cast<int32_t *>(wsb + vl.chunk_offset),
                                               (int32_t)vl.nchunks, st);
    if (err == hipSuccess && T > 0) err = gdn::launch_chunk_prep(p, s->chunk, workspace, st);
    if (err == hipSuccess) err = gdn::launch_prefill_scan(p, s->chunk, workspace, st);
    if (err != hipSuccess) return fail(GDN_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(err));
    return GDN_OK;
}

gdn_status gdn_gated_rmsnorm(const gdn_shape *s, void *o, const void *gate, const float *weight, float eps,
                             void *stream) {
    GDN_TRY(check_common(s));
    if (s->seq_len < 0) return fail(GDN_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", s->seq_len);
    const int d = s->head_dim_v;
    if (d != 16 && d != 32 && d != 64 && d != 128)
        return fail(GDN_ERR_UNSUPPORTED, "gated_rmsnorm supports head_dim_v 16, 32, 64 or 128 (got %d)", d);
    if (!std::isfinite(eps) || eps < 0.0f) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const int64_t rows = (int64_t)s->batch * s->num_v_heads * s->seq_len;
    if (rows == 0) return GDN_OK;
    const bool bf16 = s->qkv_dtype == GDN_DTYPE_BF16;
    const bool o16 = s->o_dtype == GDN_OUT_F16;
    GDN_TRY(check_ptr(o, "o", 16));
    GDN_TRY(check_ptr(weight, "weight", 16));
    // a lane reads 4 (float32 o) or 8 (float16 o) gate values at once
    if (gate) GDN_TRY(check_ptr(gate, "gate", bf16 && !o16 ? 8 : 16));
    const Range ins[] = {range("gate", gate, gate ? rows * d * (bf16 ? 2 : 4) : 0), range("weight", weight, d * 4)};
    const Range outs[] = {range("o", o, rows * d * (o16 ? 2 : 4))};
    GDN_TRY(check_no_overlap(outs, 1, ins, 2));
    gdn::NormParams p;
    p.o = o;
    p.gate = gate;
    p.weight = weight;
    p.rows = rows;
    p.D = d;
    p.gate_bf16 = bf16;
    p.eps = eps;
    p.o_f16 = o16;
    const hipError_t err = gdn::launch_gated_rmsnorm(p, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GDN_ERR_HIP, "gated_rmsnorm launch failed: %s", hipGetErrorString(err));
    return GDN_OK;
}

gdn_status gdn_qkv_prologue(const gdn_shape *s, const void *x, const float *conv_weight, float *conv_state,
                            void *q, void *k, void *v, float eps, void *stream) {
    GDN_TRY(check_common(s));
    if (s->seq_len < 0) return fail(GDN_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", s->seq_len);
    const int d = s->head_dim_k;
    if (s->head_dim_v != d) return fail(GDN_ERR_UNSUPPORTED, "dk != dv (%d, %d) is not supported", d, s->head_dim_v);
    if (d != 16 && d != 32 && d != 64 && d != 128)
        return fail(GDN_ERR_UNSUPPORTED, "qkv_prologue supports head_dim 16, 32, 64 or 128 (got %d)", d);
    if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and > 0");
    const int64_t B = s->batch, T = s->seq_len, Hk = s->num_k_heads, Hv = s->num_v_heads;
    if (T == 0) return GDN_OK;
    const bool bf16 = s->qkv_dtype == GDN_DTYPE_BF16;
    const int64_t esz = bf16 ? 2 : 4, C = (2 * Hk + Hv) * d;
    GDN_TRY(check_ptr(x, "x", 16));
    GDN_TRY(check_ptr(conv_weight, "conv_weight", 16));
    if (conv_state) GDN_TRY(check_ptr(conv_state, "conv_state", 16));
    GDN_TRY(check_ptr(q, "q", 16));
    GDN_TRY(check_ptr(k, "k", 16));
    GDN_TRY(check_ptr(v, "v", 16));
    const Range ins[] = {range("x", x, B * T * C * esz), range("conv_weight", conv_weight, C * 4 * 4),
                         range("conv_state", conv_state, conv_state ? B * 3 * C * 4 : 0)};
    const Range outs[] = {range("q", q, B * Hk * T * d * esz), range("k", k, B * Hk * T * d * esz),
                          range("v", v, B * Hv * T * d * esz)};
    GDN_TRY(check_no_overlap(outs, 3, ins, 3));
    GDN_TRY(check_no_overlap(outs, 1, outs + 1, 2));
    GDN_TRY(check_no_overlap(outs + 1, 1, outs + 2, 1));
    const Range st[] = {range("conv_state", conv_state, conv_state ? B * 3 * C * 4 : 0)};
    GDN_TRY(check_no_overlap(st, 1, ins, 2));
    gdn::PrologueParams p;
    p.x = x;
    p.conv_weight = conv_weight;
    p.conv_state = conv_state;
    p.q = q;
    p.k = k;
    p.v = v;
    p.B = s->batch;
    p.T = s->seq_len;
    p.Hk = s->num_k_heads;
    p.Hv = s->num_v_heads;
    p.D = d;
    p.bf16 = bf16;
    p.eps = eps;
    const hipError_t err = gdn::launch_qkv_prologue(p, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GDN_ERR_HIP, "qkv_prologue launch failed: %s", hipGetErrorString(err));
    return GDN_OK;
}

}  // extern "C"

namespace {
// gdn_decode and gdn_kda_decode: g is [B][Hv] or, with kda, [B][Hv][dk]
gdn_status decode_impl(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, void *state, void *o, const gdn_norm *norm, void *stream, bool kda) {
    GDN_TRY(check_common(s));
    if (s->seq_len != 1) return fail(GDN_ERR_INVALID_ARG, "decode needs seq_len == 1 (got %d)", s->seq_len);
    const int d = s->head_dim_k;
    if (d != 32 && d != 64 && d != 128)
        return fail(GDN_ERR_UNSUPPORTED, "decode supports head_dim 32, 64 or 128 (got %d)", d);
    const bool bf16 = s->qkv_dtype == GDN_DTYPE_BF16;
    const int64_t B = s->batch, Hk = s->num_k_heads, Hv = s->num_v_heads;
    const int64_t esz = bf16 ? 2 : 4;
    GDN_TRY(check_ptr(q, "q", 16));
    GDN_TRY(check_ptr(k, "k", 16));
    GDN_TRY(check_ptr(v, "v", 16));
    GDN_TRY(check_ptr(g, "g", kda ? 16 : 4));
    GDN_TRY(check_ptr(beta, "beta", 4));
    GDN_TRY(check_ptr(state, "state", 16));
    GDN_TRY(check_ptr(o, "o", 16));
    const Range ins[] = {range("q", q, B * Hk * d * esz), range("k", k, B * Hk * d * esz),
                         range("v", v, B * Hv * d * esz), range("g", g, B * Hv * (kda ? d : 1) * 4),
                         range("beta", beta, B * Hv * 4)};
    const bool st16 = s->state_dtype != GDN_STATE_F32, o16 = s->o_dtype == GDN_OUT_F16;
    const Range outs[] = {range("o", o, B * Hv * d * (o16 ? 2 : 4)),
                          range("state", state, B * Hv * d * d * (st16 ? 2 : 4))};
    GDN_TRY(check_no_overlap(outs, 2, ins, 5));
    if (overlaps(outs[0], outs[1])) return fail(GDN_ERR_INVALID_ARG, "o overlaps state");
    GDN_TRY(check_norm(norm, d, B * Hv, bf16, outs, 2));

    gdn::DecodeParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.state = state;
    p.o = o;
    p.B = s->batch;
    p.Hk = s->num_k_heads;
    p.Hv = s->num_v_heads;
    p.D = d;
    p.head_map = (int32_t)s->head_map;
    p.scale = s->scale;
    p.state_f16 = st16;
    p.state_bf16 = s->state_dtype == GDN_STATE_BF16;
    p.o_f16 = o16;
    p.kda = kda;
    if (norm) {
        p.norm_w = norm->weight;
        p.norm_gate = norm->gate;
        p.norm_eps = norm->eps;
    }
    const hipError_t err = gdn::launch_decode(p, bf16, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GDN_ERR_HIP, "decode launch failed: %s", hipGetErrorString(err));
    return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_decode(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, void *state, void *o, const gdn_norm *norm, void *stream) {
    return decode_impl(s, q, k, v, g, beta, state, o, norm, stream, false);
}

gdn_status gdn_kda_decode(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, void *state, void *o, void *stream) {
    return decode_impl(s, q, k, v, g, beta, state, o, nullptr, stream, true);
}

gdn_status gdn_kda_prefill(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const void *initial_state, void *o, void *final_state,
                           void *workspace, size_t workspace_bytes, void *stream) {
    GDN_TRY(check_common(s));
    if (s->seq_len < 0) return fail(GDN_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", s->seq_len);
    const int d = s->head_dim_k;
    if (d != 128) return fail(GDN_ERR_UNSUPPORTED, "per-channel decay prefill supports head_dim 128 (got %d)", d);
    const bool bf16 = s->qkv_dtype == GDN_DTYPE_BF16;
    const int64_t B = s->batch, T = s->seq_len, Hk = s->num_k_heads, Hv = s->num_v_heads;
    if ((double)B * Hv * T * d > 4.0e15) return fail(GDN_ERR_UNSUPPORTED, "tensor sizes overflow");
    const int64_t esz = bf16 ? 2 : 4;
    const bool st16 = s->state_dtype != GDN_STATE_F32, o16 = s->o_dtype == GDN_OUT_F16;
    const int64_t qk_bytes = B * Hk * T * d * esz, v_bytes = B * Hv * T * d * esz, g_bytes = B * Hv * T * d * 4;
    const int64_t b_bytes = B * Hv * T * 4, o_bytes = B * Hv * T * d * (o16 ? 2 : 4);
    const int64_t st_bytes = B * Hv * d * d * (st16 ? 2 : 4);
    if (T > 0) {
        GDN_TRY(check_ptr(q, "q", 16));
        GDN_TRY(check_ptr(k, "k", 16));
        GDN_TRY(check_ptr(v, "v", 16));
        GDN_TRY(check_ptr(g, "g", 16));
        GDN_TRY(check_ptr(beta, "beta", 4));
        GDN_TRY(check_ptr(o, "o", 16));
    }
    if (initial_state) GDN_TRY(check_ptr(initial_state, "initial_state", 16));
    if (final_state) GDN_TRY(check_ptr(final_state, "final_state", 16));
    const Range ins[] = {range("q", q, T ? qk_bytes : 0), range("k", k, T ? qk_bytes : 0),
                         range("v", v, T ? v_bytes : 0), range("g", g, T ? g_bytes : 0),
                         range("beta", beta, T ? b_bytes : 0),
                         range("initial_state", initial_state, initial_state ? st_bytes : 0)};
    const Range out_o[] = {range("o", o, T ? o_bytes : 0)};
    GDN_TRY(check_no_overlap(out_o, 1, ins, 6));
    if (final_state) {
        const Range out_s[] = {range("final_state", final_state, st_bytes)};
        GDN_TRY(check_no_overlap(out_s, 1, ins, 5));
        GDN_TRY(check_no_overlap(out_s, 1, out_o, 1));
        if (initial_state && final_state != initial_state && overlaps(out_s[0], ins[5]))
            return fail(GDN_ERR_INVALID_ARG, "final_state partially overlaps initial_state");
    }
    // bf16 with chunk 32 or 64: the chunked form in 32-token chunks, segment-parallel within the
    // workspace given (as gdn_prefill); otherwise token by token
    const bool chunked = bf16 && (s->chunk == 32 || s->chunk == 64);
    int P = 1;
    if (chunked) {
        P = gdn::seg_count(B, Hv, T, 32, workspace_bytes, workspace != nullptr);
        if (P > 1) {
            const int64_t used = gdn::seg_workspace_bytes(B * Hv, P);
            if (!aligned(workspace, 16)) return fail(GDN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
            const Range wsr[] = {range("workspace", workspace, used)};
            GDN_TRY(check_no_overlap(wsr, 1, ins, 6));
            GDN_TRY(check_no_overlap(wsr, 1, out_o, 1));
            if (final_state) {
                const Range fs[] = {range("final_state", final_state, st_bytes)};
                GDN_TRY(check_no_overlap(wsr, 1, fs, 1));
            }
        }
    }
    if (!final_state && T == 0) return GDN_OK;
    gdn::PrefillParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.init_state = initial_state;
    p.o = o;
    p.final_state = final_state;
    p.B = s->batch;
    p.T = s->seq_len;
    p.Ts = s->seq_len;
    p.Hk = s->num_k_heads;
    p.Hv = s->num_v_heads;
    p.D = d;
    p.head_map = (int32_t)s->head_map;
    p.scale = s->scale;
    p.init_f16 = p.final_f16 = st16;
    p.state_bf16 = s->state_dtype == GDN_STATE_BF16;
    p.o_f16 = o16;
    const hipError_t err = chunked ? gdn::launch_prefill_seg(p, 32, P, workspace, static_cast<hipStream_t>(stream), true)
                                   : gdn::launch_kda_prefill(p, bf16, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GDN_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(err));
    return GDN_OK;
}

}  // extern "C"
