// Batched single-token gated delta rule step: a streaming, in-place update of
// float32 or float16 states in HBM (float32 arithmetic either way).
//
// For each (b, h) and each state row i (value dimension), with alpha = exp(g):
//   r_i = S[i,:] . k,  p_i = S[i,:] . q
//   delta_i = beta (v_i - alpha r_i)
//   S[i,:] <- alpha S[i,:] + delta_i k                       (the new state)
//   o_i = S_new[i,:] . (scale q) = alpha scale p_i + delta_i scale (k . q)
// which is S <- alpha S (I - beta k k^T) + beta v k^T and o = S (scale q). The
// factorisation through delta and (k . q) is the one of the tinygrad decode
// reference test (compare page "27b 935/47", gated_delta_decode test), which
// reads the output off the pre-update state as alpha S q + delta (k . q).
//
// Mapping: one workgroup (4 waves) per (b, h), or, when there are fewer (b, h) pairs than
// compute units (a single sequence has 32), SPLIT workgroups per (b, h) that take D / SPLIT
// state rows each, so that every CU streams its share; a state row is spread over
// lanes holding 16 bytes each (4 float32 or 8 float16 values; 8 bytes for
// float16 at D = 32), so each access of a wave covers whole 128-byte lines. Each lane first issues all of its
// row loads (D/4 * 16 bytes per lane for D = 128) to keep HBM busy, then
// reduces the two dot products across the row's lanes with xor shuffles and
// streams the updated rows back with non-temporal stores.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kDecodeThreads = 256;

template <typename T>
__device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

// N consecutive q / k values (float32 or bfloat16 bits) as floats
template <int N, typename T>
__device__ __forceinline__ void load_vec(const T *p, int64_t i, float *out) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(p + i + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) out[j + e] = a[e];
        }
    } else if constexpr (N == 8) {
        const u16x8 u = *reinterpret_cast<const u16x8 *>(p + i);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = bf16_bits_to_f32(u[e]);
    } else {
        const u16x4 u = *reinterpret_cast<const u16x4 *>(p + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = bf16_bits_to_f32(u[e]);
    }
}

// N consecutive state values (float32, float16 or bfloat16), loaded and stored non-temporally
template <int N, typename SD>
struct StateRow {
    typedef SD vec __attribute__((ext_vector_type(N)));
    vec x;
    __device__ __forceinline__ void load(const SD *p) { x = __builtin_nontemporal_load(reinterpret_cast<const vec *>(p)); }
    __device__ __forceinline__ float get(int e) const { return (float)x[e]; }
    __device__ __forceinline__ static void store(SD *p, const float *y) {
        vec v;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            if constexpr (std::is_same<SD, __bf16>::value)
                v[e] = bf16_out(y[e]);  // round to nearest even
            else if constexpr (sizeof(SD) == 2)
                v[e] = f16_out(y[e]);
            else
                v[e] = y[e];
        }
        __builtin_nontemporal_store(v, reinterpret_cast<vec *>(p));
    }
};

// columns per lane: 16 bytes of state, except where a wave would cover more rows than
// it owns (float16 states at D = 32)
template <int D, typename SD>
constexpr int cols_per_lane() { return sizeof(SD) == 2 && D >= 64 ? 8 : 4; }

// T: q/k/v element (float or bfloat16 bits); SD: state element (float, _Float16 or __bf16);
// workgroups per (b, h) when the pairs alone do not fill the GPU: as many as keep every wave at
// one full access of rows or more, at most 8
template <int D, typename SD>
constexpr int max_split() {
    constexpr int rpa = 64 / (D / cols_per_lane<D, SD>());
    constexpr int s = D / ((kDecodeThreads / 64) * rpa);
    return s > 8 ? 8 : s;
}

// kKda: one decay per key channel (g [B][Hv][D]) instead of one per head; SPLIT: workgroups per
// (b, h), each taking D / SPLIT consecutive rows; kNorm (SPLIT = 1): the output row of the pair
// is normalised before it is stored, o_i = x_i / sqrt(mean(x^2) + eps) * w_i * silu(gate_i), its
// sum of squares reduced over the workgroup through LDS
template <int D, typename T, typename SD, bool kKda, int SPLIT, bool kNorm = false>
__global__ __launch_bounds__(kDecodeThreads) void gdn_decode_kernel(DecodeParams p) {
    constexpr int CPL = cols_per_lane<D, SD>();
    constexpr int LPR = D / CPL;                    // lanes per state row
    constexpr int RPA = 64 / LPR;                   // rows per wave per access
    constexpr int ROWS_PER_WAVE = D / SPLIT / (kDecodeThreads / 64);
    constexpr int ITERS = ROWS_PER_WAVE / RPA;
    static_assert(ITERS >= 1 && ROWS_PER_WAVE % RPA == 0, "row split");

    const int pair = blockIdx.x / SPLIT;
    const int part = blockIdx.x % SPLIT;
    const int b = pair / p.Hv, h = pair % p.Hv;
    const int kh = key_head(h, p.Hk, p.Hv, p.head_map);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (lane % LPR) * CPL;
    const int sub = lane / LPR;

    const T *qp = static_cast<const T *>(p.q) + ((int64_t)b * p.Hk + kh) * D;
    const T *kp = static_cast<const T *>(p.k) + ((int64_t)b * p.Hk + kh) * D;
    const T *vp = static_cast<const T *>(p.v) + ((int64_t)b * p.Hv + h) * D;
    SD *S = static_cast<SD *>(p.state) + (int64_t)pair * D * D;

    const int row0 = part * (D / SPLIT) + wave * ROWS_PER_WAVE + sub;
    StateRow<CPL, SD> s[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) s[it].load(S + (int64_t)(row0 + it * RPA) * D + col);

    float kv[CPL], qv[CPL];
    load_vec<CPL>(kp, col, kv);
    load_vec<CPL>(qp, col, qv);
    const float beta = p.beta[pair];
    float kq = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) kq += kv[e] * qv[e];
    kq = group_sum<LPR>(kq);
    const float kappa = p.scale * kq;
    // per-channel decay: the decayed state S diag(alpha) meets k and q as S (alpha k), S (alpha q)
    float alpha = 1.0f, al[CPL], ak[CPL], aq[CPL];
    if constexpr (kKda) {
        float gv[CPL];
        load_vec<CPL>(p.g + (int64_t)pair * D, col, gv);
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            al[e] = __expf(gv[e]);
            ak[e] = al[e] * kv[e];
            aq[e] = al[e] * qv[e];
        }
    } else {
        alpha = __expf(p.g[pair]);
    }
    const float as = alpha * p.scale;

    float vrow[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) vrow[it] = load_elem<T>(vp, row0 + it * RPA);
    // the norm's gate and weight of this lane's rows, requested with the rows (lanes that hold
    // column 0 of a row produce its output)
    float gw[kNorm ? ITERS : 1], ov[kNorm ? ITERS : 1];
    if constexpr (kNorm) {
        static_assert(SPLIT == 1, "the fused norm needs whole rows of the pair in the workgroup");
        const T *gp = static_cast<const T *>(p.norm_gate) + (int64_t)pair * D;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int row = row0 + it * RPA;
            float gz = 1.0f;
            if (p.norm_gate) {
                const float z = load_elem<T>(gp, row);
                gz = z / (1.0f + __expf(-z));
            }
            gw[it] = gz * p.norm_w[row];
        }
    }

#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        float rk = 0.0f, rq = 0.0f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            rk += s[it].get(e) * (kKda ? ak[e] : kv[e]);
            rq += s[it].get(e) * (kKda ? aq[e] : qv[e]);
        }
        rk = group_sum<LPR>(rk);
        rq = group_sum<LPR>(rq);
        const float delta = beta * (vrow[it] - alpha * rk);  // alpha = 1 with per-channel decay
        float y[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e)  // one explicit fma: every instantiation rounds the same way
            y[e] = __builtin_fmaf(delta, kv[e], (kKda ? al[e] : alpha) * s[it].get(e));
        const int row = row0 + it * RPA;
        StateRow<CPL, SD>::store(S + (int64_t)row * D + col, y);
        const float oi = as * rq + delta * kappa;
        if constexpr (kNorm) {
            ov[it] = oi;
        } else if (col == 0) {
            if (p.o_f16)
                static_cast<_Float16 *>(p.o)[(int64_t)pair * D + row] = f16_out(oi);
            else
                static_cast<float *>(p.o)[(int64_t)pair * D + row] = oi;
        }
    }
    if constexpr (kNorm) {
        // sum of squares of the pair's D outputs: per lane over its rows, then over the row
        // holders of each wave and the waves through LDS (every lane of a row holds its output)
        __shared__ float red[(kDecodeThreads / 64) * RPA];
        float ss = 0.0f;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) ss += ov[it] * ov[it];
        if (col == 0) red[wave * RPA + sub] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int j = 0; j < (kDecodeThreads / 64) * RPA; ++j) tot += red[j];
        const float rinv = rsqrtf(tot / D + p.norm_eps);
        if (col == 0) {
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const int row = row0 + it * RPA;
                const float y = ov[it] * rinv * gw[it];
                if (p.o_f16)
                    static_cast<_Float16 *>(p.o)[(int64_t)pair * D + row] = f16_out(y);
                else
                    static_cast<float *>(p.o)[(int64_t)pair * D + row] = y;
            }
        }
    }
}

// fewer (b, h) pairs than this: split each pair's rows over max_split workgroups
constexpr int64_t kSplitBelow = 256;

template <int D, typename T, typename SD, bool kKda>
hipError_t launch_sd(const DecodeParams &p, hipStream_t stream) {
    constexpr int S = max_split<D, SD>();
    const int64_t pairs = (int64_t)p.B * p.Hv;
    const bool split = S > 1 && pairs < kSplitBelow;
    if (split)
        hipLaunchKernelGGL((gdn_decode_kernel<D, T, SD, kKda, S>), dim3((unsigned)(pairs * S)), dim3(kDecodeThreads),
                           0, stream, p);
    else if (!kKda && p.norm_w)
        hipLaunchKernelGGL((gdn_decode_kernel<D, T, SD, false, 1, true>), dim3((unsigned)pairs),
                           dim3(kDecodeThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((gdn_decode_kernel<D, T, SD, kKda, 1>), dim3((unsigned)pairs), dim3(kDecodeThreads), 0,
                           stream, p);
    hipError_t err = hipGetLastError();
    if (err == hipSuccess && p.norm_w && split) {
        // a pair's rows are spread over S workgroups: the norm as its own pass over o
        NormParams np;
        np.o = p.o;
        np.gate = p.norm_gate;
        np.weight = p.norm_w;
        np.rows = pairs;
        np.D = D;
        np.gate_bf16 = sizeof(T) == 2;
        np.eps = p.norm_eps;
        np.o_f16 = p.o_f16;
        err = launch_gated_rmsnorm(np, stream);
    }
    return err;
}

template <int D, typename T>
hipError_t launch_dt(const DecodeParams &p, hipStream_t stream) {
    if (p.kda) {
        if (!p.state_f16) return launch_sd<D, T, float, true>(p, stream);
        return p.state_bf16 ? launch_sd<D, T, __bf16, true>(p, stream) : launch_sd<D, T, _Float16, true>(p, stream);
    }
    if (!p.state_f16) return launch_sd<D, T, float, false>(p, stream);
    return p.state_bf16 ? launch_sd<D, T, __bf16, false>(p, stream) : launch_sd<D, T, _Float16, false>(p, stream);
}

template <int D>
hipError_t launch_d(const DecodeParams &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_dt<D, uint16_t>(p, stream) : launch_dt<D, float>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, bool bf16, hipStream_t stream) {
    switch (p.D) {
        case 32: return launch_d<32>(p, bf16, stream);
        case 64: return launch_d<64>(p, bf16, stream);
        case 128: return launch_d<128>(p, bf16, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
