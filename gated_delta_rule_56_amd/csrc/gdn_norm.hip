// Gated RMSNorm of output rows (float32 or float16), in place: the output epilogue that the gated
// delta kernels on the "27b 935/47" page apply (the q8_gated_rmsnorm test, and
// the norm_weight / norm_eps arguments of gated_delta). For every row x of D
// values of o:
//   x <- x / sqrt(mean(x^2) + eps) * weight * silu(gate),  silu(z) = z / (1 + exp(-z))
// with weight [D] shared by all rows and the gate factor left out when there is
// no gate.
//
// A pure streaming pass (HBM-bound): a row is D / V lanes x 16 bytes (V = 4 float32
// or 8 float16 values per lane), so a wave covers 64 V / D rows with coalesced
// 16-byte loads and stores; the sum of squares is reduced across the row's lanes
// with DPP adds.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// A lane handles 16 bytes of o: 4 float32 or 8 float16 values (V), with the gate and the
// weight loaded to match.
template <int V>
struct Vals {
    float x[V];
};

__device__ __forceinline__ Vals<4> load_o(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return Vals<4>{{v[0], v[1], v[2], v[3]}};
}
__device__ __forceinline__ Vals<8> load_o(const _Float16 *p) {
    const f16x8 h = __builtin_nontemporal_load(reinterpret_cast<const f16x8 *>(p));
    Vals<8> r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.x[e] = (float)h[e];
    return r;
}
// float16 o is rounded to nearest even on store
__device__ __forceinline__ void store_o(float *p, const Vals<4> &y) {
    __builtin_nontemporal_store(f32x4{y.x[0], y.x[1], y.x[2], y.x[3]}, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store_o(_Float16 *p, const Vals<8> &y) {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f16_out(y.x[e]);
    __builtin_nontemporal_store(h, reinterpret_cast<f16x8 *>(p));
}

template <int V>
__device__ __forceinline__ Vals<V> load_gate(const uint16_t *g) {  // bfloat16 bits
    Vals<V> r;
    if constexpr (V == 4) {
        const u16x4 u = __builtin_nontemporal_load(reinterpret_cast<const u16x4 *>(g));
#pragma unroll
        for (int e = 0; e < 4; ++e) r.x[e] = bf16_bits_to_f32(u[e]);
    } else {
        const u16x8 u = __builtin_nontemporal_load(reinterpret_cast<const u16x8 *>(g));
#pragma unroll
        for (int e = 0; e < 8; ++e) r.x[e] = bf16_bits_to_f32(u[e]);
    }
    return r;
}
template <int V>
__device__ __forceinline__ Vals<V> load_gate(const float *g) {
    Vals<V> r;
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(g) + h);
#pragma unroll
        for (int e = 0; e < 4; ++e) r.x[4 * h + e] = v[e];
    }
    return r;
}

// OT: float or _Float16 o; GT: uint16_t (bfloat16 bits) or float gate; kGate false: no gate factor
template <int D, typename OT, typename GT, bool kGate>
__global__ __launch_bounds__(kThreads) void gdn_gated_rmsnorm_kernel(OT *o, const GT *gate, const float *weight,
                                                                     float eps, int64_t rows) {
    constexpr int V = 16 / sizeof(OT);  // values per lane
    constexpr int LPR = D / V;          // lanes per row
    constexpr int RPW = 64 / LPR;       // rows per wave
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane % LPR;
    const int64_t row = ((int64_t)blockIdx.x * (kThreads / 64) + w) * RPW + lane / LPR;
    if (row >= rows) return;  // whole row groups: the shuffles below stay inside a group
    OT *px = o + row * D + V * li;
    const Vals<V> x = load_o(px);
    Vals<V> g;
    if constexpr (kGate) g = load_gate<V>(gate + row * D + V * li);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < V; ++e) ss += x.x[e] * x.x[e];
    ss = group_sum<LPR>(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    Vals<V> y;
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        const f32x4 wt = *reinterpret_cast<const f32x4 *>(weight + V * li + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = (x.x[4 * h + e] * inv) * wt[e];
            if constexpr (kGate) t = t * silu(g.x[4 * h + e]);
            y.x[4 * h + e] = t;
        }
    }
    store_o(px, y);
}

template <int D, typename OT>
hipError_t launch_do(const NormParams &p, hipStream_t stream) {
    constexpr int rows_per_block = (kThreads / 64) * (64 / (D / (16 / (int)sizeof(OT))));
    const int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
    OT *o = static_cast<OT *>(p.o);
    if (!p.gate) {
        hipLaunchKernelGGL((gdn_gated_rmsnorm_kernel<D, OT, float, false>), grid, block, 0, stream, o,
                           static_cast<const float *>(nullptr), p.weight, p.eps, p.rows);
    } else if (p.gate_bf16) {
        hipLaunchKernelGGL((gdn_gated_rmsnorm_kernel<D, OT, uint16_t, true>), grid, block, 0, stream, o,
                           static_cast<const uint16_t *>(p.gate), p.weight, p.eps, p.rows);
    } else {
        hipLaunchKernelGGL((gdn_gated_rmsnorm_kernel<D, OT, float, true>), grid, block, 0, stream, o,
                           static_cast<const float *>(p.gate), p.weight, p.eps, p.rows);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const NormParams &p, hipStream_t stream) {
    return p.o_f16 ? launch_do<D, _Float16>(p, stream) : launch_do<D, float>(p, stream);
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormParams &p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    switch (p.D) {
        case 16: return launch_d<16>(p, stream);
        case 32: return launch_d<32>(p, stream);
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
