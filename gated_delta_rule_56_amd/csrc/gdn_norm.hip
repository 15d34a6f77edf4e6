// Gated RMSNorm of output rows (float32 or float16), in place: the output epilogue that the gated
// delta kernels on the "27b 935/47" page apply (the q8_gated_rmsnorm test, and
// the norm_weight / norm_eps arguments of gated_delta). For every row x of D
// values of o:
//   x <- x / sqrt(mean(x^2) + eps) * weight * silu(gate),  silu(z) = z / (1 + exp(-z))
// with weight [D] shared by all rows and the gate factor left out when there is
// no gate.
//
// A pure streaming pass (HBM-bound): a row is D / 4 lanes x 16 bytes, so a
// wave covers 64 / (D / 4) rows with coalesced 16-byte loads and stores; the
// sum of squares is reduced across the row's lanes with xor shuffles.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <typename GT>
__device__ __forceinline__ f32x4 load_gate(const GT *g);

template <>
__device__ __forceinline__ f32x4 load_gate<uint16_t>(const uint16_t *g) {
    const u16x4 u = __builtin_nontemporal_load(reinterpret_cast<const u16x4 *>(g));
    return f32x4{bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]), bf16_bits_to_f32(u[3])};
}

template <>
__device__ __forceinline__ f32x4 load_gate<float>(const float *g) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(g));
}

// 4 consecutive o values, float32 or float16 (rounded to nearest even on store)
__device__ __forceinline__ f32x4 load_o4(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ f32x4 load_o4(const _Float16 *p) {
    const f16x4 h = __builtin_nontemporal_load(reinterpret_cast<const f16x4 *>(p));
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
__device__ __forceinline__ void store_o4(float *p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store_o4(_Float16 *p, f32x4 v) {
    __builtin_nontemporal_store(f16x4{f16_out(v[0]), f16_out(v[1]), f16_out(v[2]), f16_out(v[3])},
                                reinterpret_cast<f16x4 *>(p));
}

// OT: float or _Float16 o; GT: uint16_t (bfloat16 bits) or float gate; kGate false: no gate factor
template <int D, typename OT, typename GT, bool kGate>
__global__ __launch_bounds__(kThreads) void gdn_gated_rmsnorm_kernel(OT *o, const GT *gate, const float *weight,
                                                                     float eps, int64_t rows) {
    constexpr int LPR = D / 4;     // lanes per row
    constexpr int RPW = 64 / LPR;  // rows per wave
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane % LPR;
    const int64_t row = ((int64_t)blockIdx.x * (kThreads / 64) + w) * RPW + lane / LPR;
    if (row >= rows) return;  // whole row groups: the shuffles below stay inside a group
    OT *px = o + row * D + 4 * li;
    const f32x4 x = load_o4(px);
    float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    const f32x4 wt = *reinterpret_cast<const f32x4 *>(weight + 4 * li);
    f32x4 y = (x * inv) * wt;
    if constexpr (kGate) {
        const f32x4 g = load_gate<GT>(gate + row * D + 4 * li);
        y = y * f32x4{silu(g[0]), silu(g[1]), silu(g[2]), silu(g[3])};
    }
    store_o4(px, y);
}

template <int D, typename OT>
hipError_t launch_do(const NormParams &p, hipStream_t stream) {
    constexpr int rows_per_block = (kThreads / 64) * (64 / (D / 4));
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
