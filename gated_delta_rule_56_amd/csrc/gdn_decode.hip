// Batched single-token gated delta rule step: a streaming, in-place update of
// fp32 states in HBM.
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
// Mapping: one workgroup (4 waves) per (b, h); a row of D floats is spread over
// D/4 lanes holding 16 bytes each, so a wave covers 256 contiguous bytes per
// access (fully coalesced 128-byte lines). Each lane first issues all of its
// row loads (D/4 * 16 bytes per lane for D = 128) to keep HBM busy, then
// reduces the two dot products across the row's lanes with xor shuffles and
// streams the updated rows back with non-temporal stores.
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

template <typename T>
__device__ __forceinline__ f32x4 load4(const T *p, int64_t i);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float *p, int64_t i) {
    return *reinterpret_cast<const f32x4 *>(p + i);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t *p, int64_t i) {
    u16x4 u = *reinterpret_cast<const u16x4 *>(p + i);
    return f32x4{bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]),
                 bf16_bits_to_f32(u[3])};
}

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <int D, typename T>
__global__ __launch_bounds__(kDecodeThreads) void gdn_decode_kernel(DecodeParams p) {
    constexpr int LPR = D / 4;                      // lanes per state row
    constexpr int RPA = 64 / LPR;                   // rows per wave per access
    constexpr int ROWS_PER_WAVE = D / (kDecodeThreads / 64);
    constexpr int ITERS = ROWS_PER_WAVE / RPA;
    static_assert(ITERS >= 1 && ROWS_PER_WAVE % RPA == 0, "row split");

    const int pair = blockIdx.x;
    const int b = pair / p.Hv, h = pair % p.Hv;
    const int kh = key_head(h, p.Hk, p.Hv, p.head_map);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (lane % LPR) * 4;
    const int sub = lane / LPR;

    const T *qp = static_cast<const T *>(p.q) + ((int64_t)b * p.Hk + kh) * D;
    const T *kp = static_cast<const T *>(p.k) + ((int64_t)b * p.Hk + kh) * D;
    const T *vp = static_cast<const T *>(p.v) + ((int64_t)b * p.Hv + h) * D;
    float *S = p.state + (int64_t)pair * D * D;

    const int row0 = wave * ROWS_PER_WAVE + sub;
    f32x4 s[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
        s[it] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(S + (int64_t)(row0 + it * RPA) * D + col));

    const f32x4 kv = load4<T>(kp, col);
    const f32x4 qv = load4<T>(qp, col);
    const float alpha = __expf(p.g[pair]);
    const float beta = p.beta[pair];
    const float kq = row_sum<LPR>(kv[0] * qv[0] + kv[1] * qv[1] + kv[2] * qv[2] + kv[3] * qv[3]);
    const float kappa = p.scale * kq;
    const float as = alpha * p.scale;

    float vrow[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) vrow[it] = load_elem<T>(vp, row0 + it * RPA);

#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const f32x4 x = s[it];
        float rk = x[0] * kv[0] + x[1] * kv[1] + x[2] * kv[2] + x[3] * kv[3];
        float rq = x[0] * qv[0] + x[1] * qv[1] + x[2] * qv[2] + x[3] * qv[3];
        rk = row_sum<LPR>(rk);
        rq = row_sum<LPR>(rq);
        const float delta = beta * (vrow[it] - alpha * rk);
        const f32x4 y = f32x4{alpha * x[0] + delta * kv[0], alpha * x[1] + delta * kv[1],
                              alpha * x[2] + delta * kv[2], alpha * x[3] + delta * kv[3]};
        const int row = row0 + it * RPA;
        __builtin_nontemporal_store(y, reinterpret_cast<f32x4 *>(S + (int64_t)row * D + col));
        if (col == 0) p.o[(int64_t)pair * D + row] = as * rq + delta * kappa;
    }
}

template <int D>
hipError_t launch_d(const DecodeParams &p, bool bf16, hipStream_t stream) {
    dim3 grid((unsigned)(p.B * p.Hv)), block(kDecodeThreads);
    if (bf16)
        hipLaunchKernelGGL((gdn_decode_kernel<D, uint16_t>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((gdn_decode_kernel<D, float>), grid, block, 0, stream, p);
    return hipGetLastError();
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
