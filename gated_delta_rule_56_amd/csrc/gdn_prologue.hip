// Input prologue of the scan in one pass: the causal depthwise convolution
// with SiLU and the q | k | v split with per-head L2 normalisation of q and k
// (causal_conv_silu and gdn_qkv on the "27b 935/47" page). For every
// sequence b and channel c of the raw projections x [B][T][(2 Hk + Hv) d],
// with window = the 3 state rows before t = 0 followed by the rows of x:
//   y[t][c] = silu(sum_{i<4} window[t + i][c] * w[c][i])
// then channels [0, Hk d) form q, [Hk d, 2 Hk d) k and the rest v, each in
// heads of d channels; q and k heads are scaled by 1 / sqrt(sum of squares +
// eps). Outputs are head-major ([B][H][T][d]), the layout gdn_prefill reads;
// the state becomes the last 3 window rows.
//
// One workgroup per (b, head of the 2 Hk + Hv, tile of 64 tokens): the tile's
// window (67 rows of d channels) is staged in LDS as fp32, each lane then
// convolves 8 channels of one token and, for q and k, the head's d / 8 lanes
// reduce the sum of squares with xor shuffles. HBM-bound: x read once (plus 3
// rows per tile), q, k, v written once.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;  // tokens per workgroup
constexpr int kTaps = 4;

// silu with the hardware reciprocal (about 1 ulp): the exact division costs about ten
// instructions, and this kernel evaluates one silu per channel and token
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool kBf16>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float *out) {
    if constexpr (kBf16) {
        const u16x8 u = *reinterpret_cast<const u16x8 *>(static_cast<const uint16_t *>(base) + idx);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = bf16_bits_to_f32(u[e]);
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[e] = a[e];
            out[4 + e] = b[e];
        }
    }
}

template <bool kBf16>
__device__ __forceinline__ void store8(void *base, int64_t idx, const float *y) {
    if constexpr (kBf16) {
        bf16x8 h;  // round to nearest even (gfx950 converts two values per instruction)
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (__bf16)y[e];
        *reinterpret_cast<u16x8 *>(static_cast<uint16_t *>(base) + idx) = __builtin_bit_cast(u16x8, h);
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + idx) = f32x4{y[0], y[1], y[2], y[3]};
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + idx + 4) = f32x4{y[4], y[5], y[6], y[7]};
    }
}

template <int D, bool kBf16>
__global__ __launch_bounds__(kThreads) void gdn_qkv_prologue_kernel(PrologueParams p) {
    constexpr int LPR = D / 8;             // lanes per token row (8 channels each)
    constexpr int RP = kThreads / LPR;     // rows per pass
    constexpr int WR = kTile + kTaps - 1;  // window rows
    __shared__ float win[WR][D];

    const int H3 = 2 * p.Hk + p.Hv;
    const int ntile = (p.T + kTile - 1) / kTile;
    // heads vary fastest, so that the workgroups in flight together read whole token rows of x
    const int hd = blockIdx.x % H3;
    const int tile = (blockIdx.x / H3) % ntile;
    const int b = blockIdx.x / (ntile * H3);
    const int64_t C = (int64_t)H3 * D;
    const int t0 = tile * kTile;
    const int tid = threadIdx.x, rr = tid / LPR, li = tid % LPR;
    const int64_t ch = (int64_t)hd * D + 8 * li;  // first channel of this lane

    // window rows: token t0 - 3 + r; state rows before t = 0, zero past the end
    for (int r = rr; r < WR; r += RP) {
        const int tau = t0 - (kTaps - 1) + r;
        float v8[8];
        if (tau < 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v8[e] = p.conv_state ? p.conv_state[((int64_t)b * (kTaps - 1) + (kTaps - 1) + tau) * C + ch + e] : 0.0f;
        } else if (tau < p.T) {
            load8<kBf16>(p.x, ((int64_t)b * p.T + tau) * C + ch, v8);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = 0.0f;
        }
        *reinterpret_cast<f32x4 *>(&win[r][8 * li]) = f32x4{v8[0], v8[1], v8[2], v8[3]};
        *reinterpret_cast<f32x4 *>(&win[r][8 * li + 4]) = f32x4{v8[4], v8[5], v8[6], v8[7]};
    }
    float w8[8][kTaps];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const f32x4 wv = *reinterpret_cast<const f32x4 *>(p.conv_weight + (ch + e) * kTaps);
#pragma unroll
        for (int i = 0; i < kTaps; ++i) w8[e][i] = wv[i];
    }
    __syncthreads();

    const bool normed = hd < 2 * p.Hk;
    void *dst = hd < p.Hk ? p.q : hd < 2 * p.Hk ? p.k : p.v;
    const int dh = hd < p.Hk ? hd : hd < 2 * p.Hk ? hd - p.Hk : hd - 2 * p.Hk;
    const int nh = hd < 2 * p.Hk ? p.Hk : p.Hv;
    for (int r = rr; r < kTile; r += RP) {  // every lane of a row takes the same trip count
        const int t = t0 + r;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < kTaps; ++i) acc += win[r + i][8 * li + e] * w8[e][i];
            y[e] = silu(acc);
        }
        if (normed) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
            const float f = __builtin_amdgcn_rsqf(ss + p.eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= f;
        }
        if (t < p.T) store8<kBf16>(dst, (((int64_t)b * nh + dh) * p.T + t) * D + 8 * li, y);
    }

    // continuation state: the last 3 window rows of the whole sequence, written by the first
    // tile's workgroup (the only one that reads the old state, and only before the barrier above)
    if (p.conv_state && tile == 0) {
        for (int j = rr; j < kTaps - 1; j += RP) {
            const int tau = p.T - (kTaps - 1) + j;  // token of the new state row j
            float v8[8];
            if (tau < kTile) {  // in this tile's window (row tau + 3)
#pragma unroll
                for (int e = 0; e < 8; ++e) v8[e] = win[tau + kTaps - 1][8 * li + e];
            } else {
                load8<kBf16>(p.x, ((int64_t)b * p.T + tau) * C + ch, v8);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) p.conv_state[((int64_t)b * (kTaps - 1) + j) * C + ch + e] = v8[e];
        }
    }
}

template <int D>
hipError_t launch_d(const PrologueParams &p, hipStream_t stream) {
    const int64_t ntile = (p.T + kTile - 1) / kTile;
    const int64_t blocks = (int64_t)p.B * (2 * p.Hk + p.Hv) * ntile;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (p.bf16)
        hipLaunchKernelGGL((gdn_qkv_prologue_kernel<D, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((gdn_qkv_prologue_kernel<D, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_prologue(const PrologueParams &p, hipStream_t stream) {
    if (p.T == 0) return hipSuccess;
    switch (p.D) {
        case 16: return launch_d<16>(p, stream);
        case 32: return launch_d<32>(p, stream);
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
