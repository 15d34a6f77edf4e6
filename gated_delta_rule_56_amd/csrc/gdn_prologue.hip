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
// A workgroup covers 1024 consecutive channels (whole heads) of one run of R
// consecutive tokens, consecutive workgroups the next channels of the same
// rows. Each lane owns 4 channels: it issues the loads of all R + 3 window rows
// at once (addresses clamped into the sequence, out-of-range rows replaced by
// state rows or zeros after the load), slides a 4-row window over them in
// registers and stores each output row right away; for q and k the head's
// D / 4 lanes reduce the sum of squares with DPP adds. No LDS and no
// barrier: HBM-bound, x read once (plus 3 rows per run, which hit in L2), q, k,
// v written once.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTaps = 4;

// silu with the hardware reciprocal (about 1 ulp): the exact division costs about ten
// instructions, and this kernel evaluates one silu per channel and token
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kCpl = 4;  // channels per lane

// kCpl consecutive channels of one row, as loaded: 8 bytes of bf16 or 16 bytes of fp32
template <bool kBf16>
struct Raw;
template <>
struct Raw<true> {
    u16x4 u;
    __device__ __forceinline__ void load(const void *base, int64_t idx) {
        u = *reinterpret_cast<const u16x4 *>(static_cast<const uint16_t *>(base) + idx);
    }
    __device__ __forceinline__ float get(int e) const { return bf16_bits_to_f32(u[e]); }
};
template <>
struct Raw<false> {
    f32x4 a;
    __device__ __forceinline__ void load(const void *base, int64_t idx) {
        a = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
    }
    __device__ __forceinline__ float get(int e) const { return a[e]; }
};

// outputs are written once and read by a later kernel: streamed past the caches
template <bool kBf16>
__device__ __forceinline__ void store_row(void *base, int64_t idx, const float *y) {
    if constexpr (kBf16) {
        // round to nearest even (gfx950 converts two values per instruction)
        const bf16x4 h{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        __builtin_nontemporal_store(__builtin_bit_cast(u16x4, h), reinterpret_cast<u16x4 *>(static_cast<uint16_t *>(base) + idx));
    } else {
        __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4 *>(static_cast<float *>(base) + idx));
    }
}

// tokens per lane: the raw window rows of a run stay in registers
template <bool kBf16>
constexpr int run_len() { return kBf16 ? 16 : 8; }

template <int D, bool kBf16>
__global__ __launch_bounds__(kThreads) void gdn_qkv_prologue_kernel(PrologueParams p) {
    constexpr int LPR = D / kCpl;                 // lanes per head row
    constexpr int R = run_len<kBf16>();           // tokens per run
    constexpr int K1 = kTaps - 1;

    const int H3 = 2 * p.Hk + p.Hv;
    const int64_t C = (int64_t)H3 * D;
    const int nblk = (int)((C + kThreads * kCpl - 1) / (kThreads * kCpl));  // channel blocks per row
    // channel blocks vary fastest: consecutive workgroups read consecutive stretches of the same rows
    const int blk = blockIdx.x % nblk;
    const int tile = blockIdx.x / nblk;  // (b, token run)
    const int ntile = (p.T + R - 1) / R;
    const int b = tile / ntile;
    const int tb = (tile % ntile) * R;  // first token of this run
    const int64_t ch = ((int64_t)blk * kThreads + threadIdx.x) * kCpl;  // first channel of this lane
    if (ch >= C) return;  // whole heads: a head's lanes are all past the last channel or none is
    const int hd = (int)(ch / D), li = (int)(ch % D) / kCpl;
    const int64_t xb = (int64_t)b * p.T;

    // window rows tb - 3 .. tb + R - 1, every load in bounds (row clamped into [0, T))
    Raw<kBf16> xr[R + K1];
#pragma unroll
    for (int r = 0; r < R + K1; ++r) {
        const int tau = min(max(tb - K1 + r, 0), p.T - 1);
        xr[r].load(p.x, (xb + tau) * C + ch);
    }
    // rows before t = 0 (only the run that starts the sequence): the conv state, or zeros
    const bool first = tb == 0;
    f32x4 st[K1];
#pragma unroll
    for (int j = 0; j < K1; ++j)
        st[j] = first && p.conv_state ? *reinterpret_cast<const f32x4 *>(p.conv_state + ((int64_t)b * K1 + j) * C + ch)
                                      : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float w[kCpl][kTaps];
#pragma unroll
    for (int e = 0; e < kCpl; ++e) {
        const f32x4 wv = *reinterpret_cast<const f32x4 *>(p.conv_weight + (ch + e) * kTaps);
#pragma unroll
        for (int i = 0; i < kTaps; ++i) w[e][i] = wv[i];
    }

    const bool normed = hd < 2 * p.Hk;
    void *dst = hd < p.Hk ? p.q : hd < 2 * p.Hk ? p.k : p.v;
    const int dh = hd < p.Hk ? hd : hd < 2 * p.Hk ? hd - p.Hk : hd - 2 * p.Hk;
    const int nh = hd < 2 * p.Hk ? p.Hk : p.Hv;
    const int64_t obase = (((int64_t)b * nh + dh) * p.T + tb) * D + kCpl * li;
    // window value of row r, channel e: state rows before t = 0, zero rows past the end
    auto win = [&](int r, int e) {
        if (r < K1 && first) return st[r][e];
        return tb - K1 + r < p.T ? xr[r].get(e) : 0.0f;
    };
#pragma unroll
    for (int j = 0; j < R; ++j) {
        float y[kCpl];
#pragma unroll
        for (int e = 0; e < kCpl; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < kTaps; ++i) acc += win(j + i, e) * w[e][i];
            y[e] = silu(acc);
        }
        if (normed) {  // uniform over the row group: every lane of a row takes this branch together
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < kCpl; ++e) ss += y[e] * y[e];
            ss = group_sum<LPR>(ss);
            const float f = __builtin_amdgcn_rsqf(ss + p.eps);
#pragma unroll
            for (int e = 0; e < kCpl; ++e) y[e] *= f;
        }
        if (tb + j < p.T) store_row<kBf16>(dst, obase + (int64_t)j * D, y);
    }

    // continuation state: the last 3 window rows of the whole sequence, written by the run that
    // read the old state (it alone reads it, and its reads have completed: their values are used above)
    if (first && p.conv_state) {
#pragma unroll
        for (int j = 0; j < K1; ++j) {
            const int tau = p.T - K1 + j;  // token of the new state row j
            f32x4 v;
            if (tau >= 0) {
                Raw<kBf16> rr;
                rr.load(p.x, (xb + tau) * C + ch);
                v = f32x4{rr.get(0), rr.get(1), rr.get(2), rr.get(3)};
            } else {  // T < 3: old state row T + j
                v = p.T + j == 0 ? st[0] : p.T + j == 1 ? st[1] : st[2];
            }
            *reinterpret_cast<f32x4 *>(p.conv_state + ((int64_t)b * K1 + j) * C + ch) = v;
        }
    }
}

template <int D, bool kBf16>
hipError_t launch_dt(const PrologueParams &p, hipStream_t stream) {
    const int64_t C = (int64_t)(2 * p.Hk + p.Hv) * D;
    const int64_t nblk = (C + kThreads * kCpl - 1) / (kThreads * kCpl);
    const int64_t blocks = (int64_t)p.B * ((p.T + run_len<kBf16>() - 1) / run_len<kBf16>()) * nblk;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gdn_qkv_prologue_kernel<D, kBf16>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrologueParams &p, hipStream_t stream) {
    return p.bf16 ? launch_dt<D, true>(p, stream) : launch_dt<D, false>(p, stream);
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
