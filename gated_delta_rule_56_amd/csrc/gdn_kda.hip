// Per-channel decay (the KDA variant): prefill of
//   S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t (scale q_t)
// with g_t one log-decay per key channel, token by token ("channel decay" of the Kimi K3
// experiments on the "master..kimi_slop" page; with every channel alike it is the gated delta
// rule). Per token, with alpha = exp(g_t) and the decayed state S diag(alpha):
//   r = S (alpha k),  p = S (alpha q),  delta = beta (v - r)
//   S <- S diag(alpha) + delta k^T,  o = scale (p + delta (k . q))
//
// A recurrent kernel, one token after the other: a workgroup keeps 16 state rows of one
// (b, h) in registers (4 waves of 4 rows; a row is 32 lanes x 4 columns), keeps the k, q, g,
// v, beta of the next kAhead tokens in flight in a register ring (each token's rows come from
// HBM, so the loads are issued that many tokens before use), and reduces the three dot
// products of a row across its 32 lanes with xor shuffles. Tokens past the end run as no-op
// steps (g = 0, beta = 0 leave the state unchanged exactly) so the loop has no branch. The chunked form of this variant
// (per-(t, s, channel) decays inside the chunk products) is not built.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kRowsPerWG = 16;
constexpr int kLPR = kD / 4;  // lanes per state row
constexpr int kAhead = 8;     // tokens whose inputs are in flight

template <typename T>
__device__ __forceinline__ f32x4 load4(const T *p, int64_t i);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float *p, int64_t i) {
    return *reinterpret_cast<const f32x4 *>(p + i);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t *p, int64_t i) {
    const u16x4 u = *reinterpret_cast<const u16x4 *>(p + i);
    return f32x4{bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]), bf16_bits_to_f32(u[3])};
}
template <typename T>
__device__ __forceinline__ float load1(const T *p, int64_t i) {
    if constexpr (sizeof(T) == 4)
        return p[i];
    else
        return bf16_bits_to_f32(p[i]);
}

__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < kLPR; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// inputs of one token for this lane
struct Tok {
    f32x4 k, q, g;
    float v[2], beta;
};

// E: q/k/v element (float, or uint16_t bfloat16 bits)
template <typename E>
__global__ __launch_bounds__(kThreads) void gdn_kda_prefill_kernel(PrefillParams p) {
    const int pair = blockIdx.x / (kD / kRowsPerWG), rb = blockIdx.x % (kD / kRowsPerWG);
    const int b = pair / p.Hv, h = pair % p.Hv;
    const int kh = key_head(h, p.Hk, p.Hv, p.head_map);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (lane % kLPR) * 4;
    const int row0 = rb * kRowsPerWG + wave * 4 + lane / kLPR;  // rows row0 and row0 + 2
    const int T = p.T;

    const E *qp = static_cast<const E *>(p.q) + ((int64_t)b * p.Hk + kh) * p.Ts * kD + col;
    const E *kp = static_cast<const E *>(p.k) + ((int64_t)b * p.Hk + kh) * p.Ts * kD + col;
    const E *vp = static_cast<const E *>(p.v) + (int64_t)pair * p.Ts * kD;
    const float *gp = p.g + (int64_t)pair * p.Ts * kD + col;
    const float *bp = p.beta + (int64_t)pair * p.Ts;

    f32x4 S[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int64_t si = ((int64_t)pair * kD + row0 + 2 * it) * kD + col;
        S[it] = p.init_state ? load_state4(p.init_state, si, p.init_f16) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // inputs of token t; past the end a no-op step (loads clamped to the last token)
    auto fetch = [&](int t) {
        const int tc = min(t, T - 1);
        const bool live = t < T;
        Tok x;
        x.k = load4<E>(kp, (int64_t)tc * kD);
        x.q = load4<E>(qp, (int64_t)tc * kD);
        const f32x4 gv = *reinterpret_cast<const f32x4 *>(gp + (int64_t)tc * kD);
        x.g = live ? gv : f32x4{0.f, 0.f, 0.f, 0.f};
        x.v[0] = load1<E>(vp, (int64_t)tc * kD + row0);
        x.v[1] = load1<E>(vp, (int64_t)tc * kD + row0 + 2);
        const float bt = bp[tc];
        x.beta = live ? bt : 0.0f;
        return x;
    };
    Tok ring[kAhead];
    if (T > 0) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u) ring[u] = fetch(u);
    }
    for (int t0 = 0; t0 < T; t0 += kAhead)
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        const int t = t0 + u;
        const Tok cur = ring[u];
        ring[u] = fetch(t + kAhead);
        f32x4 al, ak, aq;
        float kq = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            al[e] = __expf(cur.g[e]);
            ak[e] = al[e] * cur.k[e];
            aq[e] = al[e] * cur.q[e];
            kq += cur.k[e] * cur.q[e];
        }
        float r[2], pq[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            r[it] = S[it][0] * ak[0] + S[it][1] * ak[1] + S[it][2] * ak[2] + S[it][3] * ak[3];
            pq[it] = S[it][0] * aq[0] + S[it][1] * aq[1] + S[it][2] * aq[2] + S[it][3] * aq[3];
        }
        kq = row_sum(kq);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            r[it] = row_sum(r[it]);
            pq[it] = row_sum(pq[it]);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const float delta = cur.beta * (cur.v[it] - r[it]);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[it][e] = al[e] * S[it][e] + delta * cur.k[e];
            if (col == 0 && t < T) {
                const float oi = p.scale * (pq[it] + delta * kq);
                const int64_t oi_idx = ((int64_t)pair * p.Ts + t) * kD + row0 + 2 * it;
                if (p.o_f16)
                    static_cast<_Float16 *>(p.o)[oi_idx] = (_Float16)oi;
                else
                    static_cast<float *>(p.o)[oi_idx] = oi;
            }
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int it = 0; it < 2; ++it)
            store_state4(p.final_state, ((int64_t)pair * kD + row0 + 2 * it) * kD + col, S[it], p.final_f16);
    }
}

}  // namespace

hipError_t launch_kda_prefill(const PrefillParams &p, bool bf16, hipStream_t stream) {
    if (p.D != kD) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)p.B * p.Hv * (kD / kRowsPerWG);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL((gdn_kda_prefill_kernel<uint16_t>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((gdn_kda_prefill_kernel<float>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
