// Per-channel decay (the KDA variant): prefill of
//   S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t (scale q_t)
// with g_t one log-decay per key channel (the channel decay of the Kimi K3 experiments on the
// "master..kimi_slop" page; with every channel alike it is the gated delta rule). Per token,
// with alpha = exp(g_t) and the decayed state S diag(alpha):
//   r = S (alpha k),  p = S (alpha q),  delta = beta (v - r)
//   S <- S diag(alpha) + delta k^T,  o = scale (p + delta (k . q))
// The batched decode step of this variant is the decode kernel's per-channel branch.
//
// A recurrent kernel, one token after the other. A workgroup keeps 16 state rows of one (b, h)
// in registers: 8 compute waves of 2 rows (a row is 32 lanes x 4 columns), two waves per SIMD so
// that one wave's shuffle reductions overlap the other's arithmetic. A ninth wave streams the
// inputs in blocks of 16 tokens (k, q, the per-channel g, this block's v columns, beta) straight
// into a 3-slot LDS ring, two blocks ahead, with exact vmcnt waits; one LDS-only barrier per
// block. Tokens past the end run as no-op steps (g = 0, beta = 0 leave the state unchanged).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerWG = 16;
constexpr int kCompute = 8;                 // compute waves, 2 rows each
constexpr int kThreads = 64 * (kCompute + 1);
constexpr int kLPR = kD / 4;                // lanes per state row
constexpr int kBlock = 16;                  // tokens per ring slot
constexpr int kSlots = 3;

typedef __attribute__((address_space(3))) void lds_void;

// ring slot layout (bytes), sized for float32 q/k/v
constexpr int oK = 0;                        // [16][128] q/k element
constexpr int oQ = oK + kBlock * kD * 4;     // [16][128]
constexpr int oG = oQ + kBlock * kD * 4;     // [16][128] float
constexpr int oV = oG + kBlock * kD * 4;     // [16][16] this block's v columns
constexpr int oB = oV + kBlock * 16 * 4;     // [64] float (beta in the first 16)
constexpr int kSlotBytes = oB + 64 * 4;
constexpr int kSmemBytes = kSlots * kSlotBytes;

__device__ __forceinline__ void dma16(const void *g, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 4, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// barrier for LDS traffic only: outstanding global loads and stores stay in flight across it
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// v from the lane given by a DPP control (quad permutes and row mirrors stay in the VALU)
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// sum over the 32 lanes of a state row, in every lane of it: xor 1 and xor 2 (quad permutes),
// the 8-lane and 16-lane mirrors, then xor 16 (a swizzle within each 32-lane half)
__device__ __forceinline__ float row_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));  // xor 16
    return x;
}

template <typename E>
__device__ __forceinline__ f32x4 lds4(const unsigned char *p) {
    if constexpr (sizeof(E) == 4) {
        return *reinterpret_cast<const f32x4 *>(p);
    } else {
        const u16x4 u = *reinterpret_cast<const u16x4 *>(p);
        return f32x4{bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]), bf16_bits_to_f32(u[3])};
    }
}
template <typename E>
__device__ __forceinline__ float lds1(const unsigned char *p) {
    if constexpr (sizeof(E) == 4)
        return *reinterpret_cast<const float *>(p);
    else
        return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
}

// E: q/k/v element (float, or uint16_t bfloat16 bits)
template <typename E>
__global__ __launch_bounds__(kThreads) void gdn_kda_prefill_kernel(PrefillParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int ES = sizeof(E);
    constexpr int kRowVec = 16 / ES;                    // elements per 16-byte load
    constexpr int kQKInstr = kBlock * kD * ES / 1024;   // 1 KB DMA instructions for k (and for q)
    constexpr int kGInstr = kBlock * kD * 4 / 1024;
    constexpr int kPerBlock = 2 * kQKInstr + kGInstr + 2;  // + v, + beta
    static_assert(2 * kPerBlock <= 63, "vmcnt range");

    const int pair = blockIdx.x / (kD / kRowsPerWG), rb = blockIdx.x % (kD / kRowsPerWG);
    const int b = pair / p.Hv, h = pair % p.Hv;
    const int kh = key_head(h, p.Hk, p.Hv, p.head_map);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int T = p.T;
    const int nb = (T + kBlock - 1) / kBlock;

    if (wave == kCompute) {
        // ---------------------------------------------------------------- loader wave
        const E *kg = static_cast<const E *>(p.k) + ((int64_t)b * p.Hk + kh) * p.Ts * kD;
        const E *qg = static_cast<const E *>(p.q) + ((int64_t)b * p.Hk + kh) * p.Ts * kD;
        const E *vg = static_cast<const E *>(p.v) + (int64_t)pair * p.Ts * kD + rb * kRowsPerWG;
        const float *gg = p.g + (int64_t)pair * p.Ts * kD;
        const float *bg = p.beta + (int64_t)pair * p.Ts;
        // block c (< nb) into slot c % 3, tokens past the end clamped to the last one
        auto issue = [&](int c) {
            unsigned char *s = smem + (c % kSlots) * kSlotBytes;
            const int t0 = c * kBlock;
#pragma unroll
            for (int i = 0; i < kQKInstr; ++i) {
                const int e = (i * 64 + lane) * kRowVec;  // element of the [16][128] block
                const int64_t src = (int64_t)min(t0 + e / kD, T - 1) * kD + e % kD;
                dma16(kg + src, s + oK + i * 1024);
                dma16(qg + src, s + oQ + i * 1024);
            }
#pragma unroll
            for (int i = 0; i < kGInstr; ++i) {
                const int e = (i * 64 + lane) * 4;
                dma16(gg + (int64_t)min(t0 + e / kD, T - 1) * kD + e % kD, s + oG + i * 1024);
            }
            {  // v: 16 columns of each token, 16 / kRowVec lanes per token
                constexpr int lpt = 16 / kRowVec;
                const int t = min(t0 + min(lane / lpt, kBlock - 1), T - 1);
                dma16(vg + (int64_t)t * kD + (lane % lpt) * kRowVec, s + oV);
            }
            dma4(bg + min(t0 + min(lane, kBlock - 1), T - 1), s + oB);
        };
        if (nb > 1) {
            issue(0);
            issue(1);
            wait_vmcnt<kPerBlock>();  // block 0 has landed
        } else if (nb == 1) {
            issue(0);
            wait_vmcnt<0>();
        }
        lds_barrier();
        for (int c = 0; c < nb; ++c) {
            // slot (c + 2) % 3 held block c - 1, which every compute wave finished before this barrier
            if (c + 2 < nb) {
                issue(c + 2);
                wait_vmcnt<kPerBlock>();  // block c + 1 has landed
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
        }
        wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup
        return;
    }

    // -------------------------------------------------------------------- compute waves
    const int col = (lane % kLPR) * 4;
    const int lrow = wave * 2 + lane / kLPR;              // row within the workgroup
    const int row = rb * kRowsPerWG + lrow;
    const int64_t si = ((int64_t)pair * kD + row) * kD + col;
    f32x4 S = p.init_state ? load_state4(p.init_state, si, p.init_f16) : f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t obase = (int64_t)pair * p.Ts * kD + row;

    lds_barrier();
    for (int c = 0; c < nb; ++c) {
        const unsigned char *s = smem + (c % kSlots) * kSlotBytes;
#pragma unroll
        for (int u = 0; u < kBlock; ++u) {
            const int t = c * kBlock + u;
            const bool live = t < T;
            const f32x4 k = lds4<E>(s + oK + (u * kD + col) * ES);
            const f32x4 q = lds4<E>(s + oQ + (u * kD + col) * ES);
            const f32x4 g = *reinterpret_cast<const f32x4 *>(s + oG + (u * kD + col) * 4);
            const float v = lds1<E>(s + oV + (u * 16 + lrow) * ES);
            const float beta = live ? *reinterpret_cast<const float *>(s + oB + u * 4) : 0.0f;
            f32x4 al, ak, aq;
            float kq = 0.0f, r = 0.0f, pq = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                al[e] = live ? __expf(g[e]) : 1.0f;
                ak[e] = al[e] * k[e];
                aq[e] = al[e] * q[e];
                kq += k[e] * q[e];
                r += S[e] * ak[e];
                pq += S[e] * aq[e];
            }
            kq = row_sum(kq);
            r = row_sum(r);
            pq = row_sum(pq);
            const float delta = beta * (v - r);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[e] = al[e] * S[e] + delta * k[e];
            if (col == 0 && live) {
                const float oi = p.scale * (pq + delta * kq);
                if (p.o_f16)
                    static_cast<_Float16 *>(p.o)[obase + (int64_t)t * kD] = (_Float16)oi;
                else
                    static_cast<float *>(p.o)[obase + (int64_t)t * kD] = oi;
            }
        }
        lds_barrier();
    }
    if (p.final_state) store_state4(p.final_state, si, S, p.final_f16);
}

}  // namespace

hipError_t launch_kda_prefill(const PrefillParams &p, bool bf16, hipStream_t stream) {
    if (p.D != kD) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)p.B * p.Hv * (kD / kRowsPerWG);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const void *fn = bf16 ? reinterpret_cast<const void *>(&gdn_kda_prefill_kernel<uint16_t>)
                          : reinterpret_cast<const void *>(&gdn_kda_prefill_kernel<float>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    if (err != hipSuccess) return err;
    if (bf16)
        hipLaunchKernelGGL((gdn_kda_prefill_kernel<uint16_t>), dim3((unsigned)blocks), dim3(kThreads), kSmemBytes,
                           stream, p);
    else
        hipLaunchKernelGGL((gdn_kda_prefill_kernel<float>), dim3((unsigned)blocks), dim3(kThreads), kSmemBytes,
                           stream, p);
    return hipGetLastError();
}

}  // namespace gdn
