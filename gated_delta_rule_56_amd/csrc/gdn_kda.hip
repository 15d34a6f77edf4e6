// Per-channel decay (the KDA variant): prefill of
//   S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t (scale q_t)
// with g_t one log-decay per key channel (the channel decay of the Kimi K3 experiments on the
// "master..kimi_slop" page; with every channel alike it is the gated delta rule). Per token,
// with alpha = exp(g_t) and the decayed state D = S diag(alpha):
//   r = D k,  p = D q,  delta = beta (v - r)
//   S <- D + delta k^T,  o = scale (p + delta (k . q))
// The batched decode step of this variant is the decode kernel's per-channel branch.
//
// A recurrent kernel, one token after the other. A workgroup keeps 16 state rows of one (b, h)
// in registers: 4 compute waves of 4 rows, one per SIMD; a row is 16 lanes x 8 columns (lane i
// holds columns 4i .. 4i + 3 and 64 + 4i .. 64 + 4i + 3, so that the 16 lanes of a row read
// 256 contiguous bytes of an operand row per LDS instruction). The row sums of the token step
// then stay inside one 16-lane DPP row: four DPP adds, no cross-row swizzle.
// A fifth wave streams the inputs in blocks of 16 tokens (k, q, the per-channel g, this block's v
// columns, beta) straight into a 4-slot LDS ring, three blocks ahead, with exact vmcnt waits.
// What does not depend on the state row is formed once per block rather than once per row: while
// the compute waves run block c, they also turn block c + 1 into alpha = exp(g), k and q (all
// float32), beta and k . q per token, in a double-buffered LDS area. Every row reads the three
// vectors of every token, so the step is bound by LDS bandwidth (24 KB per token and
// workgroup) about as much as by VALU issue. The token step is
// then two dot products with their 16-lane row sums, the update, and
// o, which each row keeps in a register per token and stores once per block. One LDS-only
// barrier per block. Tokens past the end run as no-op steps (alpha = 1, beta = 0).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerWG = 16;
constexpr int kCompute = 4;                 // compute waves, 4 rows each
constexpr int kThreads = 64 * (kCompute + 1);
constexpr int kLPR = 16;                    // lanes per state row (8 columns each)
constexpr int kBlock = 16;                  // tokens per ring slot
constexpr int kSlots = 4;
static_assert(kBlock == kLPR, "lane i of a row keeps the o of token i of a block");

typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x2 __attribute__((ext_vector_type(2)));

// LDS layout (bytes) for q/k/v element E
template <typename E>
struct KdaSmem {
    static constexpr int ES = sizeof(E);
    // input ring slot
    static constexpr int oK = 0;                          // [16][128] E
    static constexpr int oQ = oK + kBlock * kD * ES;      // [16][128] E
    static constexpr int oG = oQ + kBlock * kD * ES;      // [16][128] float
    static constexpr int oV = oG + kBlock * kD * 4;       // [16][16] E (1 KB: one load of 64 lanes)
    static constexpr int oB = oV + 1024;                  // [64] float (beta in the first 16)
    static constexpr int kSlotBytes = oB + 256;
    static constexpr int kRing = kSlots * kSlotBytes;
    // per-block operands, two buffers
    static constexpr int pAL = 0;                         // [16][128] float alpha
    static constexpr int pKF = pAL + kBlock * kD * 4;     // [16][128] float k
    static constexpr int pQF = pKF + kBlock * kD * 4;     // [16][128] float q
    static constexpr int pBK = pQF + kBlock * kD * 4;     // [16] (beta, k . q)
    static constexpr int kOpBytes = pBK + kBlock * 8;
    static constexpr int kBytes = kRing + 2 * kOpBytes;
    static_assert(kBytes <= 160 * 1024, "LDS");
};

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
// Operands of one token for one lane: alpha, k and q at the lane's 8 columns, beta and k . q,
// and v of the lane's row
struct TokenOps {
    f32x4 al0, al1, k0, k1, q0, q1;
    f32x2 bk;
    float v;
};

// At most two waves share a SIMD (one compute wave, plus the loader on one of them), so the
// compiler may spend registers on holding the next token's operands.
template <typename E>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gdn_kda_prefill_kernel(PrefillParams p) {
    using L = KdaSmem<E>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int ES = sizeof(E);
    constexpr int kRowVec = 16 / ES;                    // elements per 16-byte load
    constexpr int kQKInstr = kBlock * kD * ES / 1024;   // 1 KB DMA instructions for k (and for q)
    constexpr int kGInstr = kBlock * kD * 4 / 1024;
    constexpr int kPerBlock = 2 * kQKInstr + kGInstr + 2;  // + v, + beta
    static_assert(kPerBlock <= 63, "vmcnt range");

    // workgroup -> (b, h, row block): the 8 row blocks of one (b, h), which read the same k, q and
    // g, sit on one XCD and share its L2 (workgroups go round-robin over the 8 XCDs)
    const int nwg = gridDim.x;
    int lin = blockIdx.x;
    if ((nwg & 7) == 0) lin = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int pair = lin / (kD / kRowsPerWG), rb = lin % (kD / kRowsPerWG);
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
        // block c (< nb) into slot c % 4, tokens past the end clamped to the last one
        auto issue = [&](int c) {
            unsigned char *s = smem + (c % kSlots) * L::kSlotBytes;
            const int t0 = c * kBlock;
#pragma unroll
            for (int i = 0; i < kQKInstr; ++i) {
                const int e = (i * 64 + lane) * kRowVec;  // element of the [16][128] block
                const int64_t src = (int64_t)min(t0 + e / kD, T - 1) * kD + e % kD;
                dma16(kg + src, s + L::oK + i * 1024);
                dma16(qg + src, s + L::oQ + i * 1024);
            }
#pragma unroll
            for (int i = 0; i < kGInstr; ++i) {
                const int e = (i * 64 + lane) * 4;
                dma16(gg + (int64_t)min(t0 + e / kD, T - 1) * kD + e % kD, s + L::oG + i * 1024);
            }
            {  // v: 16 columns of each token, 16 / kRowVec lanes per token
                constexpr int lpt = 16 / kRowVec;
                const int t = min(t0 + min(lane / lpt, kBlock - 1), T - 1);
                dma16(vg + (int64_t)t * kD + (lane % lpt) * kRowVec, s + L::oV);
            }
            dma4(bg + min(t0 + min(lane, kBlock - 1), T - 1), s + L::oB);
        };
        for (int c = 0; c < min(nb, 3); ++c) issue(c);
        if (nb >= 3)
            wait_vmcnt<kPerBlock>();  // blocks 0 and 1 have landed
        else
            wait_vmcnt<0>();
        lds_barrier();
        lds_barrier();
        for (int c = 0; c < nb; ++c) {
            // slot (c + 3) % 4 held block c - 1: run in the interval before the last barrier and
            // its operands formed in the one before that
            if (c + 3 < nb) {
                issue(c + 3);
                wait_vmcnt<kPerBlock>();  // block c + 2 has landed
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
        }
        wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup
        return;
    }

    // -------------------------------------------------------------------- compute waves
    // lane: row lrow of the workgroup, columns col .. col + 3 and col + 64 .. col + 67
    const int ci = lane % kLPR;
    const int col = ci * 4;
    const int lrow = wave * (64 / kLPR) + lane / kLPR;
    const int row = rb * kRowsPerWG + lrow;
    const int64_t si = ((int64_t)pair * kD + row) * kD + col;
    f32x4 S0 = f32x4{0.f, 0.f, 0.f, 0.f}, S1 = S0;
    if (p.init_state) {
        S0 = load_state4(p.init_state, si, p.init_f16, p.state_bf16);
        S1 = load_state4(p.init_state, si + 64, p.init_f16, p.state_bf16);
    }
    const int64_t obase = (int64_t)pair * p.Ts * kD + row;

    // operands of block cb (ring slot cb % 4) into buffer cb & 1: the 256 compute lanes take
    // token pu = (64 wave + lane) / 16, channels col .. col + 3 and col + 64 .. col + 67
    const int pu = (wave * 64 + lane) / kLPR;
    // in two parts, so that the forming of block c + 1 can sit between the token steps of block c:
    // the LDS reads, then the exponentials, k . q and the writes
    struct FormIn {
        f32x4 k[2], q[2], g[2];
        float beta;
    };
    auto form_load = [&](int cb) {
        const unsigned char *s = smem + (cb % kSlots) * L::kSlotBytes;
        FormIn in;
        in.beta = *reinterpret_cast<const float *>(s + L::oB + pu * 4);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int pj = col + 64 * hh;
            in.k[hh] = lds4<E>(s + L::oK + (pu * kD + pj) * ES);
            in.q[hh] = lds4<E>(s + L::oQ + (pu * kD + pj) * ES);
            in.g[hh] = *reinterpret_cast<const f32x4 *>(s + L::oG + (pu * kD + pj) * 4);
        }
        return in;
    };
    auto form_store = [&](int cb, const FormIn &in) {
        unsigned char *ob = smem + L::kRing + (cb & 1) * L::kOpBytes;
        const bool live = cb * kBlock + pu < T;
        float kq = 0.0f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int pj = col + 64 * hh;
            f32x4 al;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                al[e] = live ? __expf(in.g[hh][e]) : 1.0f;
                kq += in.k[hh][e] * in.q[hh][e];
            }
            const int off = (pu * kD + pj) * 4;
            *reinterpret_cast<f32x4 *>(ob + L::pAL + off) = al;
            *reinterpret_cast<f32x4 *>(ob + L::pKF + off) = in.k[hh];
            *reinterpret_cast<f32x4 *>(ob + L::pQF + off) = in.q[hh];
        }
        kq = group_sum<kLPR>(kq);
        if (ci == 0) *reinterpret_cast<f32x2 *>(ob + L::pBK + pu * 8) = f32x2{live ? in.beta : 0.0f, kq};
    };

    lds_barrier();  // blocks 0 and 1 have landed
    if (nb > 0) form_store(0, form_load(0));
    lds_barrier();
    for (int c = 0; c < nb; ++c) {
        // the forming of block c + 1 runs inside the token steps of block c, branch-free: past
        // the last block it reads a ring slot no load is still writing and fills the buffer that
        // no token step reads any more
        const FormIn fin = form_load(c + 1);
        const unsigned char *s = smem + (c % kSlots) * L::kSlotBytes;
        const unsigned char *ob = smem + L::kRing + (c & 1) * L::kOpBytes;
        float ov = 0.0f;  // o of token c * 16 + ci, row lrow
        auto load_ops = [&](int u) {
            TokenOps x;
            const int off0 = (u * kD + col) * 4, off1 = off0 + 64 * 4;
            x.al0 = *reinterpret_cast<const f32x4 *>(ob + L::pAL + off0);
            x.al1 = *reinterpret_cast<const f32x4 *>(ob + L::pAL + off1);
            x.k0 = *reinterpret_cast<const f32x4 *>(ob + L::pKF + off0);
            x.k1 = *reinterpret_cast<const f32x4 *>(ob + L::pKF + off1);
            x.q0 = *reinterpret_cast<const f32x4 *>(ob + L::pQF + off0);
            x.q1 = *reinterpret_cast<const f32x4 *>(ob + L::pQF + off1);
            x.bk = *reinterpret_cast<const f32x2 *>(ob + L::pBK + u * 8);
            x.v = lds1<E>(s + L::oV + (u * 16 + lrow) * ES);
            return x;
        };
        // the operands of token u + 2 are read while token u runs: the state chain never waits on
        // an LDS round trip
        TokenOps cur = load_ops(0), nx1 = load_ops(1);
#pragma unroll
        for (int u = 0; u < kBlock; ++u) {
            TokenOps nx2;
            if (u + 2 < kBlock) nx2 = load_ops(u + 2);
            // keep those reads ahead of this token's arithmetic (the scheduler would otherwise sink
            // them next to their first use, and each token would wait on a full LDS round trip)
            __builtin_amdgcn_sched_barrier(0);
            if (u == 2) form_store(c + 1, fin);
            float r0 = 0.0f, r1 = 0.0f, p0 = 0.0f, p1 = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S0[e] *= cur.al0[e];  // D = S diag(alpha)
                S1[e] *= cur.al1[e];
                r0 += S0[e] * cur.k0[e];
                r1 += S1[e] * cur.k1[e];
                p0 += S0[e] * cur.q0[e];
                p1 += S1[e] * cur.q1[e];
            }
            const float r = group_sum<kLPR>(r0 + r1);
            const float pq = group_sum<kLPR>(p0 + p1);
            const float delta = cur.bk[0] * (cur.v - r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S0[e] += delta * cur.k0[e];
                S1[e] += delta * cur.k1[e];
            }
            if (ci == u) ov = p.scale * (pq + delta * cur.bk[1]);
            cur = nx1;
            if (u + 2 < kBlock) nx1 = nx2;
        }
        const int t = c * kBlock + ci;
        if (t < T) {
            if (p.o_f16)
                static_cast<_Float16 *>(p.o)[obase + (int64_t)t * kD] = f16_out(ov);
            else
                static_cast<float *>(p.o)[obase + (int64_t)t * kD] = ov;
        }
        lds_barrier();
    }
    if (p.final_state) {
        store_state4(p.final_state, si, S0, p.final_f16, p.state_bf16);
        store_state4(p.final_state, si + 64, S1, p.final_f16, p.state_bf16);
    }
}

template <typename E>
hipError_t launch_e(const PrefillParams &p, int64_t blocks, hipStream_t stream) {
    constexpr int bytes = KdaSmem<E>::kBytes;
    static bool attr_set = false;  // the attribute is a property of the function: set once
    if (!attr_set) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_kda_prefill_kernel<E>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    hipLaunchKernelGGL((gdn_kda_prefill_kernel<E>), dim3((unsigned)blocks), dim3(kThreads), bytes, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_prefill(const PrefillParams &p, bool bf16, hipStream_t stream) {
    if (p.D != kD) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)p.B * p.Hv * (kD / kRowsPerWG);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    return bf16 ? launch_e<uint16_t>(p, blocks, stream) : launch_e<float>(p, blocks, stream);
}

}  // namespace gdn
