// Chunked (WY-form) gated delta rule prefill computed in fp32 on the vector ALUs,
// for float32 q/k/v (the precise path, d <= 128) and for bfloat16 q/k/v with head
// dimensions below 128 (widened exactly to fp32 on load); bfloat16 at d = 128 runs
// on the MFMA kernels.
//
// Per (b, h) and chunk of C tokens with start state S (dv x dk), local t = 0..C-1:
//   G_t = sum_{s<=t} g_s,  gamma_t = exp(G_t),  Gamma_ts = exp(G_t - G_s) (s <= t)
//   A   = strict_lower(diag(beta) (K K^T o Gamma)),  T = (I + A)^{-1}
//   U   = T diag(beta) (V - diag(gamma) K S^T)
//   O   = diag(gamma) (scale Q) S^T + lower_incl(scale Q K^T o Gamma) U
//   S  <- gamma_C S + (diag(exp(G_C - G)) U)^T K
// Gates are always formed from differences of G, never from exp(-G) alone.
// Steps past the end of the sequence are loaded as zeros with g = beta = 0, so
// they contribute nothing (the padded-step no-op of the tinygrad symbolic
// prefill, commit log of page "mergable fast RDNA3 Qwen 3.6").
//
// Mapping: one workgroup per (b, h, block of 16 state rows); the state block
// lives in LDS for the whole sequence and is written once at the end.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kF32Threads = 256;
constexpr int kRows = 16;  // state rows (value dimension) per workgroup

template <int D, int C>
struct F32Smem {
    static constexpr int QP = D + 1;  // padded pitches
    static constexpr int CP = C + 1;
    static constexpr int RP = kRows + 1;
    static constexpr int kFloats = 2 * C * QP + C * kRows + 4 * C + 3 * C * CP + 3 * C * RP + kRows * QP;
    static constexpr size_t kBytes = sizeof(float) * kFloats;
};

// element i of q, k or v: float32, or bfloat16 bits widened exactly
template <bool BF>
__device__ __forceinline__ float ld_in(const void *base, int64_t i) {
    if constexpr (BF) return bf16_bits_to_f32(static_cast<const uint16_t *>(base)[i]);
    return static_cast<const float *>(base)[i];
}

template <int D, int C, bool BF>
__global__ __launch_bounds__(kF32Threads) void gdn_prefill_f32_kernel(PrefillParams p) {
    using L = F32Smem<D, C>;
    extern __shared__ float smem[];
    float *Qs = smem;                       // [C][QP]
    float *Ks = Qs + C * L::QP;             // [C][QP]
    float *Vs = Ks + C * L::QP;             // [C][16]
    float *Gs = Vs + C * kRows;             // [C] cumulative log-decay
    float *Gam = Gs + C;                    // [C] exp(G_t)
    float *Eg = Gam + C;                    // [C] exp(G_C - G_t)
    float *Bs = Eg + C;                     // [C] beta
    float *A = Bs + C;                      // [C][CP]
    float *Aqk = A + C * L::CP;             // [C][CP]
    float *Tm = Aqk + C * L::CP;            // [C][CP]
    float *X = Tm + C * L::CP;              // [C][RP]  K S^T, then R
    float *Y = X + C * L::RP;               // [C][RP]  Q S^T
    float *U = Y + C * L::RP;               // [C][RP]
    float *S = U + C * L::RP;               // [16][QP] state rows of this block

    constexpr int NBLK = D / kRows;
    const int tid = threadIdx.x;
    const int blk = blockIdx.x % NBLK;
    const int pair = blockIdx.x / NBLK;
    const int b = pair / p.Hv, h = pair % p.Hv;
    const int kh = key_head(h, p.Hk, p.Hv, p.head_map);
    const int T = p.T;
    const int64_t qk0 = ((int64_t)b * p.Hk + kh) * T * D;
    const int64_t v0 = ((int64_t)b * p.Hv + h) * T * D;
    const float *gg = p.g + ((int64_t)b * p.Hv + h) * T;
    const float *bg = p.beta + ((int64_t)b * p.Hv + h) * T;
    const int64_t o0 = ((int64_t)b * p.Hv + h) * T * D;
    const int64_t sbase = ((int64_t)pair * D + blk * kRows) * D;

    for (int e = tid; e < kRows * D; e += kF32Threads) {
        const int i = e / D, j = e % D;
        const int64_t si = sbase + (int64_t)i * D + j;
        S[i * L::QP + j] = !p.init_state               ? 0.0f
                           : p.init_f16 && p.state_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t *>(p.init_state)[si])
                           : p.init_f16                 ? (float)static_cast<const _Float16 *>(p.init_state)[si]
                                                        : static_cast<const float *>(p.init_state)[si];
    }

    for (int t0 = 0; t0 < T; t0 += C) {
        const int n = min(C, T - t0);
        __syncthreads();
        for (int e = tid; e < C * D; e += kF32Threads) {
            const int t = e / D, j = e % D;
            const bool in = t < n;
            Qs[t * L::QP + j] = in ? ld_in<BF>(p.q, qk0 + (int64_t)(t0 + t) * D + j) : 0.0f;
            Ks[t * L::QP + j] = in ? ld_in<BF>(p.k, qk0 + (int64_t)(t0 + t) * D + j) : 0.0f;
        }
        for (int e = tid; e < C * kRows; e += kF32Threads) {
            const int t = e / kRows, i = e % kRows;
            Vs[e] = t < n ? ld_in<BF>(p.v, v0 + (int64_t)(t0 + t) * D + blk * kRows + i) : 0.0f;
        }
        if (tid < 64) {
            // inclusive prefix sum of g over the chunk (lanes >= n hold g = 0)
            float x = (tid < n) ? gg[t0 + tid] : 0.0f;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float y = __shfl_up(x, m, 64);
                if (tid >= m) x += y;
            }
            const float gc = __shfl(x, C - 1, 64);
            if (tid < C) {
                Gs[tid] = x;
                Gam[tid] = __expf(x);
                Eg[tid] = __expf(gc - x);
                Bs[tid] = (tid < n) ? bg[t0 + tid] : 0.0f;
            }
        }
        __syncthreads();

        // A (strict lower, gated by beta) and A_qk (inclusive lower, scaled)
        for (int e = tid; e < C * C; e += kF32Threads) {
            const int t = e / C, s = e % C;
            float a = 0.0f, aq = 0.0f;
            if (s <= t) {
                float kk = 0.0f, qk = 0.0f;
                for (int j = 0; j < D; ++j) {
                    kk += Ks[t * L::QP + j] * Ks[s * L::QP + j];
                    qk += Qs[t * L::QP + j] * Ks[s * L::QP + j];
                }
                const float gate = __expf(Gs[t] - Gs[s]);
                if (s < t) a = Bs[t] * gate * kk;
                aq = p.scale * gate * qk;
            }
            A[t * L::CP + s] = a;
            Aqk[t * L::CP + s] = aq;
        }
        // X = K S^T, Y = Q S^T for this block's rows
        for (int e = tid; e < C * kRows; e += kF32Threads) {
            const int t = e / kRows, i = e % kRows;
            float x = 0.0f, y = 0.0f;
            for (int j = 0; j < D; ++j) {
                x += Ks[t * L::QP + j] * S[i * L::QP + j];
                y += Qs[t * L::QP + j] * S[i * L::QP + j];
            }
            X[t * L::RP + i] = x;
            Y[t * L::RP + i] = y;
        }
        __syncthreads();

        // T = (I + A)^{-1} by forward substitution; lane c owns column c in registers
        if (tid < C) {
            const int c = tid;
            float col[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float acc = (r == c) ? 1.0f : 0.0f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= A[r * L::CP + s] * col[s];
                col[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < C; ++r) Tm[r * L::CP + c] = col[r];
        }
        // R = diag(beta) (V - diag(gamma) X), in place in X
        for (int e = tid; e < C * kRows; e += kF32Threads) {
            const int t = e / kRows, i = e % kRows;
            X[t * L::RP + i] = Bs[t] * (Vs[e] - Gam[t] * X[t * L::RP + i]);
        }
        __syncthreads();

        // U = T R
        for (int e = tid; e < C * kRows; e += kF32Threads) {
            const int t = e / kRows, i = e % kRows;
            float u = 0.0f;
            for (int s = 0; s <= t; ++s) u += Tm[t * L::CP + s] * X[s * L::RP + i];
            U[t * L::RP + i] = u;
        }
        __syncthreads();

        // O = diag(gamma) scale Y + A_qk U
        for (int e = tid; e < C * kRows; e += kF32Threads) {
            const int t = e / kRows, i = e % kRows;
            if (t < n) {
                float acc = Gam[t] * p.scale * Y[t * L::RP + i];
                for (int s = 0; s <= t; ++s) acc += Aqk[t * L::CP + s] * U[s * L::RP + i];
                const int64_t oi = o0 + (int64_t)(t0 + t) * D + blk * kRows + i;
                if (p.o_f16)
                    static_cast<_Float16 *>(p.o)[oi] = f16_out(acc);
                else
                    static_cast<float *>(p.o)[oi] = acc;
            }
        }
        // S <- gamma_C S + (diag(exp(G_C - G)) U)^T K
        const float gC = Gam[C - 1];
        for (int e = tid; e < kRows * D; e += kF32Threads) {
            const int i = e / D, j = e % D;
            float acc = 0.0f;
            for (int t = 0; t < C; ++t) acc += Eg[t] * U[t * L::RP + i] * Ks[t * L::QP + j];
            S[i * L::QP + j] = gC * S[i * L::QP + j] + acc;
        }
    }
    __syncthreads();
    if (p.final_state) {
        for (int e = tid; e < kRows * D; e += kF32Threads) {
            const int i = e / D, j = e % D;
            const int64_t si = sbase + (int64_t)i * D + j;
            if (p.final_f16 && p.state_bf16)
                static_cast<__bf16 *>(p.final_state)[si] = bf16_out(S[i * L::QP + j]);
            else if (p.final_f16)
                static_cast<_Float16 *>(p.final_state)[si] = f16_out(S[i * L::QP + j]);
            else
                static_cast<float *>(p.final_state)[si] = S[i * L::QP + j];
        }
    }
}

template <int D, int C, bool BF>
hipError_t launch_dc(const PrefillParams &p, hipStream_t stream) {
    const size_t bytes = F32Smem<D, C>::kBytes;
    static bool attr_set = false;  // a property of the function: set once
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_prefill_f32_kernel<D, C, BF>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    dim3 grid((unsigned)(p.B * p.Hv * (D / kRows))), block(kF32Threads);
    hipLaunchKernelGGL((gdn_prefill_f32_kernel<D, C, BF>), grid, block, bytes, stream, p);
    return hipGetLastError();
}

template <int D, bool BF>
hipError_t launch_d(const PrefillParams &p, int chunk, hipStream_t stream) {
    switch (chunk) {
        case 16: return launch_dc<D, 16, BF>(p, stream);
        case 32: return launch_dc<D, 32, BF>(p, stream);
        case 64: return launch_dc<D, 64, BF>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams &p, int chunk, bool bf16, hipStream_t stream) {
    if (bf16) {
        switch (p.D) {
            case 16: return launch_d<16, true>(p, chunk, stream);
            case 32: return launch_d<32, true>(p, chunk, stream);
            case 64: return launch_d<64, true>(p, chunk, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.D) {
        case 16: return launch_d<16, false>(p, chunk, stream);
        case 32: return launch_d<32, false>(p, chunk, stream);
        case 64: return launch_d<64, false>(p, chunk, stream);
        case 128: return launch_d<128, false>(p, chunk, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
