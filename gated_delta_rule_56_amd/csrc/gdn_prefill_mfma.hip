// Fused chunked (WY-form) gated delta rule prefill for bfloat16 q/k/v on
// gfx950 matrix cores (fp16 MFMA operands, fp32 accumulation), with the fp32
// state resident in registers for the whole sequence.
//
// Per (b, h) and chunk of C tokens with start state S (dv x dk), local t:
//   G_t = sum_{s<=t} g_s,  gamma_t = exp(G_t),  Gamma_ts = exp(G_t - G_s), s <= t
//   A   = strict_lower(diag(beta) (K K^T o Gamma))       -> T = (I + A)^{-1}
//   R   = diag(beta) (V - diag(gamma) K S^T),  U = T R
//   O   = diag(gamma) (scale Q) S^T + lower_incl(scale Q K^T o Gamma) U
//   S  <- gamma_C S + (diag(exp(G_C - G)) U)^T K
// This is the recurrence S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) +
// beta_t v_t k_t^T, o_t = S_t (scale q_t) regrouped per chunk: with
// u_t = beta_t (v_t - exp(g_t) S_{t-1} k_t), S_t = gamma_t S + sum_s Gamma_ts u_s k_s^T,
// and the u_t solve the unit-lower system (I + A) U = R. The triangular inverse
// is the forward substitution of the tinygrad helper inverse_unit_lower
// (compare page "27b 935/47", llm/kernels/generic.py: inverse of I - x for
// strictly lower x; here x = -A), done blockwise: 16x16 diagonal blocks by
// substitution, off-diagonal blocks by MFMA recursive doubling. Steps past
// the sequence end are zero rows with g = beta = 0 and add nothing (the padded
// no-op rule, commit log of page "mergable fast RDNA3 Qwen 3.6").
//
// Mapping: one workgroup of 4 waves per (b, h, block of 16 state rows); the 8
// row blocks of a head (and the heads sharing a key head) are placed on the
// same XCD so that their q/k tiles are shared through that XCD's L2. Wave w
// owns state columns [32w, 32w + 32) of the 16 rows as fp32 MFMA accumulators.
// The dv-independent work of a chunk (K K^T, Q K^T, the solve) is recomputed
// by each row block; the state-dependent chain (K S^T, Q S^T, U, O, the
// update) is split across the waves.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;       // head dimension (dk = dv)
constexpr int kRows = 16;     // state rows per workgroup
constexpr int kThreads = 256;

template <int C>
struct MfmaSmem {
    static constexpr int NT = C / 16;
    static constexpr int QP = kD + 8;   // f16 pitch of the q/k tiles
    static constexpr int CP = C + 8;    // f16 pitch of the C x C matrices
    // byte offsets
    static constexpr size_t kQ = 0;
    static constexpr size_t kK = kQ + 2 * C * QP;
    static constexpr size_t kV = kK + 2 * C * QP;             // f32 [C][16]
    static constexpr size_t kG = kV + 4 * C * kRows;          // f32 [64] x 4: G, gamma, exp(G_C-G), beta
    static constexpr size_t kAd = kG + 4 * 4 * 64;            // f32 [NT][16][17]
    static constexpr size_t kXp = kAd + 4 * NT * 16 * 17;     // f32 [4][NT][64][4]
    static constexpr size_t kYp = kXp + 4 * 4 * NT * 256;
    static constexpr size_t kAh = kYp + 4 * 4 * NT * 256;     // f16 [C][CP]
    static constexpr size_t kAqk = kAh + 2 * C * CP;
    static constexpr size_t kTm = kAqk + 2 * C * CP;
    static constexpr size_t kRt = kTm + 2 * C * CP;           // f16 [16][CP]
    static constexpr size_t kBytes = kRt + 2 * kRows * CP;
    static_assert(kXp % 16 == 0 && kYp % 16 == 0 && kAh % 16 == 0, "alignment");
};

__device__ __forceinline__ f16x4 ld4(const _Float16 *p) { return *reinterpret_cast<const f16x4 *>(p); }
__device__ __forceinline__ f16x8 ld8(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

template <int C>
__global__ __launch_bounds__(kThreads) void gdn_prefill_mfma_kernel(PrefillParams p) {
    using L = MfmaSmem<C>;
    constexpr int NT = L::NT, QP = L::QP, CP = L::CP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *Qs = reinterpret_cast<_Float16 *>(smem + L::kQ);
    _Float16 *Ks = reinterpret_cast<_Float16 *>(smem + L::kK);
    float *Vs = reinterpret_cast<float *>(smem + L::kV);
    float *Gs = reinterpret_cast<float *>(smem + L::kG);
    float *Gam = Gs + 64;
    float *Eg = Gam + 64;
    float *Bs = Eg + 64;
    float *Ad = reinterpret_cast<float *>(smem + L::kAd);
    float *Xp = reinterpret_cast<float *>(smem + L::kXp);
    float *Yp = reinterpret_cast<float *>(smem + L::kYp);
    _Float16 *Ah = reinterpret_cast<_Float16 *>(smem + L::kAh);
    _Float16 *Aqk = reinterpret_cast<_Float16 *>(smem + L::kAqk);
    _Float16 *Tm = reinterpret_cast<_Float16 *>(smem + L::kTm);
    _Float16 *Rt = reinterpret_cast<_Float16 *>(smem + L::kRt);

    // ---- workgroup -> (b, key head, value head, row block); XCD-aware order
    const int nb = gridDim.x;
    int lin = blockIdx.x;
    if ((nb & 7) == 0) lin = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
    const int dvb = lin & 7;
    int rest = lin >> 3;
    const int ratio = p.Hv / p.Hk;
    const int jj = rest % ratio;
    rest /= ratio;
    const int kh = rest % p.Hk;
    const int b = rest / p.Hk;
    const int h = p.head_map == 0 ? kh + jj * p.Hk : kh * ratio + jj;
    const int pair = b * p.Hv + h;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, q4 = lane >> 4;
    const int T = p.T;
    const uint16_t *qg = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hk + kh) * T * kD;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hk + kh) * T * kD;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + (int64_t)pair * T * kD;
    const float *gg = p.g + (int64_t)pair * T;
    const float *bg = p.beta + (int64_t)pair * T;
    const int64_t o0 = (int64_t)pair * T * kD;

    // ---- state fragment: S[jl][r] = state[16 dvb + li][32 w + 16 jl + 4 q4 + r]
    const int64_t srow = ((int64_t)pair * kD + kRows * dvb + li) * kD + 32 * w + 4 * q4;
    f32x4 S[2];
#pragma unroll
    for (int jl = 0; jl < 2; ++jl)
        S[jl] = p.init_state ? load_state4(p.init_state, srow + 16 * jl, p.init_f16, p.state_bf16) : f32x4{0.f, 0.f, 0.f, 0.f};

    // upper-triangular tiles of A, A_qk and T stay zero for the whole sequence
    for (int e = tid; e < 3 * C * CP; e += kThreads) Ah[e] = (_Float16)0.0f;  // Ah, Aqk, Tm are contiguous

    const int NC = (T + C - 1) / C;
    for (int c = 0; c < NC; ++c) {
        const int t0 = c * C;
        const int n = min(C, T - t0);
        __syncthreads();

        // ---- a1: load the chunk (bf16 -> fp16), zero rows past the end
        for (int idx = tid; idx < C * 16; idx += kThreads) {
            const int row = idx >> 4, c8 = (idx & 15) * 8;
            u16x8 qb = {0, 0, 0, 0, 0, 0, 0, 0}, kb = {0, 0, 0, 0, 0, 0, 0, 0};
            if (row < n) {
                qb = *reinterpret_cast<const u16x8 *>(qg + (int64_t)(t0 + row) * kD + c8);
                kb = *reinterpret_cast<const u16x8 *>(kg + (int64_t)(t0 + row) * kD + c8);
            }
            f16x8 qh, khv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qh[e] = (_Float16)bf16_bits_to_f32(qb[e]);
                khv[e] = (_Float16)bf16_bits_to_f32(kb[e]);
            }
            *reinterpret_cast<f16x8 *>(Qs + row * QP + c8) = qh;
            *reinterpret_cast<f16x8 *>(Ks + row * QP + c8) = khv;
        }
        if (tid < 2 * C) {
            const int row = tid >> 1, half = (tid & 1) * 8;
            u16x8 vb = {0, 0, 0, 0, 0, 0, 0, 0};
            if (row < n) vb = *reinterpret_cast<const u16x8 *>(vg + (int64_t)(t0 + row) * kD + kRows * dvb + half);
#pragma unroll
            for (int e = 0; e < 8; ++e) Vs[row * kRows + half + e] = bf16_bits_to_f32(vb[e]);
        }
        // ---- a2: gate prefix (wave 0), beta (wave 3)
        if (w == 0) {
            float x = (lane < n) ? gg[t0 + lane] : 0.0f;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float y = __shfl_up(x, m, 64);
                if (lane >= m) x += y;
            }
            const float gc = __shfl(x, C - 1, 64);
            if (lane < C) {
                Gs[lane] = x;
                Gam[lane] = __expf(x);
                Eg[lane] = __expf(gc - x);
            }
        } else if (w == 3 && lane < C) {
            Bs[lane] = (lane < n) ? bg[t0 + lane] : 0.0f;
        }
        __syncthreads();

        // ---- a3/a4: lower tiles of K K^T (-> A) and Q K^T (-> A_qk)
        constexpr int NL = NT * (NT + 1) / 2;
        for (int job = w; job < 2 * NL; job += 4) {
            const bool isq = job >= NL;
            int jt = isq ? job - NL : job;
            int mt = 0;
            while (jt > mt) { jt -= mt + 1; ++mt; }
            const int nt = jt;
            const _Float16 *arow = (isq ? Qs : Ks) + (16 * mt + li) * QP + 8 * q4;
            const _Float16 *brow = Ks + (16 * nt + li) * QP + 8 * q4;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < kD / 32; ++kb) acc = mfma16x16x32(ld8(arow + 32 * kb), ld8(brow + 32 * kb), acc);
            const int s = 16 * nt + li;
            const float gs = Gs[s];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * mt + 4 * q4 + r;
                const float gate = __expf(Gs[t] - gs);
                if (!isq) {
                    const float a = (s < t) ? Bs[t] * gate * acc[r] : 0.0f;
                    Ah[t * CP + s] = (_Float16)a;
                    if (mt == nt) Ad[(mt * 16 + (t & 15)) * 17 + (s & 15)] = a;
                } else {
                    Aqk[t * CP + s] = (_Float16)((s <= t) ? p.scale * gate * acc[r] : 0.0f);
                }
            }
        }
        __syncthreads();

        // ---- a5: T = (I + A)^{-1}. Diagonal 16x16 blocks by forward substitution
        // (every lane computes column li of block w; lanes of one column agree).
        if (w < NT) {
            float x[16];
            const float *ab = Ad + w * 16 * 17;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == li) ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) acc -= ab[r * 17 + s2] * x[s2];
                x[r] = acc;
            }
            if (q4 == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Tm[(16 * w + r) * CP + 16 * w + li] = (_Float16)x[r];
            }
        }
        if constexpr (NT >= 2) {
            __syncthreads();
            // level 1: T_{u,l} = -T_{u,u} A_{u,l} T_{l,l} for (l, u) = (0, 1), (2, 3)
            if (w < NT / 2) {
                const int lo = 2 * w, up = 2 * w + 1;
                f16x4 bt;
#pragma unroll
                for (int e = 0; e < 4; ++e) bt[e] = Tm[(16 * lo + 4 * q4 + e) * CP + 16 * lo + li];
                f32x4 pm = mfma16x16x16(ld4(Ah + (16 * up + li) * CP + 16 * lo + 4 * q4), bt,
                                        f32x4{0.f, 0.f, 0.f, 0.f});
                const f16x4 pb = to_f16x4(-pm);
                const f32x4 out = mfma16x16x16(ld4(Tm + (16 * up + li) * CP + 16 * up + 4 * q4), pb,
                                               f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int r = 0; r < 4; ++r) Tm[(16 * up + 4 * q4 + r) * CP + 16 * lo + li] = (_Float16)out[r];
            }
        }
        if constexpr (NT == 4) {
            __syncthreads();
            // level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32],
            // wave j computes 16-column block j
            if (w < 2) {
                const int j = w;
                f16x4 t0j, t1j;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t0j[e] = Tm[(4 * q4 + e) * CP + 16 * j + li];
                    t1j[e] = Tm[(16 + 4 * q4 + e) * CP + 16 * j + li];
                }
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                f32x4 p0 = mfma16x16x16(ld4(Ah + (32 + li) * CP + 16 + 4 * q4), t1j, z);
                f32x4 p1 = mfma16x16x16(ld4(Ah + (48 + li) * CP + 16 + 4 * q4), t1j, z);
                if (j == 0) {
                    p0 = mfma16x16x16(ld4(Ah + (32 + li) * CP + 4 * q4), t0j, p0);
                    p1 = mfma16x16x16(ld4(Ah + (48 + li) * CP + 4 * q4), t0j, p1);
                }
                const f16x4 b0 = to_f16x4(-p0), b1 = to_f16x4(-p1);
                const f32x4 o0 = mfma16x16x16(ld4(Tm + (32 + li) * CP + 32 + 4 * q4), b0, z);
                f32x4 o1 = mfma16x16x16(ld4(Tm + (48 + li) * CP + 32 + 4 * q4), b0, z);
                o1 = mfma16x16x16(ld4(Tm + (48 + li) * CP + 48 + 4 * q4), b1, o1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Tm[(32 + 4 * q4 + r) * CP + 16 * j + li] = (_Float16)o0[r];
                    Tm[(48 + 4 * q4 + r) * CP + 16 * j + li] = (_Float16)o1[r];
                }
            }
        }

        // ---- a7 (first half): partial K S^T and Q S^T over this wave's 32 state columns
        {
            f16x8 sb;
#pragma unroll
            for (int e = 0; e < 8; ++e) sb[e] = (_Float16)S[e >> 2][e & 3];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                const _Float16 *kr = Ks + (16 * mt + li) * QP + 32 * w + 4 * q4;
                const _Float16 *qr = Qs + (16 * mt + li) * QP + 32 * w + 4 * q4;
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 x = mfma16x16x32(cat(ld4(kr), ld4(kr + 16)), sb, z);
                const f32x4 y = mfma16x16x32(cat(ld4(qr), ld4(qr + 16)), sb, z);
                *reinterpret_cast<f32x4 *>(Xp + ((w * NT + mt) * 64 + lane) * 4) = x;
                *reinterpret_cast<f32x4 *>(Yp + ((w * NT + mt) * 64 + lane) * 4) = y;
            }
        }
        __syncthreads();

        // ---- reduce the partials of token tile w; R = diag(beta) (V - diag(gamma) K S^T)
        f32x4 yw = {0.f, 0.f, 0.f, 0.f};
        if (w < NT) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                x += *reinterpret_cast<const f32x4 *>(Xp + ((w2 * NT + w) * 64 + lane) * 4);
                yw += *reinterpret_cast<const f32x4 *>(Yp + ((w2 * NT + w) * 64 + lane) * 4);
            }
            f16x4 rr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * q4 + r;
                rr[r] = (_Float16)(Bs[t] * (Vs[t * kRows + li] - Gam[t] * x[r]));
            }
            *reinterpret_cast<f16x4 *>(Rt + li * CP + 16 * w + 4 * q4) = rr;
        }
        __syncthreads();

        // ---- a6/a7: U = T R (all token tiles, in every wave)
        f32x4 U[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            U[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (C >= 32) {
#pragma unroll
                for (int kb = 0; kb <= mt / 2; ++kb) {
                    const _Float16 *tr = Tm + (16 * mt + li) * CP + 32 * kb + 4 * q4;
                    const _Float16 *rr = Rt + li * CP + 32 * kb + 4 * q4;
                    U[mt] = mfma16x16x32(cat(ld4(tr), ld4(tr + 16)), cat(ld4(rr), ld4(rr + 16)), U[mt]);
                }
            } else {
                U[mt] = mfma16x16x16(ld4(Tm + li * CP + 4 * q4), ld4(Rt + li * CP + 4 * q4), U[mt]);
            }
        }

        // ---- a8: O = diag(gamma) scale (Q S^T) + A_qk U for token tile w
        if (w < NT) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (C >= 32) {
#pragma unroll
                for (int kb = 0; kb < NT / 2; ++kb) {
                    if (kb <= w / 2) {
                        const _Float16 *ar = Aqk + (16 * w + li) * CP + 32 * kb + 4 * q4;
                        acc = mfma16x16x32(cat(ld4(ar), ld4(ar + 16)),
                                           cat(to_f16x4(U[2 * kb]), to_f16x4(U[2 * kb + 1])), acc);
                    }
                }
            } else {
                acc = mfma16x16x16(ld4(Aqk + li * CP + 4 * q4), to_f16x4(U[0]), acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * q4 + r;
                if (t < n) {
                    const float ov = Gam[t] * p.scale * yw[r] + acc[r];
                    const int64_t oi = o0 + (int64_t)(t0 + t) * kD + kRows * dvb + li;
                    if (p.o_f16)
                        static_cast<_Float16 *>(p.o)[oi] = f16_out(ov);
                    else
                        static_cast<float *>(p.o)[oi] = ov;
                }
            }
        }

        // ---- a9: S <- gamma_C S + (diag(exp(G_C - G)) U)^T K on this wave's columns
        {
            const float gC = Gam[C - 1];
#pragma unroll
            for (int jl = 0; jl < 2; ++jl) S[jl] *= gC;
            if constexpr (C >= 32) {
#pragma unroll
                for (int kb = 0; kb < NT / 2; ++kb) {
                    f16x8 ub;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int mtp = 2 * kb + (e >> 2), r = e & 3;
                        ub[e] = (_Float16)(Eg[16 * mtp + 4 * q4 + r] * U[mtp][r]);
                    }
#pragma unroll
                    for (int jl = 0; jl < 2; ++jl) {
                        const int j = 32 * w + 16 * jl + li;
                        f16x8 ka;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            ka[e] = Ks[(32 * kb + 16 * (e >> 2) + 4 * q4 + (e & 3)) * QP + j];
                        S[jl] = mfma16x16x32(ka, ub, S[jl]);
                    }
                }
            } else {
                f16x4 ub;
#pragma unroll
                for (int e = 0; e < 4; ++e) ub[e] = (_Float16)(Eg[4 * q4 + e] * U[0][e]);
#pragma unroll
                for (int jl = 0; jl < 2; ++jl) {
                    const int j = 32 * w + 16 * jl + li;
                    f16x4 ka;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ka[e] = Ks[(4 * q4 + e) * QP + j];
                    S[jl] = mfma16x16x16(ka, ub, S[jl]);
                }
            }
        }
    }

    if (p.final_state) {
#pragma unroll
        for (int jl = 0; jl < 2; ++jl) store_state4(p.final_state, srow + 16 * jl, S[jl], p.final_f16, p.state_bf16);
    }
}

template <int C>
hipError_t launch_c(const PrefillParams &p, hipStream_t stream) {
    const size_t bytes = MfmaSmem<C>::kBytes;
    static bool attr_set = false;  // the attribute is a property of the function: set once
    if (!attr_set) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_prefill_mfma_kernel<C>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    dim3 grid((unsigned)(p.B * p.Hv * (kD / kRows))), block(kThreads);
    hipLaunchKernelGGL((gdn_prefill_mfma_kernel<C>), grid, block, bytes, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams &p, int chunk, hipStream_t stream) {
    if (p.D != kD) return hipErrorInvalidValue;
    switch (chunk) {
        case 16: return launch_c<16>(p, stream);
        case 32: return launch_c<32>(p, stream);
        case 64: return launch_c<64>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
