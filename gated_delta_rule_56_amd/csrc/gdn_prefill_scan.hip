// Sequential half of the bf16 prefill: the pass over the chunks of one
// (b, h, block of 16 state rows), with the fp32 state resident in registers.
//
// Per chunk c with start state S (rows i of this block), T and A_qk from the
// chunk kernel (gdn_prefill_chunk.hip):
//   X = K S^T,  R = diag(beta) (V - diag(gamma) X),  U = T R
//   S <- gamma_C S + (diag(exp(G_C - G)) U)^T K
//   O = diag(gamma) (scale Q S^T) + A_qk U
// (the chunked WY form of S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) +
// beta_t v_t k_t^T, o_t = S_t scale q_t, with U solving (I + A) U = R).
//
// Roles inside the workgroup (4 waves, one per SIMD):
//   wave 0 ("state") owns the 16 x 128 fp32 state block as MFMA accumulators
//   and runs only the chain S -> X -> R -> U -> S: 38 MFMAs per 64-token
//   chunk, all operands in registers or one LDS read away.
//   waves 1-3 ("helpers") stage the next chunk (k in fragment order and
//   transposed, v transposed, gates) into the other half of a double-buffered
//   LDS area, and compute the outputs off the critical path: Q S^T of the
//   current chunk from an fp16 copy of S, and O of the previous chunk from the
//   fp16 copy of its U.
// One workgroup barrier per chunk. Matrix operands are fp16 with fp32
// accumulation; all k contractions use the fragment order of gdn_frag.h.
#include "gdn_device.h"
#include "gdn_frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRows = 16;
constexpr int kThreads = 256;
constexpr int kHelpers = 3;

template <int C>
struct ScanSmem {
    static constexpr int NT = C / 16;      // token tiles per chunk
    static constexpr int KBC = C / 32;     // 32-wide k blocks over the chunk
    static constexpr int KP = kD + 8;      // fp16 pitch of the fragment-permuted k rows
    static constexpr int TP = C + 8;       // fp16 pitch of the transposed k rows
    static constexpr int VP = C + 4;       // f32 pitch of the transposed v block
    // one stage buffer
    static constexpr size_t kKf = 0;                          // f16 [C][KP]
    static constexpr size_t kKt = kKf + 2 * C * KP;           // f16 [128][TP]
    static constexpr size_t kVt = kKt + 2 * kD * TP;          // f32 [16][VP]
    static constexpr size_t kGam = kVt + 4 * kRows * VP;      // f32 [64] gamma_t
    static constexpr size_t kBeta = kGam + 4 * 64;            // f32 [64]
    static constexpr size_t kEg = kBeta + 4 * 64;             // f32 [64] exp(G_C - G_t)
    static constexpr size_t kStage = kEg + 4 * 64;
    // exchange buffers
    static constexpr size_t kS16 = 2 * kStage;                // f16 [2][4][64][8]
    static constexpr size_t kU16 = kS16 + 2 * 2 * 4 * 64 * 8;  // f16 [2][KBC][64][8]
    static constexpr size_t kBytes = kU16 + 2 * 2 * KBC * 64 * 8;
    static_assert(kKt % 16 == 0 && kVt % 16 == 0 && kGam % 16 == 0 && kStage % 16 == 0, "alignment");
};

__device__ __forceinline__ f16x8 ld8(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

__device__ __forceinline__ f16x8 pack8(f32x4 lo, f32x4 hi) {
    return f16x8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                 (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
}

__device__ __forceinline__ f16x4 bf16x4_to_f16(u16x4 u) {
    return f16x4{(_Float16)bf16_bits_to_f32(u[0]), (_Float16)bf16_bits_to_f32(u[1]),
                 (_Float16)bf16_bits_to_f32(u[2]), (_Float16)bf16_bits_to_f32(u[3])};
}

template <int C>
__global__ __launch_bounds__(kThreads) void gdn_prefill_scan_kernel(PrefillParams p, const _Float16 *ws) {
    using L = ScanSmem<C>;
    constexpr int NT = L::NT, KBC = L::KBC, KP = L::KP, TP = L::TP, VP = L::VP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // ---- workgroup -> (b, key head, value head, row block); the row blocks and
    // value heads of one key head sit on one XCD (workgroups go round-robin over 8 XCDs)
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
    const int NC = (T + C - 1) / C;
    const uint16_t *qg = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hk + kh) * T * kD;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hk + kh) * T * kD;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + (int64_t)pair * T * kD + kRows * dvb;
    const float *gg = p.g + (int64_t)pair * T;
    const float *bg = p.beta + (int64_t)pair * T;
    const _Float16 *wsp = ws + (int64_t)pair * NC * 2 * C * C;   // [NC][2][C][C]

    _Float16 *S16 = reinterpret_cast<_Float16 *>(smem + L::kS16);  // [2][4][64][8]
    _Float16 *U16 = reinterpret_cast<_Float16 *>(smem + L::kU16);  // [2][KBC][64][8]

    if (w == 0) {
        // ================================================================ state wave
        // S[jt][r] = state[16 dvb + li][16 jt + 4 q4 + r]
        const int64_t srow = ((int64_t)pair * kD + kRows * dvb + li) * kD + 4 * q4;
        f32x4 S[8];
#pragma unroll
        for (int jt = 0; jt < 8; ++jt)
            S[jt] = p.init_state ? *reinterpret_cast<const f32x4 *>(p.init_state + srow + 16 * jt)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
        // T fragments of the current chunk: Tf[m][kb] = T[16 m + li][frag_col(kb, q4, .)]
        f16x8 Tf[NT][KBC], Tn[NT][KBC];
        auto load_T = [&](int c, f16x8 (&dst)[NT][KBC]) {
            const _Float16 *src = wsp + (int64_t)c * 2 * C * C;
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (kb <= m / 2) dst[m][kb] = ld8(src + (16 * m + li) * C + 32 * kb + 8 * q4);
        };
        auto write_S16 = [&](int buf) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                *reinterpret_cast<f16x8 *>(S16 + ((buf * 4 + kb) * 64 + lane) * 8) = pack8(S[2 * kb], S[2 * kb + 1]);
        };
        if (NC > 0) load_T(0, Tf);
        write_S16(0);
        __syncthreads();

        for (int c = 0; c < NC; ++c) {
            const unsigned char *stage = smem + (c & 1) * L::kStage;
            const _Float16 *Kf = reinterpret_cast<const _Float16 *>(stage + L::kKf);
            const _Float16 *Kt = reinterpret_cast<const _Float16 *>(stage + L::kKt);
            const float *Vt = reinterpret_cast<const float *>(stage + L::kVt);
            const float *gam = reinterpret_cast<const float *>(stage + L::kGam);
            const float *bet = reinterpret_cast<const float *>(stage + L::kBeta);
            const float *eg = reinterpret_cast<const float *>(stage + L::kEg);
            if (c + 1 < NC) load_T(c + 1, Tn);

            // operands from the stage buffer
            f16x8 ka[NT][4];
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) ka[m][kb] = ld8(Kf + (16 * m + li) * KP + 32 * kb + 8 * q4);
            f16x8 kt[8][KBC];
#pragma unroll
            for (int jt = 0; jt < 8; ++jt)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) kt[jt][kb] = ld8(Kt + (16 * jt + li) * TP + 32 * kb + 8 * q4);
            f32x4 vv[NT], gm[NT], bt[NT], ge[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                vv[m] = *reinterpret_cast<const f32x4 *>(Vt + li * VP + 16 * m + 4 * q4);
                gm[m] = *reinterpret_cast<const f32x4 *>(gam + 16 * m + 4 * q4);
                bt[m] = *reinterpret_cast<const f32x4 *>(bet + 16 * m + 4 * q4);
                ge[m] = *reinterpret_cast<const f32x4 *>(eg + 16 * m + 4 * q4);
            }
            const float gC = gam[C - 1];

            // X = K S^T
            f16x8 sb[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
            f32x4 X[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                X[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) X[m] = mfma16x16x32(ka[m][kb], sb[kb], X[m]);
            }
            // R = diag(beta) (V - diag(gamma) X)
            f32x4 R[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) R[m] = bt[m] * (vv[m] - gm[m] * X[m]);
            // U = T R
            f16x8 rb[KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) rb[kb] = pack8(R[2 * kb], R[2 * kb + 1]);
            f32x4 U[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                U[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (kb <= m / 2) U[m] = mfma16x16x32(Tf[m][kb], rb[kb], U[m]);
            }
            // hand U (fp16, fragment order) to the helpers for the output
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb)
                *reinterpret_cast<f16x8 *>(U16 + (((c & 1) * KBC + kb) * 64 + lane) * 8) = pack8(U[2 * kb], U[2 * kb + 1]);
            // S <- gamma_C S + K^T (diag(exp(G_C - G)) U)
            f16x8 ub[KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) ub[kb] = pack8(ge[2 * kb] * U[2 * kb], ge[2 * kb + 1] * U[2 * kb + 1]);
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                S[jt] *= gC;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) S[jt] = mfma16x16x32(kt[jt][kb], ub[kb], S[jt]);
            }
            write_S16((c + 1) & 1);
            if (c + 1 < NC) {
#pragma unroll
                for (int m = 0; m < NT; ++m)
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb) Tf[m][kb] = Tn[m][kb];
            }
            __syncthreads();
        }
        if (p.final_state) {
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) *reinterpret_cast<f32x4 *>(p.final_state + srow + 16 * jt) = S[jt];
        }
    } else {
        // ================================================================ helper waves
        const int hw = w - 1;              // 0..2
        const int hl = hw * 64 + lane;     // 0..191
        // token tiles whose outputs this helper computes
        constexpr int MAXT = (NT + kHelpers - 1) / kHelpers;
        // staging registers for the next chunk
        constexpr int KV = (C * 16 + kHelpers * 64 - 1) / (kHelpers * 64);  // k vectors per lane
        constexpr int VV = (C * 2 + kHelpers * 64 - 1) / (kHelpers * 64);   // v vectors per lane
        u16x8 kreg[KV], vreg[VV];
        float greg = 0.f, breg = 0.f;
        u16x4 qreg[MAXT][4][2];            // q fragments of the next chunk, per tile and k block
        f16x8 aqk[MAXT][KBC], aqk_n[MAXT][KBC];
        f32x4 Y[MAXT], gmy[MAXT];

        auto issue_stage_loads = [&](int c) {
            const int t0 = c * C, n = min(C, T - t0);
#pragma unroll
            for (int i = 0; i < KV; ++i) {
                const int v = hl + i * kHelpers * 64;
                const int t = v % C, j0 = 8 * (v / C);
                kreg[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (v < C * 16 && t < n) kreg[i] = *reinterpret_cast<const u16x8 *>(kg + (int64_t)(t0 + t) * kD + j0);
            }
#pragma unroll
            for (int i = 0; i < VV; ++i) {
                const int v = hl + i * kHelpers * 64;
                const int t = v % C, i0 = 8 * (v / C);
                vreg[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (v < C * 2 && t < n) vreg[i] = *reinterpret_cast<const u16x8 *>(vg + (int64_t)(t0 + t) * kD + i0);
            }
            if (hw == 0) {
                greg = (lane < n) ? gg[t0 + lane] : 0.f;
                breg = (lane < n) ? bg[t0 + lane] : 0.f;
            }
        };
        auto write_stage = [&](int c) {
            unsigned char *stage = smem + (c & 1) * L::kStage;
            _Float16 *Kf = reinterpret_cast<_Float16 *>(stage + L::kKf);
            _Float16 *Kt = reinterpret_cast<_Float16 *>(stage + L::kKt);
            float *Vt = reinterpret_cast<float *>(stage + L::kVt);
#pragma unroll
            for (int i = 0; i < KV; ++i) {
                const int v = hl + i * kHelpers * 64;
                if (v < C * 16) {
                    const int t = v % C, j0 = 8 * (v / C);
                    f16x8 kh8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) kh8[e] = (_Float16)bf16_bits_to_f32(kreg[i][e]);
                    // fragment-permuted row: columns j0..j0+3 and j0+4..j0+7 are 4-runs
                    *reinterpret_cast<f16x4 *>(Kf + t * KP + frag_pos(j0)) = f16x4{kh8[0], kh8[1], kh8[2], kh8[3]};
                    *reinterpret_cast<f16x4 *>(Kf + t * KP + frag_pos(j0 + 4)) = f16x4{kh8[4], kh8[5], kh8[6], kh8[7]};
                    const int tp = frag_pos(t);
#pragma unroll
                    for (int e = 0; e < 8; ++e) Kt[(j0 + e) * TP + tp] = kh8[e];
                }
            }
#pragma unroll
            for (int i = 0; i < VV; ++i) {
                const int v = hl + i * kHelpers * 64;
                if (v < C * 2) {
                    const int t = v % C, i0 = 8 * (v / C);
#pragma unroll
                    for (int e = 0; e < 8; ++e) Vt[(i0 + e) * VP + t] = bf16_bits_to_f32(vreg[i][e]);
                }
            }
            if (hw == 0) {
                float x = greg;
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) {
                    const float y = __shfl_up(x, m, 64);
                    if (lane >= m) x += y;
                }
                const float gc = __shfl(x, C - 1, 64);
                if (lane < C) {
                    reinterpret_cast<float *>(stage + L::kGam)[lane] = __expf(x);
                    reinterpret_cast<float *>(stage + L::kBeta)[lane] = breg;
                    reinterpret_cast<float *>(stage + L::kEg)[lane] = __expf(gc - x);
                }
            }
        };
        auto load_q = [&](int c) {
            const int t0 = c * C, n = min(C, T - t0);
#pragma unroll
            for (int s = 0; s < MAXT; ++s) {
                const int m = hw + kHelpers * s;
                const int t = 16 * m + li;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        qreg[s][kb][hh] = u16x4{0, 0, 0, 0};
                        if (m < NT && t < n)
                            qreg[s][kb][hh] = *reinterpret_cast<const u16x4 *>(
                                qg + (int64_t)(t0 + t) * kD + 32 * kb + 16 * hh + 4 * q4);
                    }
            }
        };
        auto load_aqk = [&](int c) {
            const _Float16 *src = wsp + ((int64_t)c * 2 + 1) * C * C;
#pragma unroll
            for (int s = 0; s < MAXT; ++s) {
                const int m = hw + kHelpers * s;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (m < NT && kb <= m / 2) aqk_n[s][kb] = ld8(src + (16 * m + li) * C + 32 * kb + 8 * q4);
            }
        };

        if (NC > 0) {
            issue_stage_loads(0);
            load_q(0);
            write_stage(0);
        }
        __syncthreads();

        for (int c = 0; c <= NC; ++c) {
            const bool has_next = c + 1 < NC;
            if (has_next) issue_stage_loads(c + 1);
            if (c < NC) load_aqk(c);
            // O of the previous chunk
            if (c > 0) {
                const int tp0 = (c - 1) * C, np = min(C, T - tp0);
                float *og = p.o + ((int64_t)pair * T + tp0) * kD + kRows * dvb + li;
#pragma unroll
                for (int s = 0; s < MAXT; ++s) {
                    const int m = hw + kHelpers * s;
                    if (m < NT) {
                        f32x4 acc = gmy[s] * (p.scale * Y[s]);
#pragma unroll
                        for (int kb = 0; kb < KBC; ++kb)
                            if (kb <= m / 2)
                                acc = mfma16x16x32(aqk[s][kb],
                                                   ld8(U16 + ((((c - 1) & 1) * KBC + kb) * 64 + lane) * 8), acc);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * m + 4 * q4 + r;
                            if (t < np) og[(int64_t)t * kD] = acc[r];
                        }
                    }
                }
            }
            if (c < NC) {
                // Y = Q S^T of this chunk, with S the state at the chunk start
                const float *gam = reinterpret_cast<const float *>(smem + (c & 1) * L::kStage + L::kGam);
                f16x8 sbf[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) sbf[kb] = ld8(S16 + (((c & 1) * 4 + kb) * 64 + lane) * 8);
#pragma unroll
                for (int s = 0; s < MAXT; ++s) {
                    const int m = hw + kHelpers * s;
                    if (m < NT) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
                            acc = mfma16x16x32(cat(bf16x4_to_f16(qreg[s][kb][0]), bf16x4_to_f16(qreg[s][kb][1])),
                                               sbf[kb], acc);
                        Y[s] = acc;
                        gmy[s] = *reinterpret_cast<const f32x4 *>(gam + 16 * m + 4 * q4);
#pragma unroll
                        for (int kb = 0; kb < KBC; ++kb) aqk[s][kb] = aqk_n[s][kb];
                    }
                }
                if (has_next) load_q(c + 1);
            }
            if (has_next) write_stage(c + 1);
            if (c < NC) __syncthreads();
        }
    }
}

template <int C>
hipError_t launch_c(const PrefillParams &p, const _Float16 *ws, hipStream_t stream) {
    const size_t bytes = ScanSmem<C>::kBytes;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_prefill_scan_kernel<C>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (err != hipSuccess) return err;
    dim3 grid((unsigned)(p.B * p.Hv * (kD / kRows))), block(kThreads);
    hipLaunchKernelGGL((gdn_prefill_scan_kernel<C>), grid, block, bytes, stream, p, ws);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_scan(const PrefillParams &p, int chunk, const void *ws, hipStream_t stream) {
    if (p.D != kD) return hipErrorInvalidValue;
    const _Float16 *w = static_cast<const _Float16 *>(ws);
    switch (chunk) {
        case 32: return launch_c<32>(p, w, stream);
        case 64: return launch_c<64>(p, w, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
