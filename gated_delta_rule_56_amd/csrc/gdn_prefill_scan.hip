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
//   wave 0, "state": owns the 16 x 128 fp32 state block as MFMA accumulators
//     and runs only the chain S -> X -> R -> U -> S (38 MFMAs per 64-token
//     chunk). K^T operands come straight from the row-major k tile through
//     transposing LDS reads (ds_read_b64_tr_b16).
//   wave 1, "loader": streams chunk c+2 into a 3-slot LDS ring with direct
//     global->LDS loads (the fp16 k tile and T fragments and gates prepared by
//     the chunk kernel, q and v as bf16) and waits for chunk c+1 with an exact
//     vmcnt; nothing is converted in LDS.
//   waves 2-3, "output": Y = Q S^T of chunk c from an fp16 copy of S, and
//     O of chunk c-1 = gamma scale Y + A_qk U from an fp16 copy of U.
// One workgroup barrier per chunk. The k and q tiles are stored with their 16-byte
// column groups XOR-swizzled by row (group g of row t at g ^ (t % 16)) so that
// MFMA fragment reads spread over the LDS banks.
#include "gdn_device.h"
#include "gdn_frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRows = 16;
constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int C>
struct ScanSmem {
    static constexpr int NT = C / 16;     // token tiles per chunk
    static constexpr int KBC = C / 32;    // 32-wide k blocks over the chunk
    // one ring slot
    static constexpr size_t sK = 0;                        // [C][128] fp16, swizzled
    static constexpr size_t sQ = sK + 256 * C;             // [C][128] bf16, swizzled
    static constexpr size_t sT = sQ + 256 * C;             // T fragments [NT][KBC][64][8] fp16
    static constexpr size_t sV = sT + 2 * C * C;           // [C][16] bf16
    static constexpr size_t sGate = sV + 32 * C;           // gamma [C], beta [C], exp(G_C - G) [C] f32
    static constexpr size_t kSlot = sGate + 12 * C;
    static constexpr int kDmaPerChunk = C / 4 + C / 4 + NT * KBC + C / 32 + 1;
    // offsets
    static constexpr size_t kRing = 0;
    static constexpr size_t kS16 = 3 * kSlot;              // f16 [2][4][64][8]
    static constexpr size_t kU16 = kS16 + 2 * 4 * 64 * 16; // f16 [2][KBC][64][8]
    static constexpr size_t kBytes = kU16 + 2 * KBC * 64 * 16;
    static_assert(sT % 16 == 0 && sV % 16 == 0 && sGate % 16 == 0 && kSlot % 16 == 0, "alignment");
    static_assert(kDmaPerChunk <= 63, "vmcnt range");
};

__device__ __forceinline__ f16x8 ld8(const unsigned char *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ f16x4 ld4h(const unsigned char *p) { return *reinterpret_cast<const f16x4 *>(p); }

__device__ __forceinline__ f16x8 pack8(f32x4 lo, f32x4 hi) {
    return f16x8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                 (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
}

__device__ __forceinline__ f16x4 bf16x4_to_f16(u16x4 u) {
    return f16x4{(_Float16)bf16_bits_to_f32(u[0]), (_Float16)bf16_bits_to_f32(u[1]),
                 (_Float16)bf16_bits_to_f32(u[2]), (_Float16)bf16_bits_to_f32(u[3])};
}

// byte offset of the 8-byte run of row t starting at column col (col % 4 == 0) in a swizzled tile
__device__ __forceinline__ int swz(int t, int col) {
    return t * 256 + ((((col >> 3) ^ (t & 15)) << 4) | ((col & 4) << 1));
}

// transposing LDS read: with source lane 4e + a (within 16) pointing at row r0 + e, column c0 + 4a,
// lane a' receives rows r0 .. r0 + 3 of column c0 + a'
__device__ __forceinline__ f16x4 ld_tr(const unsigned char *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(f16x4, v);
}

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

// Workgroup barrier for LDS traffic only: waits for this wave's LDS reads and
// writes, not for its outstanding global loads, so the loader's direct-to-LDS
// prefetches stay in flight across it (their completion is tracked with exact
// vmcnt waits by the loader itself before any other wave reads that data).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int C>
__global__ __launch_bounds__(kThreads) void gdn_prefill_scan_kernel(PrefillParams p, const _Float16 *ws) {
    using L = ScanSmem<C>;
    constexpr int NT = L::NT, KBC = L::KBC;
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
    const ChunkWs<C> wl(p.B, p.Hk, p.Hv, NC);

    unsigned char *S16 = smem + L::kS16;  // [2][4][64] x 16 B
    unsigned char *U16 = smem + L::kU16;  // [2][KBC][64] x 16 B
    auto slot = [&](int c) { return smem + L::kRing + (c % 3) * L::kSlot; };

    if (w == 0) {
        // ================================================================ state wave
        // S[jt][r] = state[16 dvb + li][16 jt + 4 q4 + r]
        const int64_t srow = ((int64_t)pair * kD + kRows * dvb + li) * kD + 4 * q4;
        f32x4 S[8];
#pragma unroll
        for (int jt = 0; jt < 8; ++jt)
            S[jt] = p.init_state ? *reinterpret_cast<const f32x4 *>(p.init_state + srow + 16 * jt)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
        auto write_S16 = [&](int buf) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                *reinterpret_cast<f16x8 *>(S16 + ((buf * 4 + kb) * 64 + lane) * 16) = pack8(S[2 * kb], S[2 * kb + 1]);
        };
        write_S16(0);
        lds_barrier();

        for (int c = 0; c < NC; ++c) {
            const unsigned char *sl = slot(c);
            const unsigned char *kt = sl + L::sK;
            const uint16_t *vr = reinterpret_cast<const uint16_t *>(sl + L::sV);
            const float *gam = reinterpret_cast<const float *>(sl + L::sGate);
            const float *bet = gam + C;
            const float *eg = gam + 2 * C;

            // X = K S^T; A operand: row 16 m + li, columns frag_col(kb, q4, .) (two 8-byte runs)
            f16x8 sb[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
            f32x4 X[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const int t = 16 * m + li;
                X[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const f16x8 a = cat(ld4h(kt + swz(t, 32 * kb + 4 * q4)), ld4h(kt + swz(t, 32 * kb + 16 + 4 * q4)));
                    X[m] = mfma16x16x32(a, sb[kb], X[m]);
                }
            }
            // K^T fragments for the update: rows frag_col(kb, q4, .) of column 16 jt + li
            f16x8 ktf[8][KBC];
            {
                const int e = li >> 2, a4 = (li & 3) * 4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt)
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb) {
                        const int r0 = 32 * kb + 4 * q4 + e;
                        ktf[jt][kb] = cat(ld_tr(kt + swz(r0, 16 * jt + a4)), ld_tr(kt + swz(r0 + 16, 16 * jt + a4)));
                    }
            }
            f16x8 Tf[NT][KBC];
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (kb <= m / 2) Tf[m][kb] = ld8(sl + L::sT + ((m * KBC + kb) * 64 + lane) * 16);
            f32x4 vv[NT], gm[NT], bt[NT], ge[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) vv[m][r] = bf16_bits_to_f32(vr[(16 * m + 4 * q4 + r) * kRows + li]);
                gm[m] = *reinterpret_cast<const f32x4 *>(gam + 16 * m + 4 * q4);
                bt[m] = *reinterpret_cast<const f32x4 *>(bet + 16 * m + 4 * q4);
                ge[m] = *reinterpret_cast<const f32x4 *>(eg + 16 * m + 4 * q4);
            }
            const float gC = gam[C - 1];

            // R = diag(beta) (V - diag(gamma) X);  U = T R
            f32x4 R[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) R[m] = bt[m] * (vv[m] - gm[m] * X[m]);
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
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb)
                *reinterpret_cast<f16x8 *>(U16 + (((c & 1) * KBC + kb) * 64 + lane) * 16) = pack8(U[2 * kb], U[2 * kb + 1]);
            // S <- gamma_C S + K^T (diag(exp(G_C - G)) U)
            f16x8 ub[KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) ub[kb] = pack8(ge[2 * kb] * U[2 * kb], ge[2 * kb + 1] * U[2 * kb + 1]);
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                S[jt] *= gC;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) S[jt] = mfma16x16x32(ktf[jt][kb], ub[kb], S[jt]);
            }
            write_S16((c + 1) & 1);
            lds_barrier();
        }
        if (p.final_state) {
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) *reinterpret_cast<f32x4 *>(p.final_state + srow + 16 * jt) = S[jt];
        }
    } else if (w == 1) {
        // ================================================================ loader wave
        const uint16_t *qg = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hk + kh) * T * kD;
        const uint16_t *vg = static_cast<const uint16_t *>(p.v) + (int64_t)pair * T * kD + kRows * dvb;
        // issue every direct-to-LDS load of chunk c (exactly L::kDmaPerChunk instructions)
        auto issue = [&](int c) {
            unsigned char *sl = slot(c);
            const int t0 = c * C, last = min(C, T - t0) - 1;
            const _Float16 *kw = ws + wl.key_chunk((int64_t)b * p.Hk + kh, c);
            const _Float16 *pw = ws + wl.pair_chunk(pair, c);
#pragma unroll
            for (int i = 0; i < C / 4; ++i) {
                // k: prepared fp16 tile, copied verbatim; q: bf16 rows, swizzled on the way in
                dma16(kw + (i * 64 + lane) * 8, sl + L::sK + i * 1024);
                const int pidx = i * 64 + lane, t = pidx >> 4, g = (pidx & 15) ^ (t & 15);
                dma16(qg + (int64_t)(t0 + min(t, last)) * kD + 8 * g, sl + L::sQ + i * 1024);
            }
#pragma unroll
            for (int i = 0; i < NT * KBC; ++i) dma16(pw + (i * 64 + lane) * 8, sl + L::sT + i * 1024);
#pragma unroll
            for (int i = 0; i < C / 32; ++i) {
                const int t = 32 * i + (lane >> 1);
                dma16(vg + (int64_t)(t0 + min(t, last)) * kD + 8 * (lane & 1), sl + L::sV + i * 1024);
            }
            if (lane < 3 * C / 4) dma16(pw + 2 * C * C + lane * 8, sl + L::sGate);
        };

        if (NC > 0) issue(0);
        if (NC > 1) {
            issue(1);
            wait_vmcnt<L::kDmaPerChunk>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (c + 2 < NC) {
                issue(c + 2);
                wait_vmcnt<L::kDmaPerChunk>();
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
        }
    } else {
        // ================================================================ output waves
        const int ow = w - 2;  // 0, 1: token tiles ow, ow + 2
        constexpr int MAXT = (NT + 1) / 2;
        f32x4 Y[MAXT], gmy[MAXT];
        f16x8 aqk[MAXT][KBC];
        auto load_aqk = [&](int c) {
            const _Float16 *src = ws + wl.pair_chunk(pair, c) + C * C;
#pragma unroll
            for (int s = 0; s < MAXT; ++s) {
                const int m = ow + 2 * s;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (m < NT && kb <= m / 2)
                        aqk[s][kb] = *reinterpret_cast<const f16x8 *>(src + ((m * KBC + kb) * 64 + lane) * 8);
            }
        };
        lds_barrier();
        for (int c = 0; c <= NC; ++c) {
            if (c > 0) {
                // O of the previous chunk
                const int tp0 = (c - 1) * C, np = min(C, T - tp0);
                float *og = p.o + ((int64_t)pair * T + tp0) * kD + kRows * dvb + li;
#pragma unroll
                for (int s = 0; s < MAXT; ++s) {
                    const int m = ow + 2 * s;
                    if (m < NT) {
                        f32x4 acc = gmy[s] * (p.scale * Y[s]);
#pragma unroll
                        for (int kb = 0; kb < KBC; ++kb)
                            if (kb <= m / 2)
                                acc = mfma16x16x32(aqk[s][kb], ld8(U16 + ((((c - 1) & 1) * KBC + kb) * 64 + lane) * 16), acc);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * m + 4 * q4 + r;
                            if (t < np) og[(int64_t)t * kD] = acc[r];
                        }
                    }
                }
            }
            if (c < NC) {
                load_aqk(c);
                // Y = Q S^T of this chunk, with S the state at the chunk start
                const unsigned char *qt = slot(c) + L::sQ;
                const float *gam = reinterpret_cast<const float *>(slot(c) + L::sGate);
                f16x8 sbf[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) sbf[kb] = ld8(S16 + (((c & 1) * 4 + kb) * 64 + lane) * 16);
#pragma unroll
                for (int s = 0; s < MAXT; ++s) {
                    const int m = ow + 2 * s;
                    if (m < NT) {
                        const int t = 16 * m + li;
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const u16x4 lo = *reinterpret_cast<const u16x4 *>(qt + swz(t, 32 * kb + 4 * q4));
                            const u16x4 hi = *reinterpret_cast<const u16x4 *>(qt + swz(t, 32 * kb + 16 + 4 * q4));
                            acc = mfma16x16x32(cat(bf16x4_to_f16(lo), bf16x4_to_f16(hi)), sbf[kb], acc);
                        }
                        Y[s] = acc;
                        gmy[s] = *reinterpret_cast<const f32x4 *>(gam + 16 * m + 4 * q4);
                    }
                }
                lds_barrier();
            }
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
