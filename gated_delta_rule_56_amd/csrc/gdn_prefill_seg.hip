// Segmented bf16 prefill: the chunks of one sequence are cut into P segments that
// run in parallel, each workgroup holding all dv = 128 rows of the state of one
// (b, value head, segment), with the chunk preparation fused in.
//
// Chunked WY form, per chunk of C tokens with start state S (dv x dk), local t:
//   G_t = sum_{s<=t} g_s,  Gamma_ts = exp(G_t - G_s) (s <= t)
//   A = strict_lower(diag(beta) (K K^T o Gamma)),  T = (I + A)^{-1}
//   X = K S^T,  R = diag(beta) V - diag(beta gamma) X,  U = T R
//   O = diag(gamma) (scale Q S^T) + lower_incl(scale Q K^T o Gamma) U
//   S <- gamma_C S + (diag(exp(G_C - G)) U)^T K
// (of S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t scale q_t; the state update and the output taken from the updated
// state are those of the gated-delta reference tests on the "27b 935/47" compare
// page; padded steps with beta = 0, g = 0 are exact no-ops, the symbolic-length
// prefill entry of the "mergable fast RDNA3 Qwen 3.6" commit log).
//
// The chunk update is affine in the start state: S_new = S M_c + N_c. A segment
// of chunks therefore maps its start S_p to S_p M_p + N_p, with N_p the end state
// from a zero start and M_p the end "state" of the identity run with v = 0 (each
// identity row is a state row; rows never mix). Three launches:
//   1. map pass (OUT = false): segment 0 from the initial state (its end is the
//      true start of segment 1), and for segments 1 .. P-2 both N_p (role 0) and
//      M_p (role 1);
//   2. combine: S_{p+1} = S_p M_p + N_p, sequential over the segments, in fp32;
//   3. output pass (OUT = true): every segment from its true start, writing o and,
//      in the last segment, the final state.
// With P = 1 only the output pass runs.
//
// Workgroup of 8 waves (wave i on SIMD i % 4):
//   waves 0-3, "row waves": state rows 32 w .. 32 w + 31 as two 16-row MFMA blocks
//     held in registers for the whole segment; per chunk X, R, U, the update and
//     (OUT) Y = S Q^T and O^T. Every operand of chunk i is in LDS slot i & 1 when
//     the chunk starts.
//   waves 4-7, "prep waves", token tile m = w - 4: prepare chunk i + 1 into slot
//     (i + 1) & 1 during chunk i, in three phases separated by workgroup barriers:
//     P1 converts the raw bf16 k, q rows of tile m (loaded one chunk earlier into
//     registers) to the fp16 k and q tiles and stores the v rows, then issues the
//     loads of chunk i + 2; P2 forms K K^T and Q K^T of tile m against tiles <= m
//     on MFMA, the gates, A and A_qk, and the 16 x 16 diagonal block of T by
//     substitution; P3 (wave 4) joins the diagonal blocks into T by MFMA doubling
//     and writes the T fragments.
//   Every wave runs exactly three barriers per chunk.
//
// LDS tiles of k and q: row-major 256-byte token rows, each 32-column block in
// fragment order (gdn_frag.h), 16-byte groups XOR-swizzled by row; v is stored
// in plain column order with the same swizzle and read transposed
// (ds_read_b64_tr_b16) by the row waves.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kSegThreads = 512;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// fragment block of token tile m, k block kb (kb <= m / 2), counted over the blocks on or
// below the diagonal: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__host__ __device__ constexpr int fblk(int m, int kb) { return m + (m > 2 ? m - 2 : 0) + kb; }

template <int C, bool OUT>
struct SegSmem {
    static constexpr int NT = C / 16, KBC = C / 32;
    static constexpr int CP = C + 8;                             // fp16 pitch of Ah, Tm
    static constexpr int DP = 20;                                // f32 pitch of a transposed diagonal block
    static constexpr int kFr = fblk(NT - 1, (NT - 1) / 2) + 1;   // fragment blocks of T / A_qk
    static constexpr size_t kTile = (size_t)C * 256;             // C x 128 16-bit values
    static constexpr size_t oK = 0;                              // [2] fp16 k tiles
    static constexpr size_t oQ = oK + 2 * kTile;                 // [2] fp16 q tiles (OUT)
    static constexpr size_t oV = oQ + (OUT ? 2 * kTile : 0);     // [2] bf16 v tiles
    static constexpr size_t oT = oV + 2 * kTile;                 // [2][kFr][64] x 16 B T fragments
    static constexpr size_t oA = oT + 2 * kFr * 1024;            // [2][kFr][64] x 16 B A_qk fragments (OUT)
    static constexpr size_t oG = oA + (OUT ? 2 * kFr * 1024 : 0);  // [2][4][C] f32: gamma, beta, exp(G_C-G), beta gamma
    static constexpr size_t oAh = oG + 2 * 16 * C;               // fp16 [C][CP]: A below the diagonal blocks
    static constexpr size_t oTm = oAh + 2 * C * CP;              // fp16 [C][CP]: T
    static constexpr size_t oAd = oTm + 2 * C * CP;              // f32 [NT][16][DP]: diagonal blocks of A, transposed
    static constexpr size_t oGt = oAd + 4 * NT * 16 * DP;        // f32 [4][2][64]: G and beta per prep wave
    static constexpr size_t kBytes = oGt + 4 * 2 * 64 * 4;
    static_assert(oQ % 16 == 0 && oV % 16 == 0 && oT % 16 == 0 && oA % 16 == 0 && oG % 16 == 0 &&
                      oAh % 16 == 0 && oTm % 16 == 0 && oAd % 16 == 0 && oGt % 16 == 0,
                  "alignment");
    static_assert(kBytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ f16x8 ld8(const unsigned char *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ f32x4 ldf4(const unsigned char *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f16x4 ld4h(const _Float16 *p) { return *reinterpret_cast<const f16x4 *>(p); }

__device__ __forceinline__ f16x8 pack8(f32x4 lo, f32x4 hi) {
    return f16x8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                 (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
}

// transposing LDS read of 16-bit values: with source lane 4e + a (within 16 lanes) pointing at
// row r0 + e, columns c0 + 4a .. + 3, lane a' receives rows r0 .. r0 + 3 of column c0 + a'
__device__ __forceinline__ s16x4 ld_tr_raw(const unsigned char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ f16x4 ld_tr(const unsigned char *p) { return __builtin_bit_cast(f16x4, ld_tr_raw(p)); }

// Workgroup barrier for LDS traffic only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
using IC = std::integral_constant<int, N>;

// bf16 -> fp16 for 4 values (exact within fp16 range)
__device__ __forceinline__ f16x4 bf4_to_h4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
    return f16x4{(_Float16)bf16_bits_to_f32(a), (_Float16)bf16_bits_to_f32(b), (_Float16)bf16_bits_to_f32(c),
                 (_Float16)bf16_bits_to_f32(d)};
}

template <int C, bool OUT>
__global__ __launch_bounds__(kSegThreads, 1) void gdn_seg_pass_kernel(SegParams sp) {
    using L = SegSmem<C, OUT>;
    constexpr int NT = L::NT, KBC = L::KBC, CP = L::CP, DP = L::DP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // every argument into a scalar local: a reference to the argument structure would make
    // the compiler copy it to scratch memory
    struct Args {
        const void *q, *k, *v, *init_state;
        const float *g, *beta;
        void *o, *final_state;
        float *ws_start, *ws_n, *ws_m;
        int B, T, Hk, Hv, Ts, head_map, P, seg_chunks;
        float scale;
        bool init_f16, final_f16, o_f16;
    };
    const Args p = {sp.p.q, sp.p.k, sp.p.v, sp.p.init_state, sp.p.g, sp.p.beta, sp.p.o, sp.p.final_state,
                    sp.ws_start, sp.ws_n, sp.ws_m, sp.p.B, sp.p.T, sp.p.Hk, sp.p.Hv, sp.p.Ts, sp.p.head_map,
                    sp.P, sp.seg_chunks, sp.p.scale, sp.p.init_f16, sp.p.final_f16, sp.p.o_f16};

    // ---- workgroup -> (b, key head, unit, value head of the key head). Consecutive indices
    // share the key head's k and q and sit on one XCD (workgroups go round-robin over 8 XCDs).
    const int nb = gridDim.x;
    int lin = blockIdx.x;
    if ((nb & 7) == 0) lin = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
    const int ratio = p.Hv / p.Hk;
    const int jj = lin % ratio;
    int rest = lin / ratio;
    int seg, role;  // role 0: state rows (from the start state, with v); 1: identity rows, v = 0
    if (OUT) {
        seg = rest % p.P;
        rest /= p.P;
        role = 0;
    } else {
        const int units = 2 * p.P - 3;
        const int u = rest % units;
        rest /= units;
        seg = u == 0 ? 0 : 1 + (u - 1) / 2;
        role = u == 0 ? 0 : (u - 1) % 2;
    }
    const int kh = rest % p.Hk, b = rest / p.Hk;
    const int h = p.head_map == 0 ? kh + jj * p.Hk : kh * ratio + jj;
    const int pair = b * p.Hv + h;
    const bool has_v = role == 0;

    const int T = p.T;
    const int NC = (T + C - 1) / C;
    const int cb = seg * p.seg_chunks;
    const int n = max(0, min(NC, cb + p.seg_chunks) - cb);  // chunks of this segment
    const int64_t ktok = ((int64_t)b * p.Hk + kh) * p.Ts;      // first token row of q, k
    const int64_t vtok = (int64_t)pair * p.Ts;                 // first token row of v, g, beta, o
    const int64_t wsi = ((int64_t)pair * p.P + seg) * (kD * kD);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, q4 = lane >> 4;

    if (w < 4) {
        // ================================================================ row waves
        // S[bb][jt][r] = state[r0 + li][16 jt + 4 q4 + r], r0 = 32 w + 16 bb
        f32x4 S[2][8];
        {
            // start state: the output pass reads the float32 copies in the workspace when the
            // sequence is split (segment 0's copy of initial_state, then the combined starts),
            // else initial_state itself; the map pass starts segment 0 from initial_state,
            // the other segments from zero (role 0) or the identity (role 1)
            const void *src = nullptr;
            bool ws_layout = false, f16 = false;
            if (OUT && p.P > 1) {
                src = (seg > 0 || p.init_state) ? p.ws_start + wsi : nullptr;
                ws_layout = true;
            } else if (seg == 0 && role == 0) {
                src = p.init_state;
                f16 = p.init_f16;
            }
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int r0 = 32 * w + 16 * bb;
                const int64_t srow = ws_layout ? (int64_t)(r0 + li) * kD + 4 * q4
                                               : ((int64_t)pair * kD + r0 + li) * kD + 4 * q4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) {
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
                    if (!OUT && role == 1) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = (16 * jt + 4 * q4 + r == r0 + li) ? 1.0f : 0.0f;
                    } else if (src) {
                        x = load_state4(src, srow + 16 * jt, f16);
                    }
                    S[bb][jt] = x;
                }
            }
        }
        // the map pass's segment 0 keeps a float32 copy of the initial state for the output pass
        // (which must not read initial_state when it is also final_state)
        if (!OUT && role == 0 && seg == 0 && p.init_state) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int64_t wrow = (int64_t)(32 * w + 16 * bb + li) * kD + 4 * q4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt)
                    *reinterpret_cast<f32x4 *>(p.ws_start + wsi + wrow + 16 * jt) = S[bb][jt];
            }
        }
        f16x8 sb[2][4];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sb[bb][kb] = pack8(S[bb][2 * kb], S[bb][2 * kb + 1]);

        // per-lane LDS addresses (slot, tile and block offsets are immediates)
        int xo[4];  // offset in a k / q tile: row li, group 4 kb + q4
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) xo[kb] = li * 256 + (((4 * kb + q4) ^ ksw(li)) << 4);
        const unsigned char *ta[8];  // k tile read transposed: column tile jt of the update
        {
            const int rt = 4 * q4 + (li >> 2);
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                const int g = 4 * (jt >> 1) + (li & 3);
                ta[jt] = smem + L::oK + rt * 256 + ((g ^ ksw(rt)) << 4) + (jt & 1) * 8;
            }
        }
        const unsigned char *va[2];  // v tile read transposed: tokens 4 q4 + (li >> 2), columns r0 + 4 (li & 3)
        {
            const int rt = 4 * q4 + (li >> 2);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int c = 32 * w + 16 * bb + 4 * (li & 3);
                va[bb] = smem + L::oV + rt * 256 + (((c >> 3) ^ ksw(rt)) << 4) + (c & 7) * 2;
            }
        }
        const unsigned char *fa = smem + lane * 16;          // T / A_qk fragments
        const unsigned char *ga = smem + L::oG + 16 * q4;    // gate vectors, tokens 4 q4 .. + 3 of a tile
        float *o_f32 = static_cast<float *>(p.o);
        _Float16 *o_f16 = static_cast<_Float16 *>(p.o);

        lds_barrier();
        lds_barrier();
        lds_barrier();

        auto interval = [&](auto sl, int i) __attribute__((always_inline)) {
            constexpr int s = decltype(sl)::value;
            const unsigned char *Kt = smem + L::oK + s * L::kTile;
            const float *gts = reinterpret_cast<const float *>(smem + L::oG + s * 16 * C);

            // X = K S^T for both row blocks
            f32x4 X[2][NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                X[0][m] = f32x4{0.f, 0.f, 0.f, 0.f};
                X[1][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const f16x8 kf = ld8(Kt + xo[kb] + m * 4096);
                    X[0][m] = mfma16x16x32(kf, sb[0][kb], X[0][m]);
                    X[1][m] = mfma16x16x32(kf, sb[1][kb], X[1][m]);
                }
            }
            lds_barrier();  // b1
            // Y^T = S Q^T (lane: row 4 q4 + r of the block, token 16 m + li), from the chunk-start S
            f32x4 Y[2][NT];
            if constexpr (OUT) {
                const unsigned char *Qt = smem + L::oQ + s * L::kTile;
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    Y[0][m] = f32x4{0.f, 0.f, 0.f, 0.f};
                    Y[1][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const f16x8 qf = ld8(Qt + xo[kb] + m * 4096);
                        Y[0][m] = mfma16x16x32(sb[0][kb], qf, Y[0][m]);
                        Y[1][m] = mfma16x16x32(sb[1][kb], qf, Y[1][m]);
                    }
                }
            }
            // R = beta V - beta gamma X  (v read transposed: tokens 16 m + 4 q4 + r, column r0 + li)
            f16x8 rb[2][KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                f32x4 R[2][2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int m = 2 * kb + hh;
                    const f32x4 bt = ldf4(ga + s * 16 * C + 4 * C + 64 * m);
                    const f32x4 bg = ldf4(ga + s * 16 * C + 12 * C + 64 * m);
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) {
                        f32x4 vv = {0.f, 0.f, 0.f, 0.f};
                        if (has_v) {
                            const s16x4 raw = ld_tr_raw(va[bb] + s * L::kTile + m * 4096);
#pragma unroll
                            for (int r = 0; r < 4; ++r) vv[r] = bf16_bits_to_f32((uint16_t)raw[r]);
                        }
                        R[bb][hh] = bt * vv - bg * X[bb][m];
                    }
                }
                rb[0][kb] = pack8(R[0][0], R[0][1]);
                rb[1][kb] = pack8(R[1][0], R[1][1]);
            }
            // U = T R
            f32x4 U[2][NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                U[0][m] = f32x4{0.f, 0.f, 0.f, 0.f};
                U[1][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= m / 2; ++kb) {
                    const f16x8 tf = ld8(fa + L::oT + s * L::kFr * 1024 + fblk(m, kb) * 1024);
                    U[0][m] = mfma16x16x32(tf, rb[0][kb], U[0][m]);
                    U[1][m] = mfma16x16x32(tf, rb[1][kb], U[1][m]);
                }
            }
            // O^T = scale Y^T diag(gamma) + U^T A_qk^T; lane: token 16 m + li, columns r0 + 4 q4 .. + 3
            if constexpr (OUT) {
                f16x8 ua[2][KBC];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) {
                    ua[0][kb] = pack8(U[0][2 * kb], U[0][2 * kb + 1]);
                    ua[1][kb] = pack8(U[1][2 * kb], U[1][2 * kb + 1]);
                }
                const int c = cb + i;
                const int ntok = min(C, T - c * C);
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    const float gs = gts[16 * m + li] * p.scale;
                    f32x4 O0 = gs * Y[0][m], O1 = gs * Y[1][m];
#pragma unroll
                    for (int kb = 0; kb <= m / 2; ++kb) {
                        const f16x8 af = ld8(fa + L::oA + s * L::kFr * 1024 + fblk(m, kb) * 1024);
                        O0 = mfma16x16x32(ua[0][kb], af, O0);
                        O1 = mfma16x16x32(ua[1][kb], af, O1);
                    }
                    const int t = 16 * m + li;
                    if (t < ntok) {
                        const int64_t row = (vtok + (int64_t)c * C + t) * kD + 32 * w + 4 * q4;
                        if (p.o_f16) {
                            *reinterpret_cast<f16x4 *>(o_f16 + row) =
                                f16x4{f16_out(O0[0]), f16_out(O0[1]), f16_out(O0[2]), f16_out(O0[3])};
                            *reinterpret_cast<f16x4 *>(o_f16 + row + 16) =
                                f16x4{f16_out(O1[0]), f16_out(O1[1]), f16_out(O1[2]), f16_out(O1[3])};
                        } else {
                            *reinterpret_cast<f32x4 *>(o_f32 + row) = O0;
                            *reinterpret_cast<f32x4 *>(o_f32 + row + 16) = O1;
                        }
                    }
                }
            }
            lds_barrier();  // b2
            // S <- gamma_C S + K^T (diag(exp(G_C - G)) U)
            f16x8 ub[2][KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                const f32x4 e0 = ldf4(ga + s * 16 * C + 8 * C + 64 * (2 * kb));
                const f32x4 e1 = ldf4(ga + s * 16 * C + 8 * C + 64 * (2 * kb + 1));
                ub[0][kb] = pack8(e0 * U[0][2 * kb], e1 * U[0][2 * kb + 1]);
                ub[1][kb] = pack8(e0 * U[1][2 * kb], e1 * U[1][2 * kb + 1]);
            }
            const float gC = gts[C - 1];
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                S[0][jt] *= gC;
                S[1][jt] *= gC;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) {
                    const f16x8 kt = cat(ld_tr(ta[jt] + s * L::kTile + kb * 8192),
                                         ld_tr(ta[jt] + s * L::kTile + kb * 8192 + 4096));
                    S[0][jt] = mfma16x16x32(kt, ub[0][kb], S[0][jt]);
                    S[1][jt] = mfma16x16x32(kt, ub[1][kb], S[1][jt]);
                }
            }
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) sb[bb][kb] = pack8(S[bb][2 * kb], S[bb][2 * kb + 1]);
            lds_barrier();  // b3
        };
        for (int i = 0; i < n; i += 2) {
            interval(IC<0>{}, i);
            if (i + 1 < n) interval(IC<1>{}, i + 1);
        }

        // ---- the segment's end state
        void *dst = nullptr;
        bool f16 = false;
        if (OUT) {
            if (seg == p.P - 1) {
                dst = p.final_state;
                f16 = p.final_f16;
            }
        } else {
            dst = role == 1 ? p.ws_m + wsi : seg == 0 ? p.ws_start + wsi + kD * kD : p.ws_n + wsi;
        }
        if (dst) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int r0 = 32 * w + 16 * bb;
                const int64_t srow = ((int64_t)(OUT ? pair * kD : 0) + r0 + li) * kD + 4 * q4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) store_state4(dst, srow + 16 * jt, S[bb][jt], f16);
            }
        }
    } else {
        // ================================================================ prep waves
        const int m = w - 4;  // token tile of this wave
        const bool tile = m < NT;
        _Float16 *Ah = reinterpret_cast<_Float16 *>(smem + L::oAh);
        _Float16 *Tm = reinterpret_cast<_Float16 *>(smem + L::oTm);
        float *adt = reinterpret_cast<float *>(smem + L::oAd) + (tile ? m : 0) * 16 * DP;
        float *gtab = reinterpret_cast<float *>(smem + L::oGt) + m * 128;
        const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ktok * kD;
        const uint16_t *qg = static_cast<const uint16_t *>(p.q) + ktok * kD;
        const uint16_t *vg = static_cast<const uint16_t *>(p.v) + vtok * kD;
        const float *gg = p.g + vtok;
        const float *bgp = p.beta + vtok;

        // the upper blocks inside written T fragments ((0,1), (2,3)) stay zero
        if (m == 0) {
            for (int e = lane; e < 16 * 16; e += 64) {
                Tm[(e >> 4) * CP + 16 + (e & 15)] = (_Float16)0.0f;
                if (NT == 4) Tm[(32 + (e >> 4)) * CP + 48 + (e & 15)] = (_Float16)0.0f;
            }
        }

        // raw rows of tile m of one chunk: lane l holds token 16 m + l / 4; k and q columns
        // 32 kb + 8 j + 0..7 and 32 kb + 16 + 8 j + 0..7 (kb = l % 4, j = 0, 1); v columns
        // 32 (l % 4) + 0..31; g and beta of token l (all C tokens of the chunk)
        u16x8 kr[4], qr[4], vr[4];
        float graw = 0.f, braw = 0.f;
        const int lt = lane >> 2, lkb = lane & 3;
        auto issue = [&](int c) __attribute__((always_inline)) {  // chunk c (absolute), loads into the registers above
            const int t0 = c * C;
            const int tt = min(t0 + 16 * m + lt, T - 1);
            if (tile) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    kr[2 * j] = *reinterpret_cast<const u16x8 *>(kg + (int64_t)tt * kD + 32 * lkb + 8 * j);
                    kr[2 * j + 1] = *reinterpret_cast<const u16x8 *>(kg + (int64_t)tt * kD + 32 * lkb + 16 + 8 * j);
                    if (OUT) {
                        qr[2 * j] = *reinterpret_cast<const u16x8 *>(qg + (int64_t)tt * kD + 32 * lkb + 8 * j);
                        qr[2 * j + 1] = *reinterpret_cast<const u16x8 *>(qg + (int64_t)tt * kD + 32 * lkb + 16 + 8 * j);
                    }
                }
                if (has_v) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        vr[j] = *reinterpret_cast<const u16x8 *>(vg + (int64_t)tt * kD + 32 * lkb + 8 * j);
                }
            }
            const int tg = min(t0 + lane, T - 1);
            graw = gg[tg];
            braw = bgp[tg];
        };
        // P1: chunk c into slot s (waits for its loads)
        auto phase1 = [&](int c, int s) __attribute__((always_inline)) {
            const int t0 = c * C;
            const bool live = t0 + 16 * m + lt < T;
            if (tile) {
                const int t = 16 * m + lt;
                unsigned char *krow = smem + L::oK + s * L::kTile + t * 256;
                unsigned char *qrow = smem + L::oQ + s * L::kTile + t * 256;
                unsigned char *vrow = smem + L::oV + s * L::kTile + t * 256;
                const int sw = ksw(t & 15);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u16x8 a = kr[2 * j], bq = kr[2 * j + 1];
                    f16x8 g0 = cat(bf4_to_h4(a[0], a[1], a[2], a[3]), bf4_to_h4(bq[0], bq[1], bq[2], bq[3]));
                    f16x8 g1 = cat(bf4_to_h4(a[4], a[5], a[6], a[7]), bf4_to_h4(bq[4], bq[5], bq[6], bq[7]));
                    if (!live) g0 = g1 = f16x8{};
                    *reinterpret_cast<f16x8 *>(krow + (((4 * lkb + 2 * j) ^ sw) << 4)) = g0;
                    *reinterpret_cast<f16x8 *>(krow + (((4 * lkb + 2 * j + 1) ^ sw) << 4)) = g1;
                    if (OUT) {
                        const u16x8 qa = qr[2 * j], qb = qr[2 * j + 1];
                        f16x8 h0 = cat(bf4_to_h4(qa[0], qa[1], qa[2], qa[3]), bf4_to_h4(qb[0], qb[1], qb[2], qb[3]));
                        f16x8 h1 = cat(bf4_to_h4(qa[4], qa[5], qa[6], qa[7]), bf4_to_h4(qb[4], qb[5], qb[6], qb[7]));
                        if (!live) h0 = h1 = f16x8{};
                        *reinterpret_cast<f16x8 *>(qrow + (((4 * lkb + 2 * j) ^ sw) << 4)) = h0;
                        *reinterpret_cast<f16x8 *>(qrow + (((4 * lkb + 2 * j + 1) ^ sw) << 4)) = h1;
                    }
                }
                if (has_v) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u16x8 x = vr[j];
                        if (!live) x = u16x8{};
                        *reinterpret_cast<u16x8 *>(vrow + (((4 * lkb + j) ^ sw) << 4)) = x;
                    }
                }
            }
        };
        // P2: gates, K K^T and Q K^T of tile m, A, A_qk, the diagonal block of T (chunk c, slot s)
        auto phase2 = [&](int c, int s, float graw_c, float braw_c) __attribute__((always_inline)) {
            const int t0 = c * C;
            const bool gl = lane < C && t0 + lane < T;
            const float gv = gl ? graw_c : 0.f, bv = gl ? braw_c : 0.f;
            float G = gv;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(G, o, 64);
                if (lane >= o) G += y;
            }
            if (!tile) return;
            gtab[lane] = G;
            gtab[64 + lane] = bv;
            if (m == 0 && lane < C) {
                const float gC = __shfl(G, C - 1, 64);
                float *gts = reinterpret_cast<float *>(smem + L::oG + s * 16 * C);
                const float gam = __expf(G);
                gts[lane] = gam;
                gts[C + lane] = bv;
                gts[2 * C + lane] = __expf(gC - G);
                gts[3 * C + lane] = bv * gam;
            }
            // raw products, lane (q4, li): t = 16 m + li, s = 16 nt + 4 q4 + r
            const unsigned char *Kt = smem + L::oK + s * L::kTile;
            const unsigned char *Qt = smem + L::oQ + s * L::kTile;
            f32x4 rk[NT], rq[NT];
            f16x8 bk[4], bq[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bk[kb] = ld8(Kt + (16 * m + li) * 256 + (((4 * kb + q4) ^ ksw(li)) << 4));
                if (OUT) bq[kb] = ld8(Qt + (16 * m + li) * 256 + (((4 * kb + q4) ^ ksw(li)) << 4));
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                rk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                rq[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (nt <= m) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const f16x8 a = ld8(Kt + (16 * nt + li) * 256 + (((4 * kb + q4) ^ ksw(li)) << 4));
                        rk[nt] = mfma16x16x32(a, bk[kb], rk[nt]);
                        if (OUT) rq[nt] = mfma16x16x32(a, bq[kb], rq[nt]);
                    }
                }
            }
            const int t = 16 * m + li;
            const float Gt = gtab[t], bt = gtab[64 + t];
            f32x4 a[NT], aq[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                a[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                aq[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (nt <= m) {
                    const f32x4 Gs = *reinterpret_cast<const f32x4 *>(gtab + 16 * nt + 4 * q4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int sidx = 16 * nt + 4 * q4 + r;
                        const float gate = __expf(Gt - Gs[r]);
                        a[nt][r] = sidx < t ? bt * gate * rk[nt][r] : 0.0f;
                        if (OUT) aq[nt][r] = sidx <= t ? p.scale * gate * rq[nt][r] : 0.0f;
                    }
                    if (nt < m) *reinterpret_cast<f16x4 *>(Ah + t * CP + 16 * nt + 4 * q4) = to_f16x4(a[nt]);
                }
            }
            if (OUT) {
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (2 * kb <= m)
                        *reinterpret_cast<f16x8 *>(smem + L::oA + s * L::kFr * 1024 + fblk(m, kb) * 1024 + lane * 16) =
                            cat(to_f16x4(aq[2 * kb]), to_f16x4(aq[2 * kb + 1]));
            }
            // diagonal block T_mm = (I + A_mm)^{-1}: lane li computes column li by forward
            // substitution in fp32; A_mm goes through LDS transposed, adt[s][i] = A[i][s]
            {
                f32x4 dm = a[0];
#pragma unroll
                for (int nt = 1; nt < NT; ++nt)
                    if (nt == m) dm = a[nt];
#pragma unroll
                for (int r = 0; r < 4; ++r) adt[(4 * q4 + r) * DP + li] = dm[r];
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = r == li ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < 15; ++s2) {
                    float col[16];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const f32x4 c4 = *reinterpret_cast<const f32x4 *>(adt + s2 * DP + 4 * v);
                        col[4 * v] = c4[0];
                        col[4 * v + 1] = c4[1];
                        col[4 * v + 2] = c4[2];
                        col[4 * v + 3] = c4[3];
                    }
#pragma unroll
                    for (int r = s2 + 1; r < 16; ++r) x[r] -= col[r] * x[s2];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = q4 == 0 ? x[r] : q4 == 1 ? x[4 + r] : q4 == 2 ? x[8 + r] : x[12 + r];
                    Tm[(16 * m + 4 * q4 + r) * CP + 16 * m + li] = (_Float16)v;
                }
            }
        };
        // P3 (wave 4): off-diagonal blocks of T by MFMA doubling, then the T fragments into slot s
        auto phase3 = [&](int s) __attribute__((always_inline)) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            // level 1: T_ul = -T_uu A_ul T_ll for (l, u) = (0, 1) and (2, 3)
#pragma unroll
            for (int pr = 0; pr < NT / 2; ++pr) {
                const int lo = 2 * pr, up = 2 * pr + 1;
                f16x4 btl;
#pragma unroll
                for (int e = 0; e < 4; ++e) btl[e] = Tm[(16 * lo + 4 * q4 + e) * CP + 16 * lo + li];
                const f32x4 pm = mfma16x16x16(ld4h(Ah + (16 * up + li) * CP + 16 * lo + 4 * q4), btl, z);
                const f32x4 out = mfma16x16x16(ld4h(Tm + (16 * up + li) * CP + 16 * up + 4 * q4), to_f16x4(-pm), z);
#pragma unroll
                for (int r = 0; r < 4; ++r) Tm[(16 * up + 4 * q4 + r) * CP + 16 * lo + li] = (_Float16)out[r];
            }
            if constexpr (NT == 4) {
                // level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32], column block jc
#pragma unroll
                for (int jc = 0; jc < 2; ++jc) {
                    f16x4 t0j, t1j;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        t0j[e] = Tm[(4 * q4 + e) * CP + 16 * jc + li];
                        t1j[e] = Tm[(16 + 4 * q4 + e) * CP + 16 * jc + li];
                    }
                    f32x4 p0 = mfma16x16x16(ld4h(Ah + (32 + li) * CP + 16 + 4 * q4), t1j, z);
                    f32x4 p1 = mfma16x16x16(ld4h(Ah + (48 + li) * CP + 16 + 4 * q4), t1j, z);
                    if (jc == 0) {
                        p0 = mfma16x16x16(ld4h(Ah + (32 + li) * CP + 4 * q4), t0j, p0);
                        p1 = mfma16x16x16(ld4h(Ah + (48 + li) * CP + 4 * q4), t0j, p1);
                    }
                    const f16x4 b0 = to_f16x4(-p0), b1 = to_f16x4(-p1);
                    const f32x4 o0 = mfma16x16x16(ld4h(Tm + (32 + li) * CP + 32 + 4 * q4), b0, z);
                    f32x4 o1 = mfma16x16x16(ld4h(Tm + (48 + li) * CP + 32 + 4 * q4), b0, z);
                    o1 = mfma16x16x16(ld4h(Tm + (48 + li) * CP + 48 + 4 * q4), b1, o1);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Tm[(32 + 4 * q4 + r) * CP + 16 * jc + li] = (_Float16)o0[r];
                        Tm[(48 + 4 * q4 + r) * CP + 16 * jc + li] = (_Float16)o1[r];
                    }
                }
            }
            // T fragments: tile mm, k block kb: lane (q4, li) holds row 16 mm + li at columns
            // frag_col(kb, q4, 0..7)
#pragma unroll
            for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                for (int kb = 0; kb <= mm / 2; ++kb) {
                    const _Float16 *src = Tm + (16 * mm + li) * CP + 32 * kb + 4 * q4;
                    *reinterpret_cast<f16x8 *>(smem + L::oT + s * L::kFr * 1024 + fblk(mm, kb) * 1024 + lane * 16) =
                        cat(ld4h(src), ld4h(src + 16));
                }
        };

        // prologue: chunk 0 of the segment into slot 0
        float g0 = 0.f, b0 = 0.f;
        if (n > 0) {
            issue(cb);
            phase1(cb, 0);
            g0 = graw;
            b0 = braw;
            if (n > 1) issue(cb + 1);
        }
        lds_barrier();
        if (n > 0) phase2(cb, 0, g0, b0);
        lds_barrier();
        if (n > 0 && m == 0) phase3(0);
        lds_barrier();

        auto interval = [&](auto sl, int i) __attribute__((always_inline)) {
            constexpr int s1 = 1 - decltype(sl)::value;  // slot of chunk i + 1
            const int c1 = cb + i + 1;
            float g1 = 0.f, b1 = 0.f;
            if (i + 1 < n) {
                phase1(c1, s1);
                g1 = graw;
                b1 = braw;
                if (i + 2 < n) issue(c1 + 1);
            }
            lds_barrier();  // b1
            if (i + 1 < n) phase2(c1, s1, g1, b1);
            lds_barrier();  // b2
            if (i + 1 < n && m == 0) phase3(s1);
            lds_barrier();  // b3
        };
        for (int i = 0; i < n; i += 2) {
            interval(IC<0>{}, i);
            if (i + 1 < n) interval(IC<1>{}, i + 1);
        }
    }
}

// S_{p+1} = S_p M_p + N_p for p = 1 .. P-2, one workgroup per (pair, block of 16 rows), fp32.
// Thread (r, cg) owns row r of the block, columns 8 cg .. 8 cg + 7; M_p is staged through LDS
// in halves of 64 rows.
__global__ __launch_bounds__(256) void gdn_seg_combine_kernel(SegParams sp) {
    __shared__ __attribute__((aligned(16))) float srow[16][kD + 4];
    __shared__ __attribute__((aligned(16))) float mt[kD / 2][kD];
    const int pair = blockIdx.x >> 3, rb = blockIdx.x & 7;
    const int tid = threadIdx.x, r = tid >> 4, cg = tid & 15;
    const int64_t base = (int64_t)pair * sp.P;
    const float *s1 = sp.ws_start + (base + 1) * (kD * kD) + rb * 16 * kD;
    for (int e = tid; e < 16 * kD; e += 256) srow[e / kD][e % kD] = s1[e];
    for (int seg = 1; seg + 1 < sp.P; ++seg) {
        const float *M = sp.ws_m + (base + seg) * (kD * kD);
        const float *N = sp.ws_n + (base + seg) * (kD * kD) + rb * 16 * kD;
        float *Sn = sp.ws_start + (base + seg + 1) * (kD * kD) + rb * 16 * kD;
        f32x4 a0 = *reinterpret_cast<const f32x4 *>(N + r * kD + 8 * cg);
        f32x4 a1 = *reinterpret_cast<const f32x4 *>(N + r * kD + 8 * cg + 4);
        for (int half = 0; half < 2; ++half) {
            __syncthreads();  // srow written; earlier reads of mt done
            for (int e = tid; e < kD * kD / 8; e += 256)
                reinterpret_cast<f32x4 *>(&mt[0][0])[e] =
                    reinterpret_cast<const f32x4 *>(M + half * (kD / 2) * kD)[e];
            __syncthreads();
#pragma unroll 8
            for (int k = 0; k < kD / 2; ++k) {
                const float sv = srow[r][half * (kD / 2) + k];
                a0 += sv * *reinterpret_cast<const f32x4 *>(&mt[k][8 * cg]);
                a1 += sv * *reinterpret_cast<const f32x4 *>(&mt[k][8 * cg + 4]);
            }
        }
        *reinterpret_cast<f32x4 *>(Sn + r * kD + 8 * cg) = a0;
        *reinterpret_cast<f32x4 *>(Sn + r * kD + 8 * cg + 4) = a1;
        __syncthreads();  // every read of srow done
        *reinterpret_cast<f32x4 *>(&srow[r][8 * cg]) = a0;
        *reinterpret_cast<f32x4 *>(&srow[r][8 * cg + 4]) = a1;
    }
}

// T = 0: the final state is the initial state (converted to its storage type), or zero.
__global__ __launch_bounds__(256) void gdn_state_copy_kernel(PrefillParams p, int64_t count) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= count) return;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (p.init_state) x = load_state4(p.init_state, i, p.init_f16);
    store_state4(p.final_state, i, x, p.final_f16);
}

template <int C, bool OUT>
hipError_t launch_pass(const SegParams &sp, int64_t nblocks, hipStream_t stream) {
    const size_t bytes = SegSmem<C, OUT>::kBytes;
    static bool attr_set = false;  // the attribute is a property of the function: set once
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_seg_pass_kernel<C, OUT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    if (nblocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gdn_seg_pass_kernel<C, OUT>), dim3((unsigned)nblocks), dim3(kSegThreads), bytes, stream, sp);
    return hipGetLastError();
}

template <int C>
hipError_t launch_seg_c(const SegParams &sp, hipStream_t stream) {
    const int64_t pairs = (int64_t)sp.p.B * sp.p.Hv;
    hipError_t err = hipSuccess;
    if (sp.P > 1) {
        err = launch_pass<C, false>(sp, pairs * (2 * sp.P - 3), stream);
        if (err != hipSuccess) return err;
        if (sp.P > 2) {
            hipLaunchKernelGGL(gdn_seg_combine_kernel, dim3((unsigned)(pairs * 8)), dim3(256), 0, stream, sp);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    }
    return launch_pass<C, true>(sp, pairs * sp.P, stream);
}

}  // namespace

int64_t seg_workspace_bytes(int64_t pairs, int P) { return P > 1 ? 3 * pairs * P * kD * kD * 4 : 0; }

int seg_count(int64_t B, int64_t Hv, int64_t T, int chunk, size_t workspace_bytes, bool have_workspace) {
    if (T <= 0) return 1;
    const int64_t nc = (T + chunk - 1) / chunk;
    const int64_t pairs = B * Hv;
    // enough segments to give every CU of the GPU a workgroup in the output pass
    int64_t P = (256 + pairs - 1) / pairs;
    if (P > nc) P = nc;
    if (P > 64) P = 64;
    if (P < 1) P = 1;
    while (P > 1 && (!have_workspace || (size_t)seg_workspace_bytes(pairs, (int)P) > workspace_bytes)) --P;
    // equal chunk counts per segment, none empty
    const int64_t per = (nc + P - 1) / P;
    return (int)((nc + per - 1) / per);
}

hipError_t launch_prefill_seg(const PrefillParams &p, int chunk, int P, void *ws, hipStream_t stream) {
    if (p.D != kD) return hipErrorInvalidValue;
    if (p.T == 0) {
        if (!p.final_state) return hipSuccess;
        const int64_t count = (int64_t)p.B * p.Hv * kD * kD;
        hipLaunchKernelGGL(gdn_state_copy_kernel, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, stream, p,
                           count);
        return hipGetLastError();
    }
    SegParams sp;
    sp.p = p;
    sp.P = P;
    const int64_t nc = (p.T + chunk - 1) / chunk;
    sp.seg_chunks = (int32_t)((nc + P - 1) / P);
    const int64_t pairs = (int64_t)p.B * p.Hv;
    float *w = static_cast<float *>(ws);
    sp.ws_start = w;
    sp.ws_n = w + pairs * P * kD * kD;
    sp.ws_m = w + 2 * pairs * P * kD * kD;
    switch (chunk) {
        case 32: return launch_seg_c<32>(sp, stream);
        case 64: return launch_seg_c<64>(sp, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
