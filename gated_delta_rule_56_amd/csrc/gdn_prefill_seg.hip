// Segmented bf16 prefill: the chunks of one sequence are cut into P segments that
// run in parallel, each workgroup holding all dv = 128 rows of the state of one
// (b, value head, segment), with the chunk preparation fused in.
//
// Chunked WY form, per chunk of C tokens with start state S (dv x dk), local t:
//   G_t = sum_{s<=t} g_s,  Gamma_ts = exp(G_t - G_s) (s <= t)
//   A = strict_lower(diag(beta) (K K^T o Gamma))
//   X = K S^T,  R = diag(beta) V - diag(beta gamma) X,  U solves (I + A) U = R
//   O = diag(gamma) (scale Q S^T) + lower_incl(scale Q K^T o Gamma) U
//   S <- gamma_C S + (diag(exp(G_C - G)) U)^T K
// (of S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t scale q_t; the state update and the output taken from the updated
// state are those of the gated-delta reference tests on the "27b 935/47" compare
// page; padded steps with beta = 0, g = 0 are exact no-ops, the symbolic-length
// prefill entry of the "mergable fast RDNA3 Qwen 3.6" commit log).
//
// The unit-lower system is solved in 16-token blocks, U_m = T_mm (R_m - sum_{j<m} A_mj U_j)
// with T_mm = (I + A_mm)^{-1}: the 16 x 16 diagonal inverses and the blocks of A below them
// are all the chunk preparation has to deliver (the block form of the forward substitution
// in the tinygrad helper inverse_unit_lower, compare page "27b 935/47", llm/kernels/generic.py).
//
// The chunk update is affine in the start state: S_new = S M_c + N_c. A segment
// of chunks therefore maps its start S_p to S_p M_p + N_p, with N_p the end state
// from a zero start and M_p the end "state" of the identity run with v = 0 (each
// identity row is a state row; rows never mix). Three launches:
//   1. map pass (OUT = false): segment 0 from the initial state (its end is the
//      true start of segment 1), and for segments 1 .. P-2 both N_p (role 0) and
//      M_p (role 1). One workgroup per (pair, segment) holds both row sets over
//      one shared chunk preparation, at 32-token chunks (16 at chunk 16; the
//      64-token call's segments are whole 32-token chunks too);
//   2. combine: S_{p+1} = S_p M_p + N_p, sequential over the segments, in fp32;
//   3. output pass (OUT = true): every segment from its true start, writing o and,
//      in the last segment, the final state.
// With P = 1 only the output pass runs.
//
// Workgroup of 8 waves (wave i on SIMD i % 4), two barriers per chunk (the map pass:
// 12 waves, row waves 0-3 for the zero-start rows, 4-7 for the identity
// rows, preparation waves 8-11):
//   waves 0-3, "row waves": state rows 32 w .. 32 w + 31 as two 16-row MFMA blocks
//     held in registers for the whole segment; per chunk X and (OUT) Y = S Q^T before
//     the first barrier, then R, U, O^T and the update. Every operand of chunk i is in
//     LDS slot i & 1 when the chunk starts; LDS operands are requested in batches one
//     batch ahead of the MFMAs that use them.
//   waves 4-7 (8-11), "prep waves", token tile m: prepare chunk i + 1 into slot
//     (i + 1) & 1 during chunk i. Before the first barrier (P1) each converts its
//     16 raw bf16 k and q rows (loaded one chunk earlier into registers) to the fp16
//     tiles and stores its v rows, one prep wave also forms the gate vectors (the
//     fourth when the chunk has fewer than four tiles, so one with none), and each
//     issues the loads of chunk i + 2; after it (P2) each forms K K^T and Q K^T of
//     its tile against the tiles at or before it on MFMA, the gated blocks of A
//     and A_qk, and the inverse of its diagonal block row by row (at 32-token
//     chunks the third prep wave takes the tile below the diagonal). No prep wave
//     waits for another.
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
// threads of a segment-pass workgroup: 4 row waves and 4 preparation waves, or in the map pass
// 8 row waves (the zero-start rows and the identity rows of one segment) and 4
// preparation waves
template <bool OUT, bool KDA>
__host__ __device__ constexpr int seg_threads() { return (!OUT ? 12 : 8) * 64; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fragment block of token tile m, k block kb (kb <= m / 2), counted over the blocks on or
// below the diagonal: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__host__ __device__ constexpr int fblk(int m, int kb) { return m + (m > 2 ? m - 2 : 0) + kb; }
// 16 x 16 block (m, j), j < m, of A below the diagonal: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__host__ __device__ constexpr int ablk(int m, int j) { return m * (m - 1) / 2 + j; }

// channel vectors of a chunk (KDA; r0 = token 7, r1 = token 23, b = token 15, the last of tile 0,
// C - 1 = token 31)
constexpr int kVecR0 = 0;   // e^{G_r0}
constexpr int kVecR1 = 1;   // e^{G_r1}
constexpr int kVecCR0 = 2;  // e^{G_C-1 - G_r0}
constexpr int kVecCR1 = 3;  // e^{G_C-1 - G_r1}
constexpr int kVecR1B = 4;  // e^{G_r1 - G_b}
constexpr int kVecBR0 = 5;  // e^{G_b - G_r0}
constexpr int kVecC = 6;    // e^{G_C-1}
constexpr int kNVec = 7;
// the chunked per-channel-decay form takes log-decays below this as this: every factor of its
// diagonal-block products then lies within e^{+-80}
constexpr float kKdaGMin = -10.0f;

template <int C, bool OUT, bool NORM = false, bool KDA = false>
struct SegSmem {
    static constexpr int NT = C / 16, KBC = C / 32;
    static constexpr int kFr = fblk(NT - 1, (NT - 1) / 2) + 1;   // A_qk fragment blocks
    static constexpr int kNA = NT * (NT - 1) / 2;                // blocks of A below the diagonal
    static constexpr size_t kTile = (size_t)C * 256;             // C x 128 16-bit values
    static constexpr size_t oK = 0;                              // [2] fp16 k tiles
    static constexpr size_t oQ = oK + 2 * kTile;                 // [2] fp16 q tiles (OUT)
    static constexpr size_t oV = oQ + (OUT ? 2 * kTile : 0);     // [2] bf16 v tiles
    static constexpr size_t oA = oV + 2 * kTile;                 // [2][kFr][64] x 16 B A_qk fragments (OUT)
    static constexpr size_t oNA = oA + (OUT ? 2 * kFr * 1024 : 0);  // [2][kNA][64] x 8 B: -A blocks
    static constexpr size_t oTd = oNA + 2 * kNA * 512;           // [2][NT][2][64] x 8 B: T_mm, diag(exp(G_C-G)) T_mm
    static constexpr size_t oG = oTd + 2 * NT * 1024;             // [2][5][C] f32: gamma, beta, exp(G_C-G), beta gamma, G
    static constexpr size_t oAt = oG + 2 * 20 * C;               // f32 [NT][16][20]: diagonal blocks of A, transposed
    // per-channel decay (KDA): [2] k o e^{G_C - G} tiles (read transposed by the state update);
    // the raw k and q tiles of the chunk being prepared (fp16, for the block products); [2]
    // factors E[t][c] = e^{G_tc - G_rc}, r the 8th token of t's 16-token tile, f32 rows padded to
    // 528 B; [2][kNVec][128] f32 channel vectors (kVec*); [2][128] f32 e^{G_C} for the row waves
    static constexpr size_t kERow = 528;
    static constexpr size_t oKT = oAt + NT * 16 * 20 * 4;
    static constexpr size_t oRK = oKT + (KDA ? 2 * kTile : 0);
    static constexpr size_t oRQ = oRK + (KDA ? kTile : 0);
    static constexpr size_t oE = oRQ + (KDA && OUT ? kTile : 0);
    static constexpr size_t oEV = oE + (KDA ? 2 * C * kERow : 0);
    static constexpr size_t oEC = oEV + (KDA ? 2 * kNVec * 512 : 0);
    // output norm (NORM): a chunk's un-normalised o rows in fp16, each lane's 8 values scaled
    // by a power of two taken from their own sum of squares (stage_scale), rows padded to 272 B
    // so that the 8-byte accesses of 32 lanes (16 tokens, two column groups) meet all 64 banks;
    // the partial sums of squares [C][20] f32 (16 used: 4 row waves x 4 lanes of 8 columns);
    // the norm weight [128] f32
    // per-channel-decay output pass: the second channel half of the blocks (1,0) of -A ([2][64] x
    // 8 B) and of A_qk ([2][64] x 16 B, the fragment's first half; the second is zero)
    static constexpr size_t oNA2 = oEC + (KDA ? 2 * 512 : 0);
    static constexpr size_t oAQ2 = oNA2 + (KDA && OUT ? 2 * 512 : 0);
    // the map pass: a zero v tile read by the identity rows
    static constexpr size_t oZV = oAQ2 + (KDA && OUT ? 2 * 1024 : 0);
    static constexpr size_t oNO = oZV + (!OUT ? kTile : 0);
    static constexpr size_t oNP = oNO + (NORM ? (size_t)C * 272 : 0);
    static constexpr size_t oNW = oNP + (NORM ? (size_t)C * 80 : 0);
    static constexpr size_t kBytes = oNW + (NORM ? 512 : 0);
    static_assert(!NORM || OUT, "the norm belongs to the output pass");
    static_assert(!KDA || (C == 32 && !NORM), "the per-channel decay runs at C = 32, without the norm");
    static_assert(oQ % 16 == 0 && oV % 16 == 0 && oA % 16 == 0 && oNA % 16 == 0 && oTd % 16 == 0 &&
                      oG % 16 == 0 && oAt % 16 == 0 && oKT % 16 == 0 && oRK % 16 == 0 && oRQ % 16 == 0 &&
                      oE % 16 == 0 && oEV % 16 == 0 && oEC % 16 == 0 && oNA2 % 16 == 0 && oAQ2 % 16 == 0 && oZV % 16 == 0 && oNO % 16 == 0 && oNP % 16 == 0 &&
                      oNW % 16 == 0,
                  "alignment");
    static_assert(kBytes <= 160 * 1024, "LDS");
};


__device__ __forceinline__ f16x8 ld8(const unsigned char *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ f16x4 ld4(const unsigned char *p) { return *reinterpret_cast<const f16x4 *>(p); }
__device__ __forceinline__ f32x4 ldf4(const unsigned char *p) { return *reinterpret_cast<const f32x4 *>(p); }

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
// The gate vectors of a chunk into its LDS slot, lane = token: G = inclusive prefix of g over
// the chunk, gamma = e^G, beta, e^{G_C - G}, beta gamma, G ([5][C] float32). Tokens past the
// end come in with g = beta = 0.
template <int C>
__device__ __forceinline__ void form_gates(unsigned char *slot, float gv, float bv, int lane);

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// keeps the compiler from moving instructions across this point (so that a batch of LDS
// reads is issued before the MFMAs of the previous batch)
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

template <int N>
using IC = std::integral_constant<int, N>;

// bf16 -> fp16 for 4 values (exact within fp16 range)
__device__ __forceinline__ f16x4 bf4_to_h4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
    return f16x4{(_Float16)bf16_bits_to_f32(a), (_Float16)bf16_bits_to_f32(b), (_Float16)bf16_bits_to_f32(c),
                 (_Float16)bf16_bits_to_f32(d)};
}

// DPP-modified copy of x (ctrl: the DPP control; rows outside row_mask, and with bound_ctrl
// lanes whose source is out of range, read 0)
template <int ctrl, int row_mask, bool bound_ctrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, row_mask, 0xF, bound_ctrl));
}

// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each row of 16 lanes, then
// the last lane of row 0 (2) broadcast into row 1 (3), then lane 31 into rows 2 and 3
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_f<0x111, 0xF, true>(x);   // row_shr:1
    x += dpp_f<0x112, 0xF, true>(x);   // row_shr:2
    x += dpp_f<0x114, 0xF, true>(x);   // row_shr:4
    x += dpp_f<0x118, 0xF, true>(x);   // row_shr:8
    x += dpp_f<0x142, 0xA, false>(x);  // row_bcast:15
    x += dpp_f<0x143, 0xC, false>(x);  // row_bcast:31
    return x;
}

// T = (I + A)^{-1} for a strictly lower 16 x 16 A, by forward substitution over the rows,
// T[r][c] = [r == c] - sum_{k<r} A[r][k] T[k][c]: lane (q, i) holds nrow = -A[i][0..15] and
// builds t[e] = T[i][4 q + e], the A-operand fragment of a 16 x 16 x 16 product. Step k adds
// nrow[k] times the finished row k, read from lane k of each row of 16 lanes by a DPP
// row_newbcast operand of the multiply-add itself (one instruction per element and step). DPP
// reads a VGPR that a VALU instruction wrote at least two instructions earlier: s_nop 1 covers
// the writes before the block, and inside it each t[e] is read three instructions after its
// last write.
__device__ __forceinline__ void inv_rows(f32x4 &t, const float (&nrow)[16]) {
    float t0 = t[0], t1 = t[1], t2 = t[2], t3 = t[3];
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3)
        : "v"(nrow[0]), "v"(nrow[1]), "v"(nrow[2]), "v"(nrow[3]), "v"(nrow[4]), "v"(nrow[5]), "v"(nrow[6]),
          "v"(nrow[7]), "v"(nrow[8]), "v"(nrow[9]), "v"(nrow[10]), "v"(nrow[11]), "v"(nrow[12]), "v"(nrow[13]),
          "v"(nrow[14]));
    t = f32x4{t0, t1, t2, t3};
}

// Power-of-two factor 2^(14 - floor(e / 2)), e the binary exponent of ss >= 0 (its biased
// exponent field minus 127, so 0 and subnormal sums give e = -127), and its inverse. With ss
// the sum of squares of a few values, every value times the factor has magnitude below 2^15:
// in float16 range, and rounded to 11 significant bits whatever the values' own magnitude.
__device__ __forceinline__ float stage_scale(float ss) {
    const int h = ((int)((__float_as_uint(ss) >> 23) & 0xff) - 127) >> 1;
    return __uint_as_float((uint32_t)(127 + 14 - h) << 23);
}
__device__ __forceinline__ float stage_unscale(float ss) {
    const int h = ((int)((__float_as_uint(ss) >> 23) & 0xff) - 127) >> 1;
    return __uint_as_float((uint32_t)(127 - 14 + h) << 23);
}

template <int C>
__device__ __forceinline__ void form_gates(unsigned char *slot, float gv, float bv, int lane) {
    const float G = wave_prefix_sum(gv);
    const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), C - 1));
    if (lane < C) {
        float *gts = reinterpret_cast<float *>(slot);
        const float gam = __expf(G);
        gts[lane] = gam;
        gts[C + lane] = bv;
        gts[2 * C + lane] = __expf(gC - G);
        gts[3 * C + lane] = bv * gam;
        gts[4 * C + lane] = G;
    }
}

// NORM: 0 no output norm, 1 the norm without a gate, 2 with a gate. KDA: one log-decay per key
// channel (g [B][Hv][T][dk]), C = 32.
template <int C, bool OUT, int NORM = 0, bool KDA = false>
__global__ __launch_bounds__((seg_threads<OUT, KDA>()), 1) void gdn_seg_pass_kernel(SegParams sp) {
    using L = SegSmem<C, OUT, (NORM > 0), KDA>;
    constexpr int NT = L::NT, KBC = L::KBC;
    // map pass: one workgroup per (pair, segment) runs both the zero-start rows
    // (waves 0-3, with v) and the identity rows (waves 4-7, v = 0) on one shared chunk
    // preparation (waves 8-11)
    constexpr bool kMerge = !OUT;
    constexpr int kRowW = kMerge ? 8 : 4;
    // three waves per SIMD leave each 168 VGPRs: the merged map pass runs 32- and 16-token chunks
    static_assert(!kMerge || C <= 32, "the merged map pass runs at C <= 32");
    // the preparation wave that forms the gate vectors: one without a tile of its own when the
    // chunk has fewer than four 16-token tiles
    constexpr int kScanW = L::NT < 4 ? 3 : 0;
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
        bool init_f16, final_f16, o_f16, state_bf16;
        const float *norm_w;
        const uint16_t *norm_gate;
        float norm_eps;
    };
    const Args p = {sp.p.q, sp.p.k, sp.p.v, sp.p.init_state, sp.p.g, sp.p.beta, sp.p.o, sp.p.final_state,
                    sp.ws_start, sp.ws_n, sp.ws_m, sp.p.B, sp.p.T, sp.p.Hk, sp.p.Hv, sp.p.Ts, sp.p.head_map,
                    sp.P, sp.seg_chunks, sp.p.scale, sp.p.init_f16, sp.p.final_f16, sp.p.o_f16, sp.p.state_bf16,
                    sp.p.norm_w, static_cast<const uint16_t *>(sp.p.norm_gate), sp.p.norm_eps};

    // ---- workgroup -> (b, key head, unit, value head of the key head). Consecutive indices
    // share the key head's k and q and sit on one XCD (workgroups go round-robin over 8 XCDs).
    const int nb = gridDim.x;
    int lin = blockIdx.x;
    if ((nb & 7) == 0) lin = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
    const int ratio = p.Hv / p.Hk;
    const int jj = lin % ratio;
    int rest = lin / ratio;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // segments: all P in the output pass, all but the last in the map pass
    const int nseg = OUT ? p.P : p.P - 1;
    const int seg = rest % nseg;
    rest /= nseg;
    // role of a row wave: 0 state rows (from the start state, with v), 1 identity rows (v = 0)
    const int role = (kMerge && (w >> 2) == 1) ? 1 : 0;
    const int kh = rest % p.Hk, b = rest / p.Hk;
    const int h = p.head_map == 0 ? kh + jj * p.Hk : kh * ratio + jj;
    const int pair = b * p.Hv + h;

    const int T = p.T;
    const int NC = (T + C - 1) / C;
    const int cb = seg * p.seg_chunks;
    const int n = max(0, min(NC, cb + p.seg_chunks) - cb);  // chunks of this segment
    const int64_t ktok = ((int64_t)b * p.Hk + kh) * p.Ts;     // first token row of q, k
    const int64_t vtok = (int64_t)pair * p.Ts;                // first token row of v, g, beta, o
    const int64_t wsi = ((int64_t)pair * p.P + seg) * (kD * kD);

    const int tid = threadIdx.x, lane = tid & 63;
    const int li = lane & 15, q4 = lane >> 4;

    if (w < kRowW) {
        // ================================================================ row waves
        const int wr = w & 3;  // row block of this wave
        // S[bb][jt][r] = state[r0 + li][16 jt + 4 q4 + r], r0 = 32 wr + 16 bb
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
                const int r0 = 32 * wr + 16 * bb;
                const int64_t srow = ws_layout ? (int64_t)(r0 + li) * kD + 4 * q4
                                               : ((int64_t)pair * kD + r0 + li) * kD + 4 * q4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) {
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
                    if (!OUT && role == 1) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = (16 * jt + 4 * q4 + r == r0 + li) ? 1.0f : 0.0f;
                    } else if (src) {
                        x = load_state4(src, srow + 16 * jt, f16, p.state_bf16);
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
                const int64_t wrow = (int64_t)(32 * wr + 16 * bb + li) * kD + 4 * q4;
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
        // the identity rows read v = 0 from a zero tile, written once (visible after the setup
        // barriers); the zero-start rows read the preparation waves' v tiles
        if constexpr (kMerge) {
            if (role == 1) {
                for (int o = (tid - 256) * 16; o < (int)L::kTile; o += 256 * 16)
                    *reinterpret_cast<u16x8 *>(smem + L::oZV + o) = u16x8{};
            }
        }
        const int voff = (kMerge && role == 1) ? (int)L::oZV : (int)L::oV;
        const int vstep = (kMerge && role == 1) ? 0 : (int)L::kTile;

        // per-lane LDS offsets (slot, tile and block offsets are immediates)
        int xo[4];  // k / q tile: row li, group 4 kb + q4
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) xo[kb] = li * 256 + (((4 * kb + q4) ^ ksw(li)) << 4);
        int ta[8];  // k tile read transposed: column tile jt of the update
        {
            const int rt = 4 * q4 + (li >> 2);
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                const int g = 4 * (jt >> 1) + (li & 3);
                ta[jt] = rt * 256 + ((g ^ ksw(rt)) << 4) + (jt & 1) * 8;
            }
        }
        int va[2];  // v tile read transposed: tokens 4 q4 + (li >> 2), columns r0 + 4 (li & 3)
        {
            const int rt = 4 * q4 + (li >> 2);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int c = 32 * wr + 16 * bb + 4 * (li & 3);
                va[bb] = rt * 256 + (((c >> 3) ^ ksw(rt)) << 4) + (c & 7) * 2;
            }
        }
        float *o_f32 = static_cast<float *>(p.o);
        _Float16 *o_f16 = static_cast<_Float16 *>(p.o);

        // output norm: the weight into LDS for the prep waves (visible after the setup barriers);
        // store_normed writes this lane's 8 normalised values of token row tok (of the pair) from
        // their float16 staging slot xo
        if constexpr (NORM > 0) {
            if (w == 0 && lane < kD / 4)
                *reinterpret_cast<f32x4 *>(smem + L::oNW + 16 * lane) = *reinterpret_cast<const f32x4 *>(p.norm_w + 4 * lane);
        }
        auto store_normed = [&](const unsigned char *xo, int64_t tok) __attribute__((always_inline)) {
            const f16x4 y0 = ld4(xo), y1 = ld4(xo + 32);
            const int64_t row = (vtok + tok) * kD + 32 * wr + 4 * q4;
            if (p.o_f16) {
                *reinterpret_cast<f16x4 *>(o_f16 + row) = y0;
                *reinterpret_cast<f16x4 *>(o_f16 + row + 16) = y1;
            } else {
                *reinterpret_cast<f32x4 *>(o_f32 + row) = f32x4{(float)y0[0], (float)y0[1], (float)y0[2], (float)y0[3]};
                *reinterpret_cast<f32x4 *>(o_f32 + row + 16) = f32x4{(float)y1[0], (float)y1[1], (float)y1[2], (float)y1[3]};
            }
        };

        lds_barrier();
        lds_barrier();
        if constexpr (KDA) lds_barrier();  // the preparation waves' first factors

        auto interval = [&](auto sl, int i) __attribute__((always_inline)) {
            constexpr int s = decltype(sl)::value;
            const unsigned char *Kt = smem + L::oK + s * L::kTile;
            const unsigned char *Qt = smem + L::oQ + s * L::kTile;
            const unsigned char *Vt = smem + voff + s * vstep;
            const unsigned char *gt = smem + L::oG + s * 20 * C;  // gate vectors of this chunk
            const unsigned char *na = smem + L::oNA + s * L::kNA * 512 + lane * 8;
            const unsigned char *td = smem + L::oTd + s * 2 * NT * 512 + lane * 8;
            const unsigned char *aq = smem + L::oA + s * L::kFr * 1024 + lane * 16;

            // ---- X = K S^T and (OUT) Y^T = S Q^T, k block by k block: the fragments of block
            // kb + 1 are requested before the products of block kb
            f32x4 X[2][NT], Y[2][NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) X[0][m] = X[1][m] = Y[0][m] = Y[1][m] = f32x4{0.f, 0.f, 0.f, 0.f};
            f16x8 kf[2][NT], qf[2][NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                kf[0][m] = ld8(Kt + xo[0] + m * 4096);
                if (OUT) qf[0][m] = ld8(Qt + xo[0] + m * 4096);
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cur = kb & 1, nxt = cur ^ 1;
                if (kb + 1 < 4) {
#pragma unroll
                    for (int m = 0; m < NT; ++m) {
                        kf[nxt][m] = ld8(Kt + xo[kb + 1] + m * 4096);
                        if (OUT) qf[nxt][m] = ld8(Qt + xo[kb + 1] + m * 4096);
                    }
                }
                fence();
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    X[0][m] = mfma16x16x32(kf[cur][m], sb[0][kb], X[0][m]);
                    X[1][m] = mfma16x16x32(kf[cur][m], sb[1][kb], X[1][m]);
                }
                if constexpr (OUT) {
#pragma unroll
                    for (int m = 0; m < NT; ++m) {
                        Y[0][m] = mfma16x16x32(sb[0][kb], qf[cur][m], Y[0][m]);
                        Y[1][m] = mfma16x16x32(sb[1][kb], qf[cur][m], Y[1][m]);
                    }
                }
                fence();
            }
            // ---- operands of the rest of the chunk: v (transposed), the gate vectors, the diagonal
            // inverses and -A blocks, the A_qk fragments. They are this chunk's slot, complete since
            // the last b2, so where the registers allow (all but the 64-token output pass) they are
            // requested before b1, to arrive while the preparation waves finish and ahead of their
            // post-b1 traffic
            constexpr bool kEarly = !OUT || C < 64;
            s16x4 vraw[2][NT];
            f32x4 bt[NT], bg[NT];
            f16x4 tdf[NT], tef[NT], naf[L::kNA > 0 ? L::kNA : 1];
            f16x8 aqf[L::kFr];
            float gam[NT];
            // per-channel-decay output pass: the blocks (1,0) of -A and A_qk come in two channel
            // halves, the second added by one more product each
            constexpr bool kSplitOff = KDA && OUT;
            f16x4 naf2;
            f16x8 aqf2;
            auto request_rest = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    vraw[0][m] = ld_tr_raw(Vt + va[0] + m * 4096);
                    vraw[1][m] = ld_tr_raw(Vt + va[1] + m * 4096);
                    bt[m] = ldf4(gt + 4 * C + 64 * m + 16 * q4);
                    bg[m] = ldf4(gt + 12 * C + 64 * m + 16 * q4);
                    tdf[m] = ld4(td + m * 1024);
                    tef[m] = ld4(td + m * 1024 + 512);
                }
#pragma unroll
                for (int e = 0; e < L::kNA; ++e) naf[e] = ld4(na + e * 512);
                if constexpr (kSplitOff) naf2 = ld4(smem + L::oNA2 + s * 512 + lane * 8);
            };
            auto request_aq = [&]() __attribute__((always_inline)) {
                if constexpr (OUT) {
#pragma unroll
                    for (int f = 0; f < L::kFr; ++f) aqf[f] = ld8(aq + f * 1024);
#pragma unroll
                    for (int m = 0; m < NT; ++m) gam[m] = *reinterpret_cast<const float *>(gt + 4 * (16 * m + li));
                    if constexpr (kSplitOff) aqf2 = ld8(smem + L::oAQ2 + s * 1024 + lane * 16);
                }
            };
            if constexpr (kEarly) {
                request_rest();
                request_aq();
                fence();
            }
            lds_barrier();  // b1: the prep waves' rows of chunk i + 1 are in place
            // issue priority to the waves on the critical path: in the output pass, the row waves
            // from here to the end of the interval (the preparation waves before b1)
            if constexpr (OUT && !KDA) __builtin_amdgcn_s_setprio(2);
            if constexpr (!kEarly) {
                request_rest();
                fence();
            }
            // R = beta V - beta gamma X  (v: tokens 16 m + 4 q4 + r, column r0 + li)
            f32x4 R[2][NT];
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    f32x4 vv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) vv[r] = bf16_bits_to_f32((uint16_t)vraw[bb][m][r]);
                    R[bb][m] = bt[m] * vv - bg[m] * X[bb][m];
                }
            if constexpr (!kEarly) request_aq();  // after R, as its registers free
            fence();
            // ---- U_m = T_mm (R_m - sum_{j<m} A_mj U_j), the two row blocks interleaved, and the
            // update's values diag(exp(G_C - G)) U_m from the scaled inverse
            f16x4 uh[2][NT], ue[2][NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                f32x4 a0 = R[0][m], a1 = R[1][m];
#pragma unroll
                for (int j = 0; j < m; ++j) {
                    a0 = mfma16x16x16(naf[ablk(m, j)], uh[0][j], a0);
                    a1 = mfma16x16x16(naf[ablk(m, j)], uh[1][j], a1);
                }
                if constexpr (kSplitOff) {
                    if (m == 1) {
                        a0 = mfma16x16x16(naf2, uh[0][0], a0);
                        a1 = mfma16x16x16(naf2, uh[1][0], a1);
                    }
                }
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f16x4 h0 = to_f16x4(a0), h1 = to_f16x4(a1);
                uh[0][m] = to_f16x4(mfma16x16x16(tdf[m], h0, z));
                uh[1][m] = to_f16x4(mfma16x16x16(tdf[m], h1, z));
                ue[0][m] = to_f16x4(mfma16x16x16(tef[m], h0, z));
                ue[1][m] = to_f16x4(mfma16x16x16(tef[m], h1, z));
            }
            // ---- O^T = scale Y^T diag(gamma) + U^T A_qk^T; lane: token 16 m + li,
            // columns r0 + 4 q4 .. + 3
            if constexpr (OUT) {
                f16x8 ua[2][KBC > 0 ? KBC : 1];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) {
                    ua[0][kb] = cat(uh[0][2 * kb], uh[0][2 * kb + 1]);
                    ua[1][kb] = cat(uh[1][2 * kb], uh[1][2 * kb + 1]);
                }
                const int c = cb + i;
                const int ntok = min(C, T - c * C);
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    const float gs = gam[m] * p.scale;
                    f32x4 O0 = gs * Y[0][m], O1 = gs * Y[1][m];
                    if constexpr (C == 16) {
                        // one 16-token tile: the A_qk block is the fragment's first half
                        const f16x4 aq0 = __builtin_shufflevector(aqf[0], aqf[0], 0, 1, 2, 3);
                        O0 = mfma16x16x16(uh[0][0], aq0, O0);
                        O1 = mfma16x16x16(uh[1][0], aq0, O1);
                    } else {
#pragma unroll
                        for (int kb = 0; kb <= m / 2; ++kb) {
                            O0 = mfma16x16x32(ua[0][kb], aqf[fblk(m, kb)], O0);
                            O1 = mfma16x16x32(ua[1][kb], aqf[fblk(m, kb)], O1);
                        }
                        if constexpr (kSplitOff) {
                            if (m == 1) {
                                O0 = mfma16x16x32(ua[0][0], aqf2, O0);
                                O1 = mfma16x16x32(ua[1][0], aqf2, O1);
                            }
                        }
                    }
                    const int t = 16 * m + li;
                    if constexpr (NORM > 0) {
                        unsigned char *xo = smem + L::oNO + t * 272 + 2 * (32 * wr + 4 * q4);
                        if (i > 0) store_normed(xo, (int64_t)(c - 1) * C + t);  // chunk c - 1: all C rows
                        // stage for the prep waves' norm (next interval): this lane's 8 columns
                        // in fp16, scaled, and their sum of squares in fp32
                        float ss = 0.0f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) ss += O0[e] * O0[e] + O1[e] * O1[e];
                        *reinterpret_cast<float *>(smem + L::oNP + t * 80 + 4 * (4 * wr + q4)) = ss;
                        const float sc = stage_scale(ss);
                        *reinterpret_cast<f16x4 *>(xo) = to_f16x4(O0 * sc);
                        *reinterpret_cast<f16x4 *>(xo + 32) = to_f16x4(O1 * sc);
                    } else if (t < ntok) {
                        const int64_t row = (vtok + (int64_t)c * C + t) * kD + 32 * wr + 4 * q4;
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
            // ---- S <- gamma_C S + K^T (diag(exp(G_C - G)) U), k block by k block of tokens
            f16x8 ub[2][KBC > 0 ? KBC : 1];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                ub[0][kb] = cat(ue[0][2 * kb], ue[0][2 * kb + 1]);
                ub[1][kb] = cat(ue[1][2 * kb], ue[1][2 * kb + 1]);
            }
            // per-channel decay: the state's columns decay by e^{G_C} each, and the update reads
            // the k o e^{G_C - G} tile
            const unsigned char *Ku = KDA ? smem + L::oKT + s * L::kTile : Kt;
            if constexpr (KDA) {
                const unsigned char *ec = smem + L::oEC + s * 512 + 16 * q4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) {
                    const f32x4 e = ldf4(ec + 64 * jt);  // columns 16 jt + 4 q4 .. + 3
                    S[0][jt] *= e;
                    S[1][jt] *= e;
                }
            } else {
                const float gC = *reinterpret_cast<const float *>(gt + 4 * (C - 1));
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) {
                    S[0][jt] *= gC;
                    S[1][jt] *= gC;
                }
            }
            if constexpr (C == 16) {
                // one 16-token tile: 16 x 16 x 16 steps over its tokens
                f16x4 kt4[8];
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) kt4[jt] = ld_tr(Ku + ta[jt]);
                fence();
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) {
                    S[0][jt] = mfma16x16x16(kt4[jt], ue[0][0], S[0][jt]);
                    S[1][jt] = mfma16x16x16(kt4[jt], ue[1][0], S[1][jt]);
                }
                fence();
            }
            f16x8 kt[2][8];
            if constexpr (C > 16) {
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) kt[0][jt] = cat(ld_tr(Ku + ta[jt]), ld_tr(Ku + ta[jt] + 4096));
            }
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                const int cur = kb & 1, nxt = cur ^ 1;
                if (kb + 1 < KBC) {
#pragma unroll
                    for (int jt = 0; jt < 8; ++jt)
                        kt[nxt][jt] = cat(ld_tr(Ku + ta[jt] + (kb + 1) * 8192),
                                          ld_tr(Ku + ta[jt] + (kb + 1) * 8192 + 4096));
                }
                fence();
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) {
                    S[0][jt] = mfma16x16x32(kt[cur][jt], ub[0][kb], S[0][jt]);
                    S[1][jt] = mfma16x16x32(kt[cur][jt], ub[1][kb], S[1][jt]);
                }
                fence();
            }
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) sb[bb][kb] = pack8(S[bb][2 * kb], S[bb][2 * kb + 1]);
            if constexpr (OUT && !KDA) __builtin_amdgcn_s_setprio(0);
            lds_barrier();  // b2: chunk i + 1 is prepared
        };
        for (int i = 0; i < n; i += 2) {
            interval(IC<0>{}, i);
            if (i + 1 < n) interval(IC<1>{}, i + 1);
        }
        if constexpr (NORM > 0) {
            lds_barrier();  // the prep waves have normalised the last chunk's rows
            if (n > 0) {
                const int c = cb + n - 1;
                const int ntok = min(C, T - c * C);
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    const int t = 16 * m + li;
                    if (t < ntok) store_normed(smem + L::oNO + t * 272 + 2 * (32 * wr + 4 * q4), (int64_t)c * C + t);
                }
            }
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
            // (the merged map pass's identity rows of segment 0 are not needed)
            if (!(kMerge && seg == 0 && role == 1))
                dst = role == 1 ? p.ws_m + wsi : seg == 0 ? p.ws_start + wsi + kD * kD : p.ws_n + wsi;
        }
        if (dst) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int r0 = 32 * wr + 16 * bb;
                const int64_t srow = ((int64_t)(OUT ? pair * kD : 0) + r0 + li) * kD + 4 * q4;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt) store_state4(dst, srow + 16 * jt, S[bb][jt], f16, p.state_bf16);
            }
        }
    } else {
        // ================================================================ prep waves
        const int m = w - kRowW;  // token tile of this wave
        // issue priority to the waves on the critical path: the preparation waves in the map
        // pass, and before b1 in the output pass (the row waves raise theirs above it after b1)
        __builtin_amdgcn_s_setprio(OUT && !KDA ? 1 : 2);
        const bool tile = m < NT;
        // the map pass at two tiles per chunk: the v rows of tile m - 2 go to waves 2 and 3, which
        // have no k tile of their own
        constexpr bool kVSplit = !OUT && !KDA && NT == 2;
        const int vm = kVSplit ? m - 2 : m;
        const bool vtile = kVSplit ? m >= 2 : tile;
        const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ktok * kD;
        const uint16_t *qg = static_cast<const uint16_t *>(p.q) + ktok * kD;
        const uint16_t *vg = static_cast<const uint16_t *>(p.v) + vtok * kD;
        const float *gg = p.g + vtok;
        const float *bgp = p.beta + vtok;

        // raw rows of tile m of one chunk: register j of lane l holds columns 8 (l % 16) + 0..7 of
        // token 16 m + 4 j + l / 16 (of k, q and v), so that each load instruction reads four whole
        // rows, 1 KB in eight 128-byte lines; the gate wave also holds g and beta of the chunk's token
        // slots (lane = slot; one pair per ring slot). Each tensor's values of the next chunk are
        // requested as soon as those of this chunk have been used (g and beta at the start of
        // P1), about one interval ahead of their use.
        u16x8 kr[4], qr[4], vr[4];
        float gr[2] = {0.f, 0.f}, br[2] = {0.f, 0.f};
        const int lrow = lane >> 4, lp = lane & 15;
        // requests of chunk c (absolute): g and beta, the rows of one tensor
        auto request_gb = [&](int c, auto slc) __attribute__((always_inline)) {
            constexpr int sl = decltype(slc)::value;
            // every prep wave loads them (only the gate wave uses them): unconditional loads keep the
            // wait counts before their use exact
            const int tg = min(c * C + lane, T - 1);
            if constexpr (!KDA) gr[sl] = gg[tg];
            br[sl] = bgp[tg];
        };
        // per-channel decay: prep waves 6 and 7 load the log-decays of a chunk one interval ahead
        // (lane: channel 64 (m - 2) + lane, every token) and form the chunk's factors E and channel
        // vectors into slot sl (the chunk's parity): the inclusive prefix G over the chunk's tokens
        // (log-decays below kKdaGMin taken as kKdaGMin, tokens past the end as 0), then
        // E[t] = e^{G_t - G_r} with r = token 7 of t's tile, and the channel vectors kVec*
        float gq[KDA ? C : 1];
        const int fch = 64 * (m - 2) + lane;  // the factor waves' channel
        const float *gch = KDA ? p.g + vtok * kD + fch : nullptr;
        auto request_g = [&](int c) __attribute__((always_inline)) {
            if constexpr (KDA) {
#pragma unroll
                for (int t = 0; t < C; ++t) gq[t] = gch[(int64_t)min(c * C + t, T - 1) * kD];
            }
        };
        auto form_factors = [&](int c, int sl) __attribute__((always_inline)) {
            if constexpr (KDA) {
                const int t0 = c * C;
                float G = 0.f;
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const bool live = t0 + t < T;
                    G += live ? fmaxf(gq[t], kKdaGMin) : 0.f;
                    gq[t] = G;
                }
                const float r0 = gq[7], r1 = gq[23], bd = gq[15], cl = gq[C - 1];
                unsigned char *Es = smem + L::oE + sl * C * L::kERow + 4 * fch;
#pragma unroll
                for (int t = 0; t < C; ++t)
                    *reinterpret_cast<float *>(Es + t * L::kERow) = __expf(gq[t] - (t < 16 ? r0 : r1));
                unsigned char *EV = smem + L::oEV + sl * kNVec * 512 + 4 * fch;
                auto put = [&](int v, float x) { *reinterpret_cast<float *>(EV + v * 512) = __expf(x); };
                put(kVecR0, r0);
                put(kVecR1, r1);
                put(kVecCR0, cl - r0);
                put(kVecCR1, cl - r1);
                put(kVecR1B, r1 - bd);
                put(kVecBR0, bd - r0);
                put(kVecC, cl);
            }
        };
        auto request_rows = [&](u16x8 (&r)[4], const uint16_t *src, int c, int tm) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[j] = *reinterpret_cast<const u16x8 *>(src + (int64_t)min(c * C + 16 * tm + 4 * j + lrow, T - 1) * kD + 8 * lp);
        };
        auto issue = [&](int c) __attribute__((always_inline)) {  // all of chunk c, into slot 0
            request_gb(c, IC<0>{});
            if (tile) {
                request_rows(kr, kg, c, m);
                if (OUT) request_rows(qr, qg, c, m);
                if constexpr (!kVSplit) request_rows(vr, vg, c, m);
            }
            if constexpr (kVSplit) {
                if (vtile) request_rows(vr, vg, c, vm);
            }
        };
        // output norm (NORM): the row waves stage chunk c's o rows between b1 and b2 of its
        // interval; in the next interval, before b1, the tile waves normalise them in place,
        // lane by lane the rows and columns of kr (NORM 2: the gate of chunk c requested one
        // interval ahead into gz), and after b1 the row waves store them. The prep waves issue
        // no global stores: with stores outstanding, every later wait for a load would have to
        // wait for all memory operations (one counter, completed out of order across the two
        // kinds), the next chunk's rows included.
        u16x8 gz[NORM == 2 ? 4 : 1];
        const uint16_t *gzp = NORM == 2 ? p.norm_gate + vtok * kD : nullptr;
        auto request_gate = [&](int c) __attribute__((always_inline)) {
            if constexpr (NORM == 2) {
                if (tile) request_rows(gz, gzp, c, m);
            }
        };
        auto norm_rows = [&]() __attribute__((always_inline)) {
            if constexpr (NORM > 0) {
                if (tile) {
                    const f32x4 w0 = ldf4(smem + L::oNW + 32 * lp), w1 = ldf4(smem + L::oNW + 32 * lp + 16);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * m + 4 * j + lrow;
                        // the row's 16 partial sums; columns 8 lp + 0..3 and + 4..7 were staged by
                        // two lanes of row wave lp / 4, whose sums sit in slots 4 (lp / 4) + 2 (lp % 2)
                        // and the next
                        const unsigned char *pp = smem + L::oNP + t * 80;
                        const f32x4 a = (ldf4(pp) + ldf4(pp + 16)) + (ldf4(pp + 32) + ldf4(pp + 48));
                        const float *own = reinterpret_cast<const float *>(pp) + 4 * (lp >> 2) + 2 * (lp & 1);
                        const float r = rsqrtf(((a[0] + a[1]) + (a[2] + a[3])) * (1.0f / kD) + p.norm_eps);
                        const float ra = r * stage_unscale(own[0]), rb = r * stage_unscale(own[1]);
                        unsigned char *xp = smem + L::oNO + t * 272 + 16 * lp;
                        const f16x8 x = ld8(xp);
                        f16x8 y;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            float f = e < 4 ? ra * w0[e] : rb * w1[e - 4];
                            if constexpr (NORM == 2) {
                                // silu(z) = z / (1 + exp(-z)) with the hardware reciprocal (1 ulp);
                                // exp(-z) = inf for z < -88 gives 0
                                const float z = bf16_bits_to_f32(gz[j][e]);
                                f *= z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
                            }
                            y[e] = f16_out((float)x[e] * f);
                        }
                        // the normalised row in place of the staged one, for the row waves' store
                        *reinterpret_cast<f16x8 *>(xp) = y;
                    }
                }
            }
        };
        // P1: prep wave kScanW forms the gate vectors of chunk c; tile m's
        // rows of chunk c into slot s (waits for their loads), each tensor's rows of chunk cn
        // requested right after
        auto phase1 = [&](int c, int cn, auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            const int t0 = c * C;
            if (KDA && m == 0) {
                // per-channel decay: the decays live in the tiles and channel vectors; the token
                // vectors are beta, with gamma = e^{G_C - G} = 1
                const bool gl = lane < C && t0 + lane < T;
                const float bv = gl ? br[s] : 0.f;
                if (lane < C) {
                    float *gts = reinterpret_cast<float *>(smem + L::oG + s * 20 * C);
                    gts[lane] = 1.0f;
                    gts[C + lane] = bv;
                    gts[2 * C + lane] = 1.0f;
                    gts[3 * C + lane] = bv;
                    gts[4 * C + lane] = 0.0f;
                }
            } else if (m == kScanW) {
                // tokens past the end have g = beta = 0
                const bool gl = lane < C && t0 + lane < T;
                form_gates<C>(smem + L::oG + s * 20 * C, gl ? gr[s] : 0.f, gl ? br[s] : 0.f, lane);
            }
            request_gb(cn, IC<1 - s>{});  // after the scan: its wait then covers only older requests
            fence();
            // rows past the end of the sequence hold the last token's values (the loads are clamped):
            // finite, and with beta = g = 0 on those tokens they contribute nothing
            if (tile) {
                // the fp16 tile's 16-byte group 4 Q + g of a row holds columns 32 Q + 4 g + 0..3 and
                // 32 Q + 16 + 4 g + 0..3: columns 8 p + 0..3 of this lane go to group
                // 4 (p / 4) + 2 (p % 2), 8 p + 4..7 to the next group, both at byte 8 ((p / 2) % 2)
                const int g0 = 4 * (lp >> 2) + 2 * (lp & 1), hb = 8 * ((lp >> 1) & 1);
                if constexpr (KDA) {
                    // per-channel decay: this lane's 8 channels 8 lp .. of each row as raw fp16 (for
                    // the block products), scaled by e^{G} = E e^{G_r} (the X / Y operand tiles),
                    // and k scaled by e^{G_C-1 - G} = e^{G_C-1 - G_r} / E (the update's tile)
                    const unsigned char *Es = smem + L::oE + s * C * L::kERow + 32 * lp;
                    const unsigned char *EV = smem + L::oEV + s * kNVec * 512;
                    const int vr = m == 0 ? kVecR0 : kVecR1, vcr = m == 0 ? kVecCR0 : kVecCR1;
                    const f32x4 eR0 = ldf4(EV + vr * 512 + 32 * lp), eR1 = ldf4(EV + vr * 512 + 32 * lp + 16);
                    const f32x4 eC0 = ldf4(EV + vcr * 512 + 32 * lp), eC1 = ldf4(EV + vcr * 512 + 32 * lp + 16);
                    if (m == 0 && lane < 32)  // e^{G_C-1} of the chunk for the row waves' state decay
                        *reinterpret_cast<f32x4 *>(smem + L::oEC + s * 512 + 16 * lane) = ldf4(EV + kVecC * 512 + 16 * lane);
                    auto put = [&](size_t base, int t, f32x4 x0, f32x4 x1) {
                        const int sw = ksw(t & 15);
                        unsigned char *row = smem + base + t * 256;
                        *reinterpret_cast<f16x4 *>(row + (((g0 ^ sw) << 4) + hb)) = to_f16x4(x0);
                        *reinterpret_cast<f16x4 *>(row + ((((g0 + 1) ^ sw) << 4) + hb)) = to_f16x4(x1);
                    };
                    auto widen = [](u16x8 a, f32x4 &x0, f32x4 &x1) {
                        x0 = f32x4{bf16_bits_to_f32(a[0]), bf16_bits_to_f32(a[1]), bf16_bits_to_f32(a[2]), bf16_bits_to_f32(a[3])};
                        x1 = f32x4{bf16_bits_to_f32(a[4]), bf16_bits_to_f32(a[5]), bf16_bits_to_f32(a[6]), bf16_bits_to_f32(a[7])};
                    };
                    auto rcp4 = [](f32x4 x) {
                        return f32x4{__builtin_amdgcn_rcpf(x[0]), __builtin_amdgcn_rcpf(x[1]), __builtin_amdgcn_rcpf(x[2]),
                                     __builtin_amdgcn_rcpf(x[3])};
                    };
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * m + 4 * j + lrow;
                        const f32x4 E0 = ldf4(Es + t * L::kERow), E1 = ldf4(Es + t * L::kERow + 16);
                        f32x4 x0, x1;
                        widen(kr[j], x0, x1);
                        put(L::oRK, t, x0, x1);
                        put(L::oK + s * L::kTile, t, x0 * E0 * eR0, x1 * E1 * eR1);
                        put(L::oKT + s * L::kTile, t, x0 * rcp4(E0) * eC0, x1 * rcp4(E1) * eC1);
                    }
                    fence();
                    request_rows(kr, kg, cn, m);
                    fence();
                    if (OUT) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int t = 16 * m + 4 * j + lrow;
                            const f32x4 E0 = ldf4(Es + t * L::kERow), E1 = ldf4(Es + t * L::kERow + 16);
                            f32x4 x0, x1;
                            widen(qr[j], x0, x1);
                            put(L::oRQ, t, x0, x1);
                            put(L::oQ + s * L::kTile, t, x0 * E0 * eR0, x1 * E1 * eR1);
                        }
                        fence();
                        request_rows(qr, qg, cn, m);
                        fence();
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * m + 4 * j + lrow;
                        const int sw = ksw(t & 15);
                        unsigned char *krow = smem + L::oK + s * L::kTile + t * 256;
                        const u16x8 a = kr[j];
                        *reinterpret_cast<f16x4 *>(krow + (((g0 ^ sw) << 4) + hb)) = bf4_to_h4(a[0], a[1], a[2], a[3]);
                        *reinterpret_cast<f16x4 *>(krow + ((((g0 + 1) ^ sw) << 4) + hb)) = bf4_to_h4(a[4], a[5], a[6], a[7]);
                    }
                    fence();
                    request_rows(kr, kg, cn, m);
                    fence();
                    if (OUT) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int t = 16 * m + 4 * j + lrow;
                            const int sw = ksw(t & 15);
                            unsigned char *qrow = smem + L::oQ + s * L::kTile + t * 256;
                            const u16x8 b = qr[j];
                            *reinterpret_cast<f16x4 *>(qrow + (((g0 ^ sw) << 4) + hb)) = bf4_to_h4(b[0], b[1], b[2], b[3]);
                            *reinterpret_cast<f16x4 *>(qrow + ((((g0 + 1) ^ sw) << 4) + hb)) = bf4_to_h4(b[4], b[5], b[6], b[7]);
                        }
                        fence();
                        request_rows(qr, qg, cn, m);
                        fence();
                    }
                }
                if constexpr (!kVSplit) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * m + 4 * j + lrow;
                        *reinterpret_cast<u16x8 *>(smem + L::oV + s * L::kTile + t * 256 + ((lp ^ ksw(t & 15)) << 4)) = vr[j];
                    }
                    fence();
                    request_rows(vr, vg, cn, m);
                    fence();
                }
            }
            if constexpr (kVSplit) {
                if (vtile) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * vm + 4 * j + lrow;
                        *reinterpret_cast<u16x8 *>(smem + L::oV + s * L::kTile + t * 256 + ((lp ^ ksw(t & 15)) << 4)) = vr[j];
                    }
                    fence();
                    request_rows(vr, vg, cn, vm);
                    fence();
                }
            }
            if constexpr (KDA) {
                // the factors of chunk cn into the other slot (its parity), from the log-decays
                // loaded during the last interval; then those of the chunk after it requested
                if (m >= 2) {
                    form_factors(cn, 1 - s);
                    request_g(min(cn + 1, cb + max(n, 1) - 1));
                }
            }
        };
        // P2: the gated blocks of A (negated, below the diagonal; the diagonal block inverted) and
        // A_qk of chunk slot s. A tile (mm, nt) is the 16 x 16 block of rows 16 mm .. and columns
        // 16 nt .. (nt <= mm) from K K^T and Q K^T; prep wave W forms its diagonal tile (W, W),
        // whose inverse it builds, and off-diagonal tiles chosen so that no wave forms more than
        // three (C = 64: W0 (3,0) (3,1), W1 (1,0) (2,0), W2 (2,1), W3 (3,2); C = 32: W1 (1,0); C = 16:
        // W0 its diagonal tile only).
        auto phase2w = [&](int s, auto wc) __attribute__((always_inline)) {
            constexpr int W = decltype(wc)::value;
            // C = 32: W0 and W1 the diagonal tiles and their inverses, W2 the tile (1,0) below them
            constexpr bool kDiag = !(C == 32 && W == 2);
            constexpr int nT = C == 64 ? (W < 2 ? 3 : 2) : C == 32 ? (W < 3 ? 1 : 0) : (W == 0 ? 1 : 0);
            constexpr int MMs[3] = {kDiag ? W : 1, C == 64 ? (W == 0 ? 3 : W == 1 ? 1 : W) : W, C == 64 ? (W == 0 ? 3 : 2) : 0};
            constexpr int NTs[3] = {kDiag ? W : 0, C == 64 ? (W == 0 ? 0 : W == 1 ? 0 : W - 1) : 0, C == 64 ? (W == 0 ? 1 : 0) : 0};
            if constexpr (nT > 0) {
                const unsigned char *Kt = smem + L::oK + s * L::kTile;
                const unsigned char *Qt = smem + L::oQ + s * L::kTile;
                const float *gts = reinterpret_cast<const float *>(smem + L::oG + s * 20 * C);
                // fragments, the diagonal tile's first: lane (q4, li) reads row 16 x + li, group
                // 4 kb + q4 (the diagonal tile's two operands are one fragment)
                f16x8 ka[nT][4], bk[nT][4], bq[nT][4];
                auto frag = [&](int j, int kb) __attribute__((always_inline)) {
                    const int off = li * 256 + (((4 * kb + q4) ^ ksw(li)) << 4);
                    ka[j][kb] = ld8(Kt + off + NTs[j] * 4096);
                    bk[j][kb] = ld8(Kt + off + MMs[j] * 4096);
                    if (OUT) bq[j][kb] = ld8(Qt + off + MMs[j] * 4096);
                };
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) frag(0, kb);
                float Gt[nT], btt[nT];
                f32x4 Gs[nT];
#pragma unroll
                for (int j = 0; j < nT; ++j) {
                    Gt[j] = gts[4 * C + 16 * MMs[j] + li];
                    btt[j] = gts[C + 16 * MMs[j] + li];
                    Gs[j] = *reinterpret_cast<const f32x4 *>(gts + 4 * C + 16 * NTs[j] + 4 * q4);
                }
#pragma unroll
                for (int j = 1; j < nT; ++j)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) frag(j, kb);
                fence();
                // raw products, lane (q4, li): t = 16 mm + li, s = 16 nt + 4 q4 + r; the diagonal
                // tile's first
                f32x4 rk[nT], rq[nT];
#pragma unroll
                for (int j = 0; j < nT; ++j) rk[j] = rq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < nT; ++j)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        rk[j] = mfma16x16x32(ka[j][kb], bk[j][kb], rk[j]);
                        if (OUT) rq[j] = mfma16x16x32(ka[j][kb], bq[j][kb], rq[j]);
                    }
                fence();
                // gating; only the diagonal tile (j = 0) needs the triangular mask
                f32x4 a[nT], aqv[nT];
                const float sct = p.scale;
                auto gate = [&](int j) __attribute__((always_inline)) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float gv = __expf(Gt[j] - Gs[j][r]);
                        if (j == 0 && kDiag) {
                            const int sidx = 4 * q4 + r;
                            a[j][r] = sidx < li ? btt[j] * gv * rk[j][r] : 0.0f;
                            if (OUT) aqv[j][r] = sidx <= li ? sct * gv * rq[j][r] : 0.0f;
                        } else {
                            a[j][r] = btt[j] * gv * rk[j][r];
                            if (OUT) aqv[j][r] = sct * gv * rq[j][r];
                        }
                    }
                };
                // A_qk: a tile's half of its 16-byte fragment (the block above the diagonal next to
                // an even diagonal tile is zero)
                unsigned char *aqb = smem + L::oA + s * L::kFr * 1024 + lane * 16;
                auto store_aq = [&](int j) __attribute__((always_inline)) {
                    if (OUT)
                        *reinterpret_cast<f16x4 *>(aqb + fblk(MMs[j], NTs[j] / 2) * 1024 + (NTs[j] & 1) * 8) =
                            to_f16x4(aqv[j]);
                };
                // the diagonal tile: its row of A_WW goes through this wave's LDS scratch (written as
                // accumulators, read back by rows) for the inverse, which starts once it is back
                gate(0);
                if constexpr (!kDiag) {
                    // a tile below the diagonal alone: A_qk and -A
                    store_aq(0);
                    *reinterpret_cast<f16x4 *>(smem + L::oNA + s * L::kNA * 512 + ablk(MMs[0], NTs[0]) * 512 + lane * 8) =
                        to_f16x4(-a[0]);
                } else {
                    float *at = reinterpret_cast<float *>(smem + L::oAt) + W * 16 * 20;
#pragma unroll
                    for (int r = 0; r < 4; ++r) at[(4 * q4 + r) * 20 + li] = -a[0][r];  // at[s][i] = -A[i][s]
                    store_aq(0);
                    if constexpr (OUT && (W & 1) == 0) *reinterpret_cast<f16x4 *>(aqb + fblk(W, W / 2) * 1024 + 8) = f16x4{};
                    fence();
                    // the tiles below the diagonal: gated while the scratch round trip completes, stored
                    // after its reads are requested
#pragma unroll
                    for (int j = 1; j < nT; ++j) gate(j);
                    fence();
                    float nrow[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) nrow[k] = at[k * 20 + li];
                    fence();
#pragma unroll
                    for (int j = 1; j < nT; ++j) {
                        store_aq(j);
                        // -A below the diagonal (A operands of the block substitution)
                        *reinterpret_cast<f16x4 *>(smem + L::oNA + s * L::kNA * 512 + ablk(MMs[j], NTs[j]) * 512 +
                                                   lane * 8) = to_f16x4(-a[j]);
                    }
                    fence();
                    // T_WW = (I + A_WW)^{-1}: lane (q4, li) builds T[li][4 q4 + e]
                    f32x4 tq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) tq[e] = 4 * q4 + e == li ? 1.0f : 0.0f;
                    inv_rows(tq, nrow);
                    // T_WW and diag(exp(G_C - G)) T_WW (row li scaled): the latter gives the scaled
                    // values of the state update straight from the substitution
                    const float egt = gts[2 * C + 16 * W + li];
                    unsigned char *tdb = smem + L::oTd + s * 2 * NT * 512 + W * 1024 + lane * 8;
                    *reinterpret_cast<f16x4 *>(tdb) = to_f16x4(tq);
                    *reinterpret_cast<f16x4 *>(tdb + 512) = to_f16x4(egt * tq);
                }
            }
        };
        // P2, per-channel decay (C = 32). The diagonal blocks (m, m) in float32 as (k o 1/E)(k o E)^T
        // with E relative to the tile's 8th token (every factor within e^{+-80}); lane (q4, li)
        // supplies row li of both operands for k = q4: channels 4 rho .. + 3 of run rho = 4 blk +
        // q4 over the eight runs' steps. The block (1,0) relative to the last token b of tile 0,
        // (k o e^{G_b - G_r0} / E)(k o E e^{G_r1 - G_b})^T, whose operands are decays (<= 1): in fp16,
        // the same runs as 16 x 16 x 16 steps. Work: W0 A(0,0) and its inverse,
        // W1 A(1,1) and its inverse, W2 (which holds the next log-decays) A_qk(0,0), W3 A(1,0) and
        // A_qk(1,1); in the output pass the blocks (1,0) in two channel halves: of A on W0 and W3,
        // of A_qk on W1 and W2.
        auto kda_diag = [&](int s, int mm, bool qside) __attribute__((always_inline)) {
            const int tok = 16 * mm + li;
            const unsigned char *Es = smem + L::oE + s * C * L::kERow + tok * L::kERow;
            const unsigned char *rk = smem + L::oRK + tok * 256;
            const unsigned char *rb = smem + (qside ? L::oRQ : L::oRK) + tok * 256;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const int rho = 4 * blk + q4;
                const int off = ((((4 * (rho >> 3) + (rho & 3)) ^ ksw(tok & 15))) << 4) + 8 * ((rho >> 2) & 1);
                const f16x4 ks = ld4(rk + off), kt = ld4(rb + off);
                const f32x4 e = ldf4(Es + 16 * rho);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32((float)ks[r] * __builtin_amdgcn_rcpf(e[r]), (float)kt[r] * e[r],
                                                            acc, 0, 0, 0);
                if ((blk & 1) == 1) fence();  // two runs' operands live at a time
            }
            return acc;  // lane (q4, li), element r: s = 16 mm + 4 q4 + r, t = 16 mm + li
        };
        // the block (1,0) of A (QS = false: k of tile 1) or of A_qk (QS = true: q of tile 1)
        // over channel runs blk in [B0, B1) of the eight
        auto kda_off = [&](int s, auto qs, auto b0, auto b1) __attribute__((always_inline)) {
            constexpr bool QS = decltype(qs)::value;
            constexpr int B0 = decltype(b0)::value, B1 = decltype(b1)::value;
            const int tsk = li, ttk = 16 + li;
            const unsigned char *Es = smem + L::oE + s * C * L::kERow;
            const unsigned char *EV = smem + L::oEV + s * kNVec * 512;
            const unsigned char *rks = smem + L::oRK + tsk * 256;
            const unsigned char *rbt = smem + (QS ? L::oRQ : L::oRK) + ttk * 256;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int blk = B0; blk < B1; ++blk) {
                const int rho = 4 * blk + q4;
                const int grp = 4 * (rho >> 3) + (rho & 3), half = 8 * ((rho >> 2) & 1);
                const f16x4 ks = ld4(rks + ((grp ^ ksw(tsk & 15)) << 4) + half);
                const f16x4 kt = ld4(rbt + ((grp ^ ksw(ttk & 15)) << 4) + half);
                const f32x4 es = ldf4(Es + tsk * L::kERow + 16 * rho), et = ldf4(Es + ttk * L::kERow + 16 * rho);
                const f32x4 fb = ldf4(EV + kVecBR0 * 512 + 16 * rho), fr = ldf4(EV + kVecR1B * 512 + 16 * rho);
                f16x4 a, b;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a[r] = (_Float16)((float)ks[r] * (__builtin_amdgcn_rcpf(es[r]) * fb[r]));
                    b[r] = (_Float16)((float)kt[r] * (et[r] * fr[r]));
                }
                acc = mfma16x16x16(a, b, acc);
                if ((blk & 1) == 1) fence();  // two runs' operands live at a time
            }
            return acc;  // lane (q4, li), element r: s = 4 q4 + r, t = 16 + li
        };
        auto phase2k = [&](int s, auto wc) __attribute__((always_inline)) {
            constexpr int W = decltype(wc)::value;
            if constexpr (KDA) {
                const float *gts = reinterpret_cast<const float *>(smem + L::oG + s * 20 * C);
                const float sct = p.scale;
                unsigned char *aqb = smem + L::oA + s * L::kFr * 1024 + lane * 16;
                if constexpr (W < 2) {
                    // A(W, W) (strict lower, with beta), then T_WW = (I + A_WW)^{-1} as for the scalar
                    // decay (Td's scaled copy is T itself: the update's decay is in its k tile)
                    const f32x4 acc = kda_diag(s, W, false);
                    const float bt = gts[C + 16 * W + li];
                    f32x4 a;
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[r] = 4 * q4 + r < li ? bt * acc[r] : 0.0f;
                    float *at = reinterpret_cast<float *>(smem + L::oAt) + W * 16 * 20;
#pragma unroll
                    for (int r = 0; r < 4; ++r) at[(4 * q4 + r) * 20 + li] = -a[r];
                    float nrow[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) nrow[k] = at[k * 20 + li];
                    f32x4 tq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) tq[e] = 4 * q4 + e == li ? 1.0f : 0.0f;
                    inv_rows(tq, nrow);
                    unsigned char *tdb = smem + L::oTd + s * 2 * NT * 512 + W * 1024 + lane * 8;
                    *reinterpret_cast<f16x4 *>(tdb) = to_f16x4(tq);
                    *reinterpret_cast<f16x4 *>(tdb + 512) = to_f16x4(tq);
                    if constexpr (OUT) {
                        // the first channel half of the block (1,0): of -A on W0, of A_qk on W1
                        if constexpr (W == 0) {
                            const float b1 = gts[C + 16 + li];
                            *reinterpret_cast<f16x4 *>(smem + L::oNA + s * L::kNA * 512 + ablk(1, 0) * 512 + lane * 8) =
                                to_f16x4(-(b1 * kda_off(s, IC<0>{}, IC<0>{}, IC<4>{})));
                        } else {
                            *reinterpret_cast<f16x4 *>(aqb + fblk(1, 0) * 1024) =
                                to_f16x4(sct * kda_off(s, IC<1>{}, IC<0>{}, IC<4>{}));
                        }
                    }
                } else if constexpr (W == 3) {
                    // -A(1,0): all of it in the map pass, its second channel half in the output pass
                    const f32x4 acc = OUT ? kda_off(s, IC<0>{}, IC<4>{}, IC<8>{}) : kda_off(s, IC<0>{}, IC<0>{}, IC<8>{});
                    const float bt = gts[C + 16 + li];
                    *reinterpret_cast<f16x4 *>(smem + (OUT ? L::oNA2 + s * 512 : L::oNA + s * L::kNA * 512 + ablk(1, 0) * 512) +
                                               lane * 8) = to_f16x4(-(bt * acc));
                    if (OUT) {
                        const f32x4 dq = kda_diag(s, 1, true);
                        f32x4 aq;
#pragma unroll
                        for (int r = 0; r < 4; ++r) aq[r] = 4 * q4 + r <= li ? sct * dq[r] : 0.0f;
                        *reinterpret_cast<f16x4 *>(aqb + fblk(1, 0) * 1024 + 8) = to_f16x4(aq);
                    }
                } else if (OUT) {
                    // W2: A_qk(0,0) (lower incl., with scale); the fragment's other half is zero
                    const f32x4 dq = kda_diag(s, 0, true);
                    f32x4 aq;
#pragma unroll
                    for (int r = 0; r < 4; ++r) aq[r] = 4 * q4 + r <= li ? sct * dq[r] : 0.0f;
                    *reinterpret_cast<f16x4 *>(aqb + fblk(0, 0) * 1024) = to_f16x4(aq);
                    *reinterpret_cast<f16x4 *>(aqb + fblk(0, 0) * 1024 + 8) = f16x4{};
                    // and the second channel half of A_qk(1,0), with a zero second half
                    unsigned char *aq2 = smem + L::oAQ2 + s * 1024 + lane * 16;
                    *reinterpret_cast<f16x4 *>(aq2) = to_f16x4(sct * kda_off(s, IC<1>{}, IC<4>{}, IC<8>{}));
                    *reinterpret_cast<f16x4 *>(aq2 + 8) = f16x4{};
                }
            }
        };
        auto phase2 = [&](int s) __attribute__((always_inline)) {
            if constexpr (KDA) {
                if (m == 0) phase2k(s, IC<0>{});
                else if (m == 1) phase2k(s, IC<1>{});
                else if (m == 2) phase2k(s, IC<2>{});
                else phase2k(s, IC<3>{});
            } else {
                if (m == 0) phase2w(s, IC<0>{});
                else if (m == 1) phase2w(s, IC<1>{});
                else if (m == 2) phase2w(s, IC<2>{});
                else phase2w(s, IC<3>{});
            }
        };

        // prologue: chunk 0 of the segment into slot 0. Every load is issued and every P1 runs, the
        // chunk indices clamped to the segment (a clamped P1 fills the slot no one reads next),
        // so that the loop carries no register whose load is optional.
        const int clast = cb + max(n, 1) - 1;
        if constexpr (KDA) {
            // the first chunk's factors before its rows are converted
            if (m >= 2) {
                request_g(cb);
                form_factors(cb, 0);
                request_g(min(cb + 1, clast));
            }
            lds_barrier();
        }
        request_gate(cb);
        issue(cb);
        phase1(cb, min(cb + 1, clast), IC<0>{});
        lds_barrier();
        if (n > 0) phase2(0);
        lds_barrier();

        auto interval = [&](auto sl, int i) __attribute__((always_inline)) {
            constexpr int s1 = 1 - decltype(sl)::value;  // slot of chunk i + 1
            const int c1 = cb + i + 1;
            if (i > 0) norm_rows();  // chunk i - 1, staged in the previous interval
            request_gate(min(cb + i, clast));
            phase1(min(c1, clast), min(c1 + 1, clast), IC<s1>{});
            lds_barrier();  // b1
            if (i + 1 < n) phase2(s1);
            lds_barrier();  // b2
        };
        for (int i = 0; i < n; i += 2) {
            interval(IC<0>{}, i);
            if (i + 1 < n) interval(IC<1>{}, i + 1);
        }
        if constexpr (NORM > 0) {
            if (n > 0) norm_rows();  // the last chunk, staged before the last b2
            lds_barrier();           // for the row waves' store of it
        }
    }
}

// S_{p+1} = S_p M_p + N_p for p = 1 .. P-2, one workgroup per (pair, block of 16 rows), fp32,
// the 16 x 128 x 128 product on float32 MFMAs. M_p goes through LDS; the next map and the next
// N values are loaded into registers while the current product runs, so that only the chain of
// S (LDS and matrix core) is sequential.
constexpr int kCombineMRow = kD + 16;  // 144 floats: four map rows 16 banks apart

__global__ __launch_bounds__(512) void gdn_seg_combine_kernel(SegParams sp) {
    extern __shared__ __attribute__((aligned(16))) unsigned char csmem[];
    // srow: this block's 16 rows of the running start state; mt: the map M_seg, rows padded to
    // 144 floats so that the operand reads below meet 64 distinct banks
    float(*srow)[kD + 4] = reinterpret_cast<float(*)[kD + 4]>(csmem);
    float(*mt)[kCombineMRow] = reinterpret_cast<float(*)[kCombineMRow]>(csmem + 16 * (kD + 4) * 4);
    // workgroups go round-robin over the 8 XCDs: the 8 row blocks of a pair share one XCD (and
    // its L2 for the maps they all read) when the grid is a multiple of 64
    const int nb = gridDim.x;
    const int lin = (nb & 63) == 0 ? (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int pair = lin >> 3, rb = lin & 7;
    const int tid = threadIdx.x, r = tid >> 5, c4 = tid & 31;
    const int lane = tid & 63, w = tid >> 6, li = lane & 15, q4 = lane >> 4;
    const int64_t base = (int64_t)pair * sp.P;
    constexpr int kPer = kD * kD / 4 / 512;  // f32x4 of a map per thread
    // the products on float32 MFMAs (16 x 16 x 4): wave w owns the 16-column tile w; lane
    // (q4, li) holds rows 4 q4 + e, column 16 w + li of the new state, with N there as the
    // products' start
    f32x4 mnext[kPer], nnext;
    auto load_next = [&](int seg) {  // N_seg at this lane's output places (first: needed first), M_seg
        const float *N = sp.ws_n + (base + seg) * (kD * kD) + (rb * 16 + 4 * q4) * kD + 16 * w + li;
#pragma unroll
        for (int e = 0; e < 4; ++e) nnext[e] = N[e * kD];
        const f32x4 *M = reinterpret_cast<const f32x4 *>(sp.ws_m + (base + seg) * (kD * kD));
#pragma unroll
        for (int j = 0; j < kPer; ++j) mnext[j] = M[tid + 512 * j];
    };
    // S_1's rows of this block and the first map requested together
    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(sp.ws_start + (base + 1) * (kD * kD) + (rb * 16 + r) * kD + 4 * c4);
    load_next(1);
    *reinterpret_cast<f32x4 *>(&srow[r][4 * c4]) = x0;
    for (int seg = 1; seg + 1 < sp.P; ++seg) {
        float *Sn = sp.ws_start + (base + seg + 1) * (kD * kD) + (rb * 16 + 4 * q4) * kD + 16 * w + li;
        __syncthreads();  // srow written; earlier reads of mt done
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int f = tid + 512 * j;  // f32x4 index of the map: row f / 32, columns 4 (f % 32) ..
            *reinterpret_cast<f32x4 *>(&mt[f >> 5][4 * (f & 31)]) = mnext[j];
        }
        f32x4 acc = nnext;
        if (seg + 2 < sp.P) load_next(seg + 1);
        __syncthreads();
        // S_new = S M + N: A = S (row li, k = 4 s + q4), B = M (row k, column 16 w + li)
#pragma unroll 8
        for (int s = 0; s < kD / 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(srow[li][4 * s + q4], mt[4 * s + q4][16 * w + li], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Sn[e * kD] = acc[e];
        __syncthreads();  // every read of srow done
#pragma unroll
        for (int e = 0; e < 4; ++e) srow[4 * q4 + e][16 * w + li] = acc[e];
    }
}

constexpr size_t kCombineLds = 16 * (kD + 4) * 4 + kD * kCombineMRow * 4;

// T = 0: the final state is the initial state (converted to its storage type), or zero.
__global__ __launch_bounds__(256) void gdn_state_copy_kernel(PrefillParams p, int64_t count) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= count) return;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (p.init_state) x = load_state4(p.init_state, i, p.init_f16, p.state_bf16);
    store_state4(p.final_state, i, x, p.final_f16, p.state_bf16);
}

template <int C, bool OUT, int NORM = 0, bool KDA = false>
hipError_t launch_pass(const SegParams &sp, int64_t nblocks, hipStream_t stream) {
    const size_t bytes = SegSmem<C, OUT, (NORM > 0), KDA>::kBytes;
    static bool attr_set = false;  // the attribute is a property of the function: set once
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_seg_pass_kernel<C, OUT, NORM, KDA>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    if (nblocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gdn_seg_pass_kernel<C, OUT, NORM, KDA>), dim3((unsigned)nblocks), dim3(seg_threads<OUT, KDA>()), bytes,
                       stream, sp);
    return hipGetLastError();
}

template <int C, bool KDA = false>
hipError_t launch_seg_c(const SegParams &sp, hipStream_t stream) {
    const int64_t pairs = (int64_t)sp.p.B * sp.p.Hv;
    hipError_t err = hipSuccess;
    if (sp.P > 1) {
        // map pass: one workgroup per pair and segment but the last. The 64-token call's map pass
        // runs 32-token chunks (twice as many per segment: the same segment boundaries), where the
        // merged workgroup's registers fit without spills
        constexpr int CM = C == 64 ? 32 : C;
        SegParams spm = sp;
        spm.seg_chunks = sp.seg_chunks * (C / CM);
        err = launch_pass<CM, false, 0, KDA>(spm, pairs * (sp.P - 1), stream);
        if (err != hipSuccess) return err;
        if (sp.P > 2) {
            static bool attr_set = false;
            if (!attr_set) {
                err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_seg_combine_kernel),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kCombineLds);
                if (err != hipSuccess) return err;
                attr_set = true;
            }
            hipLaunchKernelGGL(gdn_seg_combine_kernel, dim3((unsigned)(pairs * 8)), dim3(512), kCombineLds, stream, sp);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    }
    if constexpr (KDA) {
        return launch_pass<C, true, 0, true>(sp, pairs * sp.P, stream);
    } else {
        if (!sp.p.norm_w) return launch_pass<C, true>(sp, pairs * sp.P, stream);
        return sp.p.norm_gate ? launch_pass<C, true, 2>(sp, pairs * sp.P, stream)
                              : launch_pass<C, true, 1>(sp, pairs * sp.P, stream);
    }
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

hipError_t launch_prefill_seg(const PrefillParams &p, int chunk, int P, void *ws, hipStream_t stream, bool kda) {
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
    if (kda) return chunk == 32 ? launch_seg_c<32, true>(sp, stream) : hipErrorInvalidValue;
    switch (chunk) {
        case 16: return launch_seg_c<16>(sp, stream);
        case 32: return launch_seg_c<32>(sp, stream);
        case 64: return launch_seg_c<64>(sp, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
