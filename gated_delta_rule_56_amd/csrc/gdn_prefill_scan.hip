// Sequential half of the bf16 prefill: the pass over the chunks of one
// (b, h, block of 16 state rows), with the fp32 state resident in registers.
//
// Per chunk c with start state S (rows i of this block), T, A_qk and the gate
// vectors from the chunk kernel (gdn_prefill_chunk.hip):
//   X = K S^T,  R = diag(beta) V - diag(beta gamma) X,  U = T R
//   S <- gamma_C S + (diag(exp(G_C - G)) U)^T K
//   O = diag(gamma) (scale Q S^T) + A_qk U
// (the chunked WY form of S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) +
// beta_t v_t k_t^T, o_t = S_t scale q_t, with U solving (I + A) U = R).
//
// Roles inside the workgroup (6 waves; wave i runs on SIMD i % 4):
//   wave 0, "state": owns the 16 x 128 fp32 state block as MFMA accumulators
//     and runs only the chain S -> X -> R -> U -> S: 38 MFMAs and about a
//     hundred VALU operations per 64-token chunk. K^T operands come straight
//     from the row-major k tile through transposing LDS reads
//     (ds_read_b64_tr_b16); every LDS address is a per-lane register plus an
//     immediate (the chunk loop is unrolled over the ring slots).
//   waves 1 and 5, "loaders": stream chunk c+3 into a 4-slot LDS ring with
//     direct global->LDS loads and wait for chunk c+1 with an exact vmcnt.
//     Wave 1 moves the fp16 k tile prepared by the chunk kernel; wave 5 the T
//     fragments on or below the diagonal, and one chunk further ahead the gate
//     vectors and the bf16 v rows. Two waves because one wave can keep at most
//     63 vector loads in flight, which is less than three chunks' worth.
//   wave 4, "prefetch and store": requests chunk c+8 into L2. The k, q, T, A_qk,
//     gate and v lines of a chunk are each read by 8 or 16 workgroups at about
//     the same time; without it all of them would wait for the same HBM miss.
//     Each line is touched by exactly one of the workgroups that share it. It
//     also writes the o rows of chunk c-2 to memory from LDS, so that the
//     output waves, which wait on their own loads, never wait on stores.
//   waves 2-3, "output": O^T rather than O, so that a lane ends up with four
//     consecutive o columns of one token and stores them with one 16-byte
//     store: Y^T = S Q^T of chunk c from an fp16 copy of S, and O^T of chunk
//     c-1 = scale Y^T diag(gamma) + U^T A_qk^T from an fp16 copy of U (in the
//     fragment order the fp16 copies are the A operands of these products as
//     they are, and the q and A_qk fragments the B operands). The q and A_qk
//     fragments (prepared by the chunk kernel in per-lane order) are
//     prefetched two chunks ahead into registers, and o rows past the sequence
//     end are dropped by a bounded buffer store rather than a branch. They also
//     form the operands of the next chunk from its v rows and gates: beta*v
//     (transposed, fp32), beta*gamma, exp(G_C - G) and gamma.
// One workgroup barrier per chunk, and one more at the end for the last o rows. The k tile is stored with its 16-byte column
// groups XOR-swizzled by row (group g of row t at g ^ ksw(t % 16)) so that MFMA
// fragment reads spread over the LDS banks.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRows = 16;
constexpr int kThreads = 384;
constexpr int kPrefetchAhead = 8;  // chunks
constexpr int kSlots = 4;
// word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format, so that
// out-of-range accesses (offset >= num_records bytes) are dropped by the hardware
constexpr int kBufferFlags = 0x00020000;


typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int C>
struct ScanSmem {
    static constexpr int NT = C / 16;     // token tiles per chunk
    static constexpr int KBC = C / 32;    // 32-wide k blocks over the chunk
    static constexpr int VP = C + 4;      // f32 pitch of the transposed beta*v block
    // ring, grouped by tensor so that slot offsets are immediates
    static constexpr size_t rK = 0;                             // [4][C][128] fp16, swizzled
    static constexpr size_t rT = rK + kSlots * 256 * C;         // [4] T fragments [NT][KBC][64][8] fp16
    static constexpr size_t rV = rT + kSlots * 2 * C * C;       // [4][C][16] bf16
    static constexpr size_t rG = rV + kSlots * 32 * C;          // [4] gamma[C], beta[C], exp(G_C - G)[C] f32
    // per-chunk operands formed from v and the gates, double-buffered by chunk parity
    static constexpr size_t gBV = rG + kSlots * 12 * C;         // [2][16][VP] f32: beta_t v[t][i]
    static constexpr size_t gGT = gBV + 2 * 4 * kRows * VP;     // [2][3][64] f32: beta_t gamma_t, exp(G_C - G_t), gamma_t
    // exchange
    static constexpr size_t kS16 = gGT + 2 * 768;               // [2][4][64] x 16 B
    static constexpr size_t kU16 = kS16 + 2 * 4 * 64 * 16;      // [2][KBC][64] x 16 B
    static constexpr size_t kOst = kU16 + 2 * KBC * 64 * 16;      // [2][C][16] f32: o rows of a chunk, to store
    static constexpr size_t kJunk = kOst + 2 * C * kRows * 4;     // [64] x 4 B: target of the L2 prefetches
    static constexpr size_t kBytes = kJunk + 256;
    static constexpr int kDmaK = C / 4;                         // k-tile loads per chunk (wave 1)
    static constexpr int kTFrags = NT * KBC - (NT / 2) * (KBC - 1);  // T fragments with kb <= m / 2
    static constexpr int kDmaT = kTFrags + C / 32 + 1;          // T of chunk c, v and gates of c + 1 (wave 5)
    static_assert(rT % 16 == 0 && rV % 16 == 0 && rG % 16 == 0 && gBV % 16 == 0 && kS16 % 16 == 0, "alignment");
    static_assert(kSlots * 256 * C <= 65536, "k-tile immediates");
    static_assert(2 * kDmaK <= 63 && 2 * kDmaT <= 63, "vmcnt range");
};

__device__ __forceinline__ f16x8 ld8(const unsigned char *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ f32x4 ldf4(const unsigned char *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ f16x8 pack8(f32x4 lo, f32x4 hi) {
    return f16x8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                 (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
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

template <int N>
using IC = std::integral_constant<int, N>;

// Calls f(IC<c % 4>, c) for c = 0 .. n-1 with a compile-time ring slot.
template <typename F>
__device__ __forceinline__ void for_chunks(int n, F &&f) {
    for (int c0 = 0; c0 < n; c0 += kSlots) {
        f(IC<0>{}, c0);
        if (c0 + 1 < n) f(IC<1>{}, c0 + 1);
        if (c0 + 2 < n) f(IC<2>{}, c0 + 2);
        if (c0 + 3 < n) f(IC<3>{}, c0 + 3);
    }
}

// Operands of chunk c formed from its v rows and gate vectors (ring slot c % 4), into the
// buffers of parity c & 1: beta_t v[t][8 h + e] for e = 0..7 (transposed), and with
// all = true also beta_t gamma_t, exp(G_C - G_t) and gamma_t. Lane t < C handles token t.
template <int C>
__device__ __forceinline__ void prepare_chunk_impl(unsigned char *smem, int c, int h, bool all, int lane) {
    using L = ScanSmem<C>;
    constexpr int VP = L::VP;
    const int s = c % kSlots, par = c & 1;
    if (lane < C) {
        const float *gt = reinterpret_cast<const float *>(smem + L::rG + s * 12 * C);
        const float bt = gt[C + lane];
        const u16x8 v8 = *reinterpret_cast<const u16x8 *>(smem + L::rV + s * 32 * C + (lane * kRows + 8 * h) * 2);
        float *bv = reinterpret_cast<float *>(smem + L::gBV + par * 4 * kRows * VP) + 8 * h * VP + lane;
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e * VP] = bt * bf16_bits_to_f32(v8[e]);
        if (all) {
            float *gg = reinterpret_cast<float *>(smem + L::gGT + par * 768) + lane;
            const float gam = gt[lane];
            gg[0] = bt * gam;
            gg[64] = gt[2 * C + lane];
            gg[128] = gam;
        }
    }
}

template <int C>
__global__ __launch_bounds__(kThreads) void gdn_prefill_scan_kernel(PrefillParams p, const _Float16 *ws) {
    using L = ScanSmem<C>;
    constexpr int NT = L::NT, KBC = L::KBC, VP = L::VP;
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
    // tokens of this sequence and where they sit: padded layout, (b, h) at token pair * Ts and
    // workspace chunks 0 .. NC - 1 of (b, key head) / (b, h); packed sequences, sequence b at
    // the first token and workspace chunk the sequence table gives, in the one token axis
    int T = p.T;
    int64_t tok = (int64_t)pair * p.Ts;                       // first token in the token-major arrays
    int64_t wkey = (int64_t)b * p.Hk + kh, wpair = pair;      // workspace rows
    int c0 = 0;                                               // first workspace chunk
    if (p.seqs) {
        const int32_t *e = p.seqs + 4 * b;
        T = e[1];
        tok = (int64_t)h * p.Ts + e[0];
        wkey = kh;
        wpair = h;
        c0 = e[2];
    }
    const int NC = (T + C - 1) / C;
    const ChunkWs<C> wl(p.seqs ? 1 : p.B, p.Hk, p.Hv, p.seqs ? p.nchunks : NC);

    if (w == 0) {
        // ================================================================ state wave
        // S[jt][r] = state[16 dvb + li][16 jt + 4 q4 + r]
        const int64_t srow = ((int64_t)pair * kD + kRows * dvb + li) * kD + 4 * q4;
        f32x4 S[8];
#pragma unroll
        for (int jt = 0; jt < 8; ++jt)
            S[jt] = p.init_state ? load_state4(p.init_state, srow + 16 * jt, p.init_f16, p.state_bf16) : f32x4{0.f, 0.f, 0.f, 0.f};
        // fp16 copy of S in fragment order: B operand of X = K S^T, and the helpers' copy
        f16x8 sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
        unsigned char *s16 = smem + L::kS16 + lane * 16;
        unsigned char *u16 = smem + L::kU16 + lane * 16;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<f16x8 *>(s16 + kb * 1024) = sb[kb];

        // per-lane LDS addresses (slot, tile and block offsets are immediates). In the k tile,
        // group g of row t holds columns frag_col(g / 4, g % 4, 0..7) at position g ^ ksw(t % 16).
        // X operand, k block kb: row 16 m + li, group 4 kb + q4 (one 16-byte read)
        const unsigned char *xa[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) xa[kb] = smem + L::rK + li * 256 + (((4 * kb + q4) ^ ksw(li)) << 4);
        // K^T operand of the update, column tile jt: source row 4 q4 + (li >> 2) (+32 kb + 16 hh)
        // holds columns 16 jt + 4 (li & 3) .. +3 in group 4 (jt / 2) + (li & 3), half jt % 2
        const unsigned char *ta[8];
        {
            const int rt = 4 * q4 + (li >> 2);
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                const int g = 4 * (jt >> 1) + (li & 3);
                ta[jt] = smem + L::rK + rt * 256 + ((g ^ ksw(rt)) << 4) + (jt & 1) * 8;
            }
        }
        const unsigned char *tfa = smem + L::rT + lane * 16;
        const unsigned char *bva = smem + L::gBV + li * VP * 4 + 16 * q4;
        const unsigned char *bga = smem + L::gGT + 16 * q4;
        const unsigned char *ega = smem + L::gGT + 256 + 16 * q4;
        lds_barrier();
        // X's k fragments are read one chunk ahead: the k tile of chunk c + 1 is in LDS during
        // chunk c, so its reads overlap the end of chunk c instead of starting chunk c + 1
        f16x8 xk[NT][4];
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) xk[m][kb] = ld8(xa[kb] + m * 4096);

        for_chunks(NC, [&](auto sl, int c) {
            constexpr int s = decltype(sl)::value;
            constexpr int par = s & 1;
            // The remaining LDS operands of the chunk are requested in two batches, in the order
            // of use, so that the MFMAs wait on in-order LDS returns rather than on one round
            // trip each: T, beta*v and beta*gamma now; the K^T fragments of the update once the
            // X products are issued.
            f16x8 Tf[NT][KBC];
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    if (kb <= m / 2) Tf[m][kb] = ld8(tfa + s * 2 * C * C + (m * KBC + kb) * 1024);
            f32x4 bv[NT], bg[NT], ge[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                bv[m] = ldf4(bva + par * 4 * kRows * VP + 64 * m);
                bg[m] = ldf4(bga + par * 768 + 64 * m);
            }
            __builtin_amdgcn_sched_barrier(0);

            // X = K S^T
            f32x4 X[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                X[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) X[m] = mfma16x16x32(xk[m][kb], sb[kb], X[m]);
            }
            __builtin_amdgcn_sched_barrier(0);
            f16x8 ktf[8][KBC];
#pragma unroll
            for (int jt = 0; jt < 8; ++jt)
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    ktf[jt][kb] = cat(ld_tr(ta[jt] + s * 256 * C + kb * 8192),
                                      ld_tr(ta[jt] + s * 256 * C + kb * 8192 + 4096));
#pragma unroll
            for (int m = 0; m < NT; ++m) ge[m] = ldf4(ega + par * 768 + 64 * m);
            const float gC = *reinterpret_cast<const float *>(smem + L::gGT + par * 768 + 512 + 4 * (C - 1));
            __builtin_amdgcn_sched_barrier(0);

            // R = beta V - beta gamma X;  U = T R
            f16x8 rb[KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb)
                rb[kb] = pack8(bv[2 * kb] - bg[2 * kb] * X[2 * kb], bv[2 * kb + 1] - bg[2 * kb + 1] * X[2 * kb + 1]);
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
                *reinterpret_cast<f16x8 *>(u16 + (par * KBC + kb) * 1024) = pack8(U[2 * kb], U[2 * kb + 1]);
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
            __builtin_amdgcn_sched_barrier(0);
            // X's k fragments of chunk c + 1 (after the last chunk this reads a stale slot, unused)
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) xk[m][kb] = ld8(xa[kb] + ((s + 1) % kSlots) * 256 * C + m * 4096);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
                *reinterpret_cast<f16x8 *>(s16 + ((1 - par) * 4 + kb) * 1024) = sb[kb];
            }
            lds_barrier();
        });
        if (p.final_state) {
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) store_state4(p.final_state, srow + 16 * jt, S[jt], p.final_f16, p.state_bf16);
        }
        lds_barrier();
    } else if (w == 4) {
        // ================================================================ prefetch wave
        // Lines of chunk c: the key block (k tile and q fragments, 4 C lines) shared by the
        // 8 * ratio workgroups of this key head; the pair block (T, A_qk, gates) and the v rows
        // (2 lines per token) shared by the 8 row blocks of this value head. Sharer s touches
        // lines s, s + S, s + 2 S, ... of each.
        const int S = 8 * ratio, sk = jj * 8 + dvb;
        constexpr int kKeyLines = 4 * C;
        constexpr int kPairLines = (int)((ChunkWs<C>::kPairElems * 2 + 127) / 128);
        const int nk = (kKeyLines + S - 1) / S;  // key lines per sharer
        constexpr int np = (kPairLines + 7) / 8, nv = C / 4;
        const int total = nk + np + nv;
        const unsigned char *wsb = reinterpret_cast<const unsigned char *>(ws);
        const unsigned char *vb = static_cast<const unsigned char *>(p.v) + tok * kD * 2;
        unsigned char *junk = smem + L::kJunk;
        auto touch = [&](int c) {
            const int n = min(C, T - c * C);
            for (int l0 = 0; l0 < total; l0 += 64) {
                const int l = l0 + lane;
                // lanes with nothing to touch repeat a line of the key block
                const unsigned char *a = wsb + wl.key_chunk(wkey, c0 + c) * 2 + (sk % kKeyLines) * 128;
                if (l < nk) {
                    const int line = sk + S * l;
                    if (line < kKeyLines) a = wsb + wl.key_chunk(wkey, c0 + c) * 2 + (int64_t)line * 128;
                } else if (l < nk + np) {
                    const int line = dvb + 8 * (l - nk);
                    if (line < kPairLines) a = wsb + wl.pair_chunk(wpair, c0 + c) * 2 + (int64_t)line * 128;
                } else if (l < total) {
                    const int line = dvb + 8 * (l - nk - np);
                    a = vb + ((int64_t)c * C + min(line >> 1, n - 1)) * kD * 2 + (line & 1) * 128;
                }
                dma4(a, junk);
            }
        };
        // o rows of chunk c (staged in LDS buffer c & 1 by the output waves): lane l stores row
        // 16 i + l / 4, columns 4 (l % 4) .. + 3 of this block; rows past the end fall outside
        // the buffer range and are dropped
        // (float16 o: the same rows and columns, rounded to nearest even, 8 bytes per lane)
        const int osz = p.o_f16 ? 2 : 4;
        auto store_o = [&](int c) {
            const int tp0 = c * C, np = min(C, T - tp0);
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<char *>(p.o) + (tok + tp0) * kD * osz, 0, np * kD * osz, kBufferFlags);
            const float *src = reinterpret_cast<const float *>(smem + L::kOst + (c & 1) * C * kRows * 4);
#pragma unroll
            for (int i = 0; i < C / 16; ++i) {
                const int row = 16 * i + (lane >> 2), col = 4 * (lane & 3);
                const f32x4 v4 = *reinterpret_cast<const f32x4 *>(src + row * kRows + col);
                const int off = (row * kD + kRows * dvb + col) * osz;
                if (p.o_f16)
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_f16x4(v4)), orsrc, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), orsrc, off, 0, 0);
            }
        };
        for (int c = 3; c < min(NC, kPrefetchAhead); ++c) {
            touch(c);
            wait_vmcnt<8>();
        }
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (c + kPrefetchAhead < NC) touch(c + kPrefetchAhead);
            if (c >= 2) store_o(c - 2);  // staged in the interval before the last barrier
            wait_vmcnt<16>();
            lds_barrier();
        }
        if (NC >= 2) store_o(NC - 2);
        lds_barrier();
        if (NC >= 1) store_o(NC - 1);
        wait_vmcnt<0>();  // the prefetches write into this workgroup's LDS
    } else if (w == 1 || w == 5) {
        // ================================================================ loader waves
        // Direct-to-LDS loads of chunk c (wave 1: L::kDmaK instructions, wave 5: L::kDmaT)
        const bool kload = w == 1;
        const uint16_t *vg = static_cast<const uint16_t *>(p.v) + tok * kD + kRows * dvb;
        // v rows and gate vectors of chunk c into ring slot c % 4 (C / 32 + 1 instructions)
        auto issue_vg = [&](int c) {
            const int s = c % kSlots;
            const int t0 = c * C, last = min(C, T - t0) - 1;
            unsigned char *vb = smem + L::rV + s * 32 * C;
#pragma unroll
            for (int i = 0; i < C / 32; ++i) {
                const int t = 32 * i + (lane >> 1);
                dma16(vg + (int64_t)(t0 + min(t, last)) * kD + 8 * (lane & 1), vb + i * 1024);
            }
            if (lane < 3 * C / 4) dma16(ws + wl.pair_chunk(wpair, c0 + c) + 2 * C * C + lane * 8, smem + L::rG + s * 12 * C);
        };
        // load group c: wave 1 the k tile of chunk c; wave 5 the T fragments of chunk c and the
        // v rows and gates of chunk c + 1 (one chunk earlier, because the output waves form the
        // beta*v block of chunk c + 1 from them while the state wave works on chunk c)
        auto issue = [&](int c) {
            const int s = c % kSlots;
            if (kload) {
                const _Float16 *kw = ws + wl.key_chunk(wkey, c0 + c);
                unsigned char *kb_ = smem + L::rK + s * 256 * C;
#pragma unroll
                for (int i = 0; i < C / 4; ++i) dma16(kw + (i * 64 + lane) * 8, kb_ + i * 1024);
            } else {
                const _Float16 *pw = ws + wl.pair_chunk(wpair, c0 + c);
                unsigned char *tb = smem + L::rT + s * 2 * C * C;
#pragma unroll
                for (int m = 0; m < NT; ++m)
#pragma unroll
                    for (int kb = 0; kb <= m / 2 && kb < KBC; ++kb)
                        dma16(pw + ((m * KBC + kb) * 64 + lane) * 8, tb + (m * KBC + kb) * 1024);
                // past the last chunk the group repeats the last chunk's v and gates, which
                // keeps the instruction count per group fixed; the slot written is free
                issue_vg(min(c + 1, NC - 1));
            }
        };
        // wait until chunk c's loads have landed, given how many chunks were issued after it
        // (the k tile is waited for one chunk earlier than the rest: see the state wave)
        auto wait_for = [&](int c) {
            if (kload) {
                const int after = min(NC - 1, c + 1) - c;
                if (after >= 1) wait_vmcnt<L::kDmaK>();
                else wait_vmcnt<0>();
            } else {
                const int after = min(NC - 1, c + 2) - c;
                if (after >= 2) wait_vmcnt<2 * L::kDmaT>();
                else if (after == 1) wait_vmcnt<L::kDmaT>();
                else wait_vmcnt<0>();
            }
        };

        if (NC > 0 && !kload) issue_vg(0);
        for (int c = 0; c < min(NC, 3); ++c) issue(c);
        if (NC > 0) {
            wait_for(kload ? min(1, NC - 1) : 0);
            if (!kload) {  // chunk 0's operands; the output waves form those of the later chunks
                prepare_chunk_impl<C>(smem, 0, 0, true, lane);
                prepare_chunk_impl<C>(smem, 0, 1, false, lane);
            }
        }
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (c + 3 < NC) issue(c + 3);
            const int next = kload ? c + 2 : c + 1;
            if (next < NC) wait_for(next);
            lds_barrier();
        }
        lds_barrier();
    } else {
        // ================================================================ output waves
        // Wave ow owns token tiles ow and ow + 2 (NT is even). The steady-state loop below is
        // branch-free: prefetches past the last chunk re-read the last chunk (never used) and o
        // rows past the sequence end fall outside the store's buffer range, so every trip issues
        // the same memory operations and the compiler's vmcnt waits stay exact instead of
        // draining the prefetch queue.
        static_assert(NT % 2 == 0, "two token tiles per output wave");
        constexpr int MAXT = NT / 2;
        const int ow = w - 2;  // 0 or 1 (waves 2 and 3)
        f32x4 Y[MAXT];   // lane (q4, li): Y^T[state row 4 q4 + r][token 16 m + li]
        float gmy[MAXT];  // gamma of token 16 m + li
        f16x8 qf[2][MAXT][4];         // q fragments, double-buffered by chunk parity
        f16x8 aqk[2][MAXT][KBC];      // A_qk fragments, double-buffered by chunk parity
        const _Float16 *qsrc0 = ws + wl.key_chunk(wkey, c0) + C * kD + lane * 8;
        const _Float16 *asrc0 = ws + wl.pair_chunk(wpair, c0) + C * C + lane * 8;
        auto load_q = [&](auto parc, int c) {
            constexpr int par = decltype(parc)::value;
            const _Float16 *src = qsrc0 + min(c, NC - 1) * ChunkWs<C>::kKeyElems;
#pragma unroll
            for (int s2 = 0; s2 < MAXT; ++s2)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    qf[par][s2][kb] = *reinterpret_cast<const f16x8 *>(src + ((ow + 2 * s2) * 4 + kb) * 512);
        };
        auto load_aqk = [&](auto parc, int c) {
            constexpr int par = decltype(parc)::value;
            const _Float16 *src = asrc0 + min(c, NC - 1) * ChunkWs<C>::kPairElems;
#pragma unroll
            for (int s2 = 0; s2 < MAXT; ++s2)
#pragma unroll
                for (int kb = 0; kb <= s2 && kb < KBC; ++kb)  // tile m = ow + 2 s2 needs k blocks kb <= m / 2 = s2
                    aqk[par][s2][kb] = *reinterpret_cast<const f16x8 *>(src + ((ow + 2 * s2) * KBC + kb) * 512);
        };
        const unsigned char *s16 = smem + L::kS16 + lane * 16;
        const unsigned char *u16 = smem + L::kU16 + lane * 16;
        auto emit_o = [&](auto parc, int c) {  // O of chunk c from buffer parity par = c & 1, into LDS
            constexpr int par = decltype(parc)::value;
            float *ost = reinterpret_cast<float *>(smem + L::kOst + par * C * kRows * 4) + li * kRows + 4 * q4;
#pragma unroll
            for (int s2 = 0; s2 < MAXT; ++s2) {
                const int m = ow + 2 * s2;
                f32x4 acc = (gmy[s2] * p.scale) * Y[s2];
#pragma unroll
                for (int kb = 0; kb <= s2 && kb < KBC; ++kb)
                    acc = mfma16x16x32(ld8(u16 + (par * KBC + kb) * 1024), aqk[par][s2][kb], acc);
                // o[16 m + li][16 dvb + 4 q4 + r], r = 0..3
                *reinterpret_cast<f32x4 *>(ost + 16 * m * kRows) = acc;
            }
        };
        // Y^T = S Q^T of chunk c with S the state at the chunk start, and gamma of its tokens
        auto chunk_y = [&](auto parc, int c) {
            constexpr int par = decltype(parc)::value;
            const float *gam = reinterpret_cast<const float *>(smem + L::gGT + par * 768 + 512) + li;
            f16x8 sbf[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sbf[kb] = ld8(s16 + (par * 4 + kb) * 1024);
#pragma unroll
            for (int s2 = 0; s2 < MAXT; ++s2) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc = mfma16x16x32(sbf[kb], qf[par][s2][kb], acc);
                Y[s2] = acc;
                gmy[s2] = gam[16 * (ow + 2 * s2)];
            }
        };
        // interval of chunk c >= 1: O of chunk c - 1, then Y of chunk c; prefetches run two
        // chunks (q) and one chunk (A_qk) ahead of their use. Then the beta*v block and gate
        // operands of chunk c + 1 (its v rows and gates landed before this interval): wave ow
        // forms columns 8 ow .. 8 ow + 7, wave 0 also the gate operands.
        auto interval = [&](auto parc, int c) {
            constexpr int par = decltype(parc)::value;
            emit_o(IC<1 - par>{}, c - 1);
            load_aqk(IC<1 - par>{}, c + 1);
            chunk_y(IC<par>{}, c);
            load_q(IC<par>{}, c + 2);
            if (c + 1 < NC) prepare_chunk_impl<C>(smem, c + 1, ow, ow == 0, lane);
            lds_barrier();
        };

        if (NC == 0) {  // empty sequence: nothing to read (the workspace may be empty)
            lds_barrier();
            lds_barrier();
        } else {
            // same issue order as the steady state: A_qk of c - 1, q of c, A_qk of c, q of c + 1
            load_q(IC<0>{}, 0);
            load_aqk(IC<0>{}, 0);
            load_q(IC<1>{}, 1);
            lds_barrier();
            load_aqk(IC<1>{}, 1);
            chunk_y(IC<0>{}, 0);
            load_q(IC<0>{}, 2);
            if (1 < NC) prepare_chunk_impl<C>(smem, 1, ow, ow == 0, lane);
            lds_barrier();
            int c = 1;
            for (; c + 1 < NC; c += 2) {
                interval(IC<1>{}, c);
                interval(IC<0>{}, c + 1);
            }
            if (c < NC) interval(IC<1>{}, c);
            if ((NC - 1) & 1) emit_o(IC<1>{}, NC - 1);
            else emit_o(IC<0>{}, NC - 1);
            lds_barrier();
        }
    }
}

template <int C>
hipError_t launch_c(const PrefillParams &p, const _Float16 *ws, hipStream_t stream) {
    const size_t bytes = ScanSmem<C>::kBytes;
    static bool attr_set = false;  // the attribute is a property of the function: set once
    if (!attr_set) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_prefill_scan_kernel<C>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
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
