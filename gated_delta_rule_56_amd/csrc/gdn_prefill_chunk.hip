// Chunk-parallel half of the bf16 prefill: everything of a chunk that does not
// depend on the state, computed for all chunks at once.
//
// For one (b, value head h) and chunk of C tokens (local t, rows past the end are
// zero with g = beta = 0):
//   G_t = sum_{s<=t} g_s,  Gamma_ts = exp(G_t - G_s) (s <= t)
//   A     = strict_lower(diag(beta) (K K^T o Gamma))
//   T     = (I + A)^{-1}                       (unit lower triangular)
//   A_qk  = lower_incl(scale Q K^T o Gamma)
// Outputs (the workspace, layout in gdn_frag.h):
//   per (b, h, chunk): T and A_qk as fp16 C x C matrices in per-lane MFMA fragment
//     order, so that a lane fetches each operand fragment with one coalesced 16-byte
//     load (only the fragments on or below the diagonal, k block kb <= m / 2 of token
//     tile m, are written: the others are never read); then gamma_t = exp(G_t),
//     beta_t and exp(G_C - G_t) as float[C] each (zero beta past the sequence end);
//   per (b, key head, chunk): the k tile in fp16 (each 32-column block in fragment
//     order, 16-byte groups swizzled by row, see ksw), ready to be copied verbatim
//     into LDS by the state-pass kernel, and q in per-lane fragment order.
//
// One workgroup per (b, key head, chunk), one wave per 16-token tile m, looping over
// the value heads that read this key head: K K^T and Q K^T do not depend on the
// value head, so they are formed once (exactly, by bf16 MFMAs on the raw inputs)
// and only the gating and the inverse are redone per value head. Wave m holds the
// tiles of its token rows transposed, lane (q, c) holding row 16 m + c at columns
// 16 nt + 4 q + r, which is directly the A-operand fragment of the scan's MFMAs.
//
// The inverse follows the forward substitution of the tinygrad helper
// inverse_unit_lower (compare page "27b 935/47", llm/kernels/generic.py: the
// inverse of I - x for strictly lower-triangular x, here x = -A), organised in
// 16 x 16 blocks: the diagonal blocks by substitution in fp32 (one wave each),
// then the off-diagonal blocks by MFMA recursive doubling,
//   T_ul = -T_uu A_ul T_ll  (16-blocks, then 32-blocks).
#include "gdn_device.h"
#include "gdn_frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;

template <int C>
struct PrepSmem {
    static constexpr int NT = C / 16;                        // token tiles = waves
    static constexpr int CP = C + 8;                         // fp16 pitch of A and T
    static constexpr int DP = 20;                            // f32 pitch of a transposed diagonal block
    static constexpr size_t kKx = 0;                         // [NT][4][64] x 16 B: k fragments (bf16)
    static constexpr size_t kAh = kKx + NT * 4 * 64 * 16;    // fp16 [C][CP]: gated A (lower tiles)
    static constexpr size_t kTm = kAh + 2 * C * CP;          // fp16 [C][CP]: T
    static constexpr size_t kAd = kTm + 2 * C * CP;          // f32 [NT][16][DP]: diagonal blocks of A, transposed
    static constexpr size_t kG = kAd + 4 * NT * 16 * DP;     // f32 [NT][2][64]: per-wave G and beta
    static constexpr size_t kBytes = kG + 4 * NT * 128;
    static_assert(kAh % 16 == 0 && kAd % 16 == 0 && kG % 16 == 0, "alignment");
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// D += A B with bf16 operands (fragment layout as mfma16x16x32); products of bf16
// values are exact in fp32
__device__ __forceinline__ f32x4 mfma_bf16(u16x8 a, u16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 bf16x8_to_f16(u16x8 u) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)bf16_bits_to_f32(u[e]);
    return r;
}

__device__ __forceinline__ f16x4 ld4(const _Float16 *p) { return *reinterpret_cast<const f16x4 *>(p); }

template <int C>
__global__ __launch_bounds__(C * 4) void gdn_chunk_prep_kernel(PrefillParams p, _Float16 *ws) {
    using L = PrepSmem<C>;
    constexpr int NT = L::NT, CP = L::CP, DP = L::DP, KBC = C / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *Ah = reinterpret_cast<_Float16 *>(smem + L::kAh);
    _Float16 *Tm = reinterpret_cast<_Float16 *>(smem + L::kTm);

    // padded layout: chunk c of sequence b at token c C; packed sequences: workspace chunk c
    // of the one token axis, at the token the chunk table gives (tokens 0: an unused slot)
    const int NC = p.chunks ? p.nchunks : (p.T + C - 1) / C;
    const ChunkWs<C> wl(p.chunks ? 1 : p.B, p.Hk, p.Hv, NC);
    const int c = blockIdx.x % NC;
    const int bk = blockIdx.x / NC;  // b * Hk + key head
    const int b = bk / p.Hk, kh = bk % p.Hk;
    const int ratio = p.Hv / p.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int m = __builtin_amdgcn_readfirstlane(tid >> 6);  // token tile of this wave
    const int li = lane & 15, q4 = lane >> 4;
    int t0 = c * C, n = min(C, p.T - t0);
    if (p.chunks) {
        t0 = p.chunks[2 * c];
        n = p.chunks[2 * c + 1];
        if (n <= 0) return;  // the whole workgroup: no barrier has been reached yet
    }
    const int t = 16 * m + li;  // token row of this lane in the fragments below
    const bool live = t < n;

    // ---- all global loads first: q, k fragments of tile m (lane: row t, columns
    // frag_col(kb, q4, 0..7)), and g, beta of the first value head
    u16x8 qf[4], kf[4];
    {
        const int64_t row = ((int64_t)bk * p.Ts + t0 + min(t, n - 1)) * kD + 4 * q4;
        const uint16_t *qr = static_cast<const uint16_t *>(p.q) + row;
        const uint16_t *kr = static_cast<const uint16_t *>(p.k) + row;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const u16x4 qa = *reinterpret_cast<const u16x4 *>(qr + 32 * kb);
            const u16x4 qb = *reinterpret_cast<const u16x4 *>(qr + 32 * kb + 16);
            const u16x4 ka = *reinterpret_cast<const u16x4 *>(kr + 32 * kb);
            const u16x4 kb_ = *reinterpret_cast<const u16x4 *>(kr + 32 * kb + 16);
            qf[kb] = u16x8{qa[0], qa[1], qa[2], qa[3], qb[0], qb[1], qb[2], qb[3]};
            kf[kb] = u16x8{ka[0], ka[1], ka[2], ka[3], kb_[0], kb_[1], kb_[2], kb_[3]};
        }
    }
    auto value_head = [&](int j) { return p.head_map == 0 ? kh + j * p.Hk : kh * ratio + j; };
    float g_next = 0.f, b_next = 0.f;
    auto load_gb = [&](int j) {
        const int64_t base = ((int64_t)b * p.Hv + value_head(j)) * p.Ts + t0;
        g_next = lane < n ? p.g[base + lane] : 0.f;
        b_next = lane < n ? p.beta[base + lane] : 0.f;
    };
    load_gb(0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {  // rows past the end are zero
        if (!live) qf[kb] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (!live) kf[kb] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    // ---- k fragments for the other waves; the key block of the workspace
    unsigned char *kx = smem + L::kKx + lane * 16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<u16x8 *>(kx + (m * 4 + kb) * 1024) = kf[kb];
    {
        _Float16 *kw = ws + wl.key_chunk(bk, c);
        _Float16 *qw = kw + C * kD;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            // k: group 4 kb + q4 of row t at position (4 kb + q4) ^ ksw(t % 16)
            *reinterpret_cast<f16x8 *>(kw + ((int64_t)t * 16 + ((4 * kb + q4) ^ ksw(li))) * 8) = bf16x8_to_f16(kf[kb]);
            // q: [m][kb][lane][8]
            *reinterpret_cast<f16x8 *>(qw + ((m * 4 + kb) * 64 + lane) * 8) = bf16x8_to_f16(qf[kb]);
        }
    }
    // the upper blocks of T inside the written fragments ((0, 1) and (2, 3)) stay zero
    if (m % 2 == 0 && m + 1 < NT) {
        for (int e = lane; e < 16 * 16; e += 64)
            Tm[(16 * m + (e >> 4)) * CP + 16 * (m + 1) + (e & 15)] = (_Float16)0.0f;
    }
    __syncthreads();

    // ---- raw products of tile m against tiles nt <= m, transposed: lane (q4, li) holds
    // rk[nt][r] = k_t . k_s and rq[nt][r] = q_t . k_s for t = 16 m + li, s = 16 nt + 4 q4 + r
    f32x4 rk[NT], rq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        rk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        rq[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (nt <= m) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const u16x8 a = *reinterpret_cast<const u16x8 *>(kx + (nt * 4 + kb) * 1024);
                rk[nt] = mfma_bf16(a, kf[kb], rk[nt]);
                rq[nt] = mfma_bf16(a, qf[kb], rq[nt]);
            }
        }
    }

    float *gtab = reinterpret_cast<float *>(smem + L::kG) + m * 128;  // this wave's G and beta
    float *adt = reinterpret_cast<float *>(smem + L::kAd) + m * 16 * DP;
    for (int j = 0; j < ratio; ++j) {
        const float gl = g_next, bl = b_next;
        if (j + 1 < ratio) load_gb(j + 1);
        const int64_t pair = (int64_t)b * p.Hv + value_head(j);
        _Float16 *pw = ws + wl.pair_chunk(pair, c);

        // G = inclusive prefix sum of g over the chunk
        float G = gl;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(G, o, 64);
            if (lane >= o) G += y;
        }
        gtab[lane] = G;
        gtab[64 + lane] = bl;
        if (m == 0 && lane < C) {
            const float gC = __shfl(G, C - 1, 64);
            float *gates = reinterpret_cast<float *>(pw + 2 * C * C);
            gates[lane] = __expf(G);
            gates[C + lane] = bl;
            gates[2 * C + lane] = __expf(gC - G);
        }

        // gating: A[t][s] (s < t) and A_qk[t][s] (s <= t)
        const float Gt = gtab[t], bt = gtab[64 + t];
        f32x4 a[NT], aq[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt <= m) {
                const f32x4 Gs = *reinterpret_cast<const f32x4 *>(gtab + 16 * nt + 4 * q4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * nt + 4 * q4 + r;
                    const float gate = __expf(Gt - Gs[r]);
                    a[nt][r] = s < t ? bt * gate * rk[nt][r] : 0.0f;
                    aq[nt][r] = s <= t ? p.scale * gate * rq[nt][r] : 0.0f;
                }
                *reinterpret_cast<f16x4 *>(Ah + t * CP + 16 * nt + 4 * q4) = to_f16x4(a[nt]);
            } else {
                a[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                aq[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        // A_qk fragments of tile m: k block kb = tiles 2 kb and 2 kb + 1
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb)
            if (2 * kb <= m)
                *reinterpret_cast<f16x8 *>(pw + C * C + ((m * KBC + kb) * 64 + lane) * 8) =
                    cat(to_f16x4(aq[2 * kb]), to_f16x4(aq[2 * kb + 1]));

        // diagonal block T_mm = (I + A_mm)^{-1} by forward substitution in fp32, lane li
        // computing column li; A_mm goes through LDS transposed, adt[s][i] = A[i][s]
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
                    col[4 * v] = c4[0]; col[4 * v + 1] = c4[1]; col[4 * v + 2] = c4[2]; col[4 * v + 3] = c4[3];
                }
#pragma unroll
                for (int r = s2 + 1; r < 16; ++r) x[r] -= col[r] * x[s2];
            }
            // lane group q4 writes rows 4 q4 .. 4 q4 + 3 of column li
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = q4 == 0 ? x[r] : q4 == 1 ? x[4 + r] : q4 == 2 ? x[8 + r] : x[12 + r];
                Tm[(16 * m + 4 * q4 + r) * CP + 16 * m + li] = (_Float16)v;
            }
        }
        __syncthreads();

        // level 1: T_{u,l} = -T_{u,u} A_{u,l} T_{l,l} for (l, u) = (0, 1), (2, 3)
        if (m < NT / 2) {
            const int lo = 2 * m, up = 2 * m + 1;
            f16x4 btl;
#pragma unroll
            for (int e = 0; e < 4; ++e) btl[e] = Tm[(16 * lo + 4 * q4 + e) * CP + 16 * lo + li];
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 pm = mfma16x16x16(ld4(Ah + (16 * up + li) * CP + 16 * lo + 4 * q4), btl, z);
            const f32x4 out = mfma16x16x16(ld4(Tm + (16 * up + li) * CP + 16 * up + 4 * q4), to_f16x4(-pm), z);
#pragma unroll
            for (int r = 0; r < 4; ++r) Tm[(16 * up + 4 * q4 + r) * CP + 16 * lo + li] = (_Float16)out[r];
        }
        if constexpr (NT == 4) {
            __syncthreads();
            // level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32]; wave j: column block j
            if (m < 2) {
                const int jc = m;
                f16x4 t0j, t1j;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t0j[e] = Tm[(4 * q4 + e) * CP + 16 * jc + li];
                    t1j[e] = Tm[(16 + 4 * q4 + e) * CP + 16 * jc + li];
                }
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                f32x4 p0 = mfma16x16x16(ld4(Ah + (32 + li) * CP + 16 + 4 * q4), t1j, z);
                f32x4 p1 = mfma16x16x16(ld4(Ah + (48 + li) * CP + 16 + 4 * q4), t1j, z);
                if (jc == 0) {
                    p0 = mfma16x16x16(ld4(Ah + (32 + li) * CP + 4 * q4), t0j, p0);
                    p1 = mfma16x16x16(ld4(Ah + (48 + li) * CP + 4 * q4), t0j, p1);
                }
                const f16x4 b0 = to_f16x4(-p0), b1 = to_f16x4(-p1);
                const f32x4 o0 = mfma16x16x16(ld4(Tm + (32 + li) * CP + 32 + 4 * q4), b0, z);
                f32x4 o1 = mfma16x16x16(ld4(Tm + (48 + li) * CP + 32 + 4 * q4), b0, z);
                o1 = mfma16x16x16(ld4(Tm + (48 + li) * CP + 48 + 4 * q4), b1, o1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Tm[(32 + 4 * q4 + r) * CP + 16 * jc + li] = (_Float16)o0[r];
                    Tm[(48 + 4 * q4 + r) * CP + 16 * jc + li] = (_Float16)o1[r];
                }
            }
        }
        __syncthreads();

        // T fragments of tile m, k blocks kb <= m / 2: lane (q4, li) holds row t at
        // columns frag_col(kb, q4, 0..7)
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb)
            if (2 * kb <= m) {
                const _Float16 *src = Tm + t * CP + 32 * kb + 4 * q4;
                *reinterpret_cast<f16x8 *>(pw + ((m * KBC + kb) * 64 + lane) * 8) = cat(ld4(src), ld4(src + 16));
            }
        // the next value head rewrites Ah and Tm only after its first barrier, which
        // every wave reaches after these reads; the diagonal block of Tm is read and
        // rewritten by its own wave only
    }
}

template <int C>
hipError_t launch_c(const PrefillParams &p, _Float16 *ws, hipStream_t stream) {
    const size_t bytes = PrepSmem<C>::kBytes;
    static bool attr_set = false;  // the attribute is a property of the function: set once
    if (!attr_set) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_chunk_prep_kernel<C>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    const int64_t NC = p.chunks ? p.nchunks : (p.T + C - 1) / C;
    const int64_t nb = (p.chunks ? 1 : p.B) * p.Hk * NC;
    if (nb > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)nb), block(C * 4);
    hipLaunchKernelGGL((gdn_chunk_prep_kernel<C>), grid, block, bytes, stream, p, ws);
    return hipGetLastError();
}

}  // namespace

namespace {
int64_t chunk_ws_bytes(int64_t B, int64_t Hk, int64_t Hv, int64_t nc, int chunk) {
    if (chunk == 32) return ChunkWs<32>(B, Hk, Hv, nc).bytes();
    if (chunk == 64) return ChunkWs<64>(B, Hk, Hv, nc).bytes();
    return 0;
}
}  // namespace

VarlenLayout varlen_layout(int64_t nseq, int64_t Hk, int64_t Hv, int64_t T, int chunk) {
    VarlenLayout v{0, 0, 0, 0};
    if (nseq < 1 || T < 0 || (chunk != 32 && chunk != 64)) return v;
    // every sequence rounds up to whole chunks: at most one partial chunk per sequence
    v.nchunks = (T + chunk - 1) / chunk + nseq;
    v.seq_offset = (chunk_ws_bytes(1, Hk, Hv, v.nchunks, chunk) + 255) / 256 * 256;
    v.chunk_offset = v.seq_offset + (nseq * 16 + 255) / 256 * 256;
    v.bytes = v.chunk_offset + v.nchunks * 8;
    return v;
}

hipError_t launch_chunk_prep(const PrefillParams &p, int chunk, void *ws, hipStream_t stream) {
    if (p.D != kD || p.T <= 0) return hipErrorInvalidValue;
    _Float16 *w = static_cast<_Float16 *>(ws);
    switch (chunk) {
        case 32: return launch_c<32>(p, w, stream);
        case 64: return launch_c<64>(p, w, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
