// Chunk-parallel half of the bf16 prefill: everything of a chunk that does not
// depend on the state, computed for all chunks at once.
//
// For one (b, h) and chunk of C tokens (local t, rows past the end are zero with
// g = beta = 0):
//   G_t = sum_{s<=t} g_s,  Gamma_ts = exp(G_t - G_s) (s <= t)
//   A     = strict_lower(diag(beta) (K K^T o Gamma))
//   T     = (I + A)^{-1}                       (unit lower triangular)
//   A_qk  = lower_incl(scale Q K^T o Gamma)
// Outputs (the workspace, see chunk_ws_layout):
//   per (b, h, chunk): T and A_qk as fp16 C x C matrices in per-lane MFMA fragment
//     order (gdn_frag.h), so a lane fetches each operand fragment with one
//     coalesced 16-byte load; then gamma_t = exp(G_t), beta_t and exp(G_C - G_t)
//     as float[C] each (zero beta past the sequence end);
//   per (b, key head, chunk): the k tile in fp16 (each 32-column block in fragment
//     order, 16-byte groups swizzled by row, see ksw), ready to be copied verbatim
//     into LDS by the state-pass kernel, and q in per-lane fragment order. Both are
//     written by the first value head of each key head.
// The state kernel then needs only T, A_qk and the chunk's q, k, v, g, beta.
//
// The inverse follows the forward substitution of the tinygrad helper
// inverse_unit_lower (compare page "27b 935/47", llm/kernels/generic.py: the
// inverse of I - x for strictly lower-triangular x, here x = -A), organised in
// 16 x 16 blocks: the four diagonal blocks by substitution in fp32, then the
// off-diagonal blocks by MFMA recursive doubling,
//   T_ul = -T_uu A_ul T_ll  (16-blocks, then 32-blocks).
#include "gdn_device.h"
#include "gdn_frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;

template <int C>
struct ChunkSmem {
    static constexpr int NT = C / 16;
    static constexpr int QP = kD + 8;
    static constexpr int CP = C + 8;
    static constexpr size_t kQ = 0;
    static constexpr size_t kK = kQ + 2 * C * QP;
    static constexpr size_t kG = kK + 2 * C * QP;      // f32 G[64], beta[64]
    static constexpr size_t kAd = kG + 4 * 128;         // f32 [NT][16][17]
    static constexpr size_t kAh = kAd + 4 * NT * 16 * 17;
    static constexpr size_t kAqk = kAh + 2 * C * CP;
    static constexpr size_t kTm = kAqk + 2 * C * CP;
    static constexpr size_t kBytes = kTm + 2 * C * CP;
    static_assert(kAh % 16 == 0, "alignment");
};

__device__ __forceinline__ f16x4 ld4(const _Float16 *p) { return *reinterpret_cast<const f16x4 *>(p); }
__device__ __forceinline__ f16x8 ld8(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

template <int C>
__global__ __launch_bounds__(kThreads) void gdn_chunk_prep_kernel(PrefillParams p, _Float16 *ws) {
    using L = ChunkSmem<C>;
    constexpr int NT = L::NT, QP = L::QP, CP = L::CP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    _Float16 *Qs = reinterpret_cast<_Float16 *>(smem + L::kQ);
    _Float16 *Ks = reinterpret_cast<_Float16 *>(smem + L::kK);
    float *Gs = reinterpret_cast<float *>(smem + L::kG);
    float *Bs = Gs + 64;
    float *Ad = reinterpret_cast<float *>(smem + L::kAd);
    _Float16 *Ah = reinterpret_cast<_Float16 *>(smem + L::kAh);
    _Float16 *Aqk = reinterpret_cast<_Float16 *>(smem + L::kAqk);
    _Float16 *Tm = reinterpret_cast<_Float16 *>(smem + L::kTm);

    const int NC = (p.T + C - 1) / C;
    const ChunkWs<C> wl(p.B, p.Hk, p.Hv, NC);
    const int c = blockIdx.x % NC;
    const int pair = blockIdx.x / NC;
    const int b = pair / p.Hv, h = pair % p.Hv;
    const int kh = key_head(h, p.Hk, p.Hv, p.head_map);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, q4 = lane >> 4;
    const int t0 = c * C;
    const int n = min(C, p.T - t0);
    const uint16_t *qg = static_cast<const uint16_t *>(p.q) + (((int64_t)b * p.Hk + kh) * p.T + t0) * kD;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + (((int64_t)b * p.Hk + kh) * p.T + t0) * kD;

    // zero A, A_qk, T (upper tiles stay zero)
    for (int e = tid; e < 3 * C * CP; e += kThreads) Ah[e] = (_Float16)0.0f;
    // q, k tiles (bf16 -> fp16), zero rows past the end
    for (int idx = tid; idx < C * 16; idx += kThreads) {
        const int row = idx >> 4, c8 = (idx & 15) * 8;
        u16x8 qb = {0, 0, 0, 0, 0, 0, 0, 0}, kb = {0, 0, 0, 0, 0, 0, 0, 0};
        if (row < n) {
            qb = *reinterpret_cast<const u16x8 *>(qg + (int64_t)row * kD + c8);
            kb = *reinterpret_cast<const u16x8 *>(kg + (int64_t)row * kD + c8);
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
    if (w == 0) {
        const float *gg = p.g + (int64_t)pair * p.T + t0;
        float x = (lane < n) ? gg[lane] : 0.0f;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const float y = __shfl_up(x, m, 64);
            if (lane >= m) x += y;
        }
        Gs[lane] = x;
        const float gc = __shfl(x, C - 1, 64);
        float *gates = reinterpret_cast<float *>(ws + wl.pair_chunk(pair, c) + 2 * C * C);
        if (lane < C) {
            gates[lane] = __expf(x);
            gates[2 * C + lane] = __expf(gc - x);
        }
    } else if (w == 1) {
        const float bt = (lane < n) ? p.beta[(int64_t)pair * p.T + t0 + lane] : 0.0f;
        Bs[lane] = bt;
        if (lane < C) reinterpret_cast<float *>(ws + wl.pair_chunk(pair, c) + 2 * C * C)[C + lane] = bt;
    }
    __syncthreads();

    // lower tiles of K K^T -> A and Q K^T -> A_qk
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
            const float gate = __expf(fminf(Gs[t] - gs, 0.0f));
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

    // diagonal 16x16 blocks of T by forward substitution (lane li owns column li)
    if (w < NT) {
        const float *ab = Ad + w * 16 * 17;
        float a[16][16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) a[r][s2] = ab[r * 17 + s2];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == li) ? 1.0f : 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) acc -= a[r][s2] * x[s2];
            x[r] = acc;
        }
        if (q4 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Tm[(16 * w + r) * CP + 16 * w + li] = (_Float16)x[r];
        }
    }
    __syncthreads();
    // level 1: T_{u,l} = -T_{u,u} A_{u,l} T_{l,l} for (l, u) = (0, 1), (2, 3)
    if (w < NT / 2) {
        const int lo = 2 * w, up = 2 * w + 1;
        f16x4 bt;
#pragma unroll
        for (int e = 0; e < 4; ++e) bt[e] = Tm[(16 * lo + 4 * q4 + e) * CP + 16 * lo + li];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pm = mfma16x16x16(ld4(Ah + (16 * up + li) * CP + 16 * lo + 4 * q4), bt, z);
        const f32x4 out = mfma16x16x16(ld4(Tm + (16 * up + li) * CP + 16 * up + 4 * q4), to_f16x4(-pm), z);
#pragma unroll
        for (int r = 0; r < 4; ++r) Tm[(16 * up + 4 * q4 + r) * CP + 16 * lo + li] = (_Float16)out[r];
    }
    if constexpr (NT == 4) {
        __syncthreads();
        // level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32]; wave j: column block j
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
    __syncthreads();

    // write T and A_qk in per-lane fragment order: [mat][m][kb][lane][8], where lane l of
    // token tile m, k block kb holds row 16 m + l % 16 at columns frag_col(kb, l / 16, 0..7)
    constexpr int KBC = C / 32;
    _Float16 *wt = ws + wl.pair_chunk(pair, c);
    for (int idx = tid; idx < 2 * NT * KBC * 64; idx += kThreads) {
        const int l = idx & 63;
        const int f = idx >> 6;            // (mat * NT + m) * KBC + kb
        const int kb = f % KBC, m = (f / KBC) % NT, mat = f / (KBC * NT);
        const _Float16 *src = (mat == 0 ? Tm : Aqk) + (16 * m + (l & 15)) * CP + 32 * kb + 4 * (l >> 4);
        *reinterpret_cast<f16x8 *>(wt + (int64_t)idx * 8) = cat(ld4(src), ld4(src + 16));
    }
    // the fp16 k tile and the q fragments, once per key head
    const int ratio = p.Hv / p.Hk;
    const bool owner = p.head_map == 0 ? (h < p.Hk) : (h % ratio == 0);
    if (owner) {
        _Float16 *kw = ws + wl.key_chunk(b * p.Hk + kh, c);
        // k: group g of row t holds columns frag_col(g / 4, g % 4, 0..7) and sits at g ^ ksw(t % 16)
        for (int idx = tid; idx < C * 16; idx += kThreads) {
            const int t = idx >> 4, g = idx & 15;
            const _Float16 *src = Ks + t * QP + 32 * (g >> 2) + 4 * (g & 3);
            *reinterpret_cast<f16x8 *>(kw + ((int64_t)t * 16 + (g ^ ksw(t & 15))) * 8) = cat(ld4(src), ld4(src + 16));
        }
        // q: per-lane fragments [m][kb][lane][8] for the A operand of Q S^T
        _Float16 *qw = kw + C * 128;
        for (int idx = tid; idx < NT * 4 * 64; idx += kThreads) {
            const int l = idx & 63, kb = (idx >> 6) & 3, m = idx >> 8;
            const _Float16 *src = Qs + (16 * m + (l & 15)) * QP + 32 * kb + 4 * (l >> 4);
            *reinterpret_cast<f16x8 *>(qw + (int64_t)idx * 8) = cat(ld4(src), ld4(src + 16));
        }
    }
}

template <int C>
hipError_t launch_c(const PrefillParams &p, _Float16 *ws, hipStream_t stream) {
    const size_t bytes = ChunkSmem<C>::kBytes;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_chunk_prep_kernel<C>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (err != hipSuccess) return err;
    const int NC = (p.T + C - 1) / C;
    dim3 grid((unsigned)((int64_t)p.B * p.Hv * NC)), block(kThreads);
    hipLaunchKernelGGL((gdn_chunk_prep_kernel<C>), grid, block, bytes, stream, p, ws);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int64_t B, int64_t Hk, int64_t Hv, int64_t T, int chunk) {
    const int64_t nc = (T + chunk - 1) / chunk;
    if (chunk == 32) return ChunkWs<32>(B, Hk, Hv, nc).bytes();
    if (chunk == 64) return ChunkWs<64>(B, Hk, Hv, nc).bytes();
    return 0;
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
