// Fragment order shared by the chunk kernel and the state kernel of the bf16
// prefill path.
//
// A 16x16x32 MFMA contracts 32 values of k per step; lane group q = lane / 16
// holds 8 of them. Any assignment works as long as the A and B operands use the
// same one. We use, within k block kb (32 consecutive k):
//   col(kb, q, e) = 32 kb + 16 (e / 4) + 4 q + (e % 4),   e = 0..7
// because then the two 16x16 result tiles of an MFMA pair (rows 32 kb + 4 q + r
// and 32 kb + 16 + 4 q + r held by lane group q) are directly the B operand of
// the next contraction over that dimension, with no data movement.
// Matrices read as A operands are stored "fragment-permuted": row-major, with
// the value of column col(kb, q, e) at position 32 kb + 8 q + e, so that each
// lane fetches its 8 values with one 16-byte load.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace gdn {

// column held by lane group q, element e of k block kb
__host__ __device__ constexpr int frag_col(int kb, int q, int e) { return 32 * kb + 16 * (e >> 2) + 4 * q + (e & 3); }

// storage position of column c in a fragment-permuted row
__host__ __device__ constexpr int frag_pos(int c) {
    return (c & ~31) + 8 * ((c & 15) >> 2) + 4 * ((c & 31) >> 4) + (c & 3);
}

// Row swizzle of the 16-byte column groups of a 256-byte tile row: group G of row t
// is stored at G ^ ksw(t % 16). ksw is a bijection on 0..15, so the 16 rows read
// by one MFMA operand fetch land in 16 different bank groups, and
// ksw(r) = r ^ ((r & 3) << 2) also keeps the transposing fetches of the k tile
// (4 rows x 4 column runs per 16 lanes) conflict-free.
__host__ __device__ constexpr int ksw(int r) { return r ^ ((r & 3) << 2); }

// Workspace of the bf16 prefill (offsets in fp16 elements):
//   pair block  [B * Hv][NC]: T frags (C*C), A_qk frags (C*C), gamma, beta, exp(G_C - G) (3*C float)
//   key block   [B * Hk][NC]: fp16 k tile (C * 128; each 32-column block in fragment
//               order, then row-swizzled), then q in per-lane fragment order (C * 128)
template <int C>
struct ChunkWs {
    static constexpr int64_t kPairElems = 2 * C * C + 3 * C * 2;  // 3*C floats = 6*C halfs
    static constexpr int64_t kKeyElems = 2 * (int64_t)C * 128;
    int64_t npair_chunks, nkey_chunks, nc;
    __host__ __device__ ChunkWs(int64_t B, int64_t Hk, int64_t Hv, int64_t NC)
        : npair_chunks(B * Hv * NC), nkey_chunks(B * Hk * NC), nc(NC) {}
    __host__ __device__ int64_t pair_chunk(int64_t pair, int64_t c) const { return (pair * nc + c) * kPairElems; }
    __host__ __device__ int64_t key_chunk(int64_t bk, int64_t c) const {
        return npair_chunks * kPairElems + (bk * nc + c) * kKeyElems;
    }
    __host__ __device__ int64_t bytes() const { return 2 * (npair_chunks * kPairElems + nkey_chunks * kKeyElems); }
};

}  // namespace gdn
