// Device-side helpers shared by the gfx950 kernels: vector types, element
// conversions, MFMA wrappers, lane-group sums and the value-head -> key-head mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Key head read by value head h (tiled: h % Hk; grouped: h / (Hv / Hk)).
__device__ __forceinline__ int key_head(int h, int Hk, int Hv, int head_map) {
    return head_map == 0 ? h % Hk : h / (Hv / Hk);
}

// D(16x16, f32) += A(16x32) * B(32x16), fp16 operands.
// Lane l holds A[l % 16][kset(l / 16)], B[kset(l / 16)][l % 16] (8 k values each, in the
// same order for A and B) and D[4 * (l / 16) + r][l % 16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D(16x16, f32) += A(16x16) * B(16x16), fp16 operands; lane l holds 4 k values
// k = 4 * (l / 16) + e of row / column l % 16, and D as above.
__device__ __forceinline__ f32x4 mfma16x16x16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
    return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) {
    return f16x4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}

// A stored result in float16: its float32 value rounded to nearest even. The empty asm hides
// how x was computed, so the compiler cannot merge the conversion into the operation that
// produced x (an fma with a float16 result rounds once from the exact value, which can differ
// in the last place and would make results depend on how a kernel was instantiated).
__device__ __forceinline__ _Float16 f16_out(float x) {
    asm("" : "+v"(x));
    return (_Float16)x;
}

// ... and in bfloat16 (the same rounding, the same reason for the empty asm)
__device__ __forceinline__ __bf16 bf16_out(float x) {
    asm("" : "+v"(x));
    return (__bf16)x;
}

// x plus the value of the lane a DPP control names (all source lanes in range)
template <int kCtrl>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 2 .. 32), in every lane of the group, on the VALU:
// xor 1 and xor 2 (quad permutes), then the 8- and 16-lane mirrors (once the smaller groups
// hold one value each, the mirror partner holds the same value as the xor partner), then
// xor 16 by a swizzle. The additions are those of an xor butterfly from xor 1 upwards.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group width");
    x = add_dpp<0xB1>(x);                             // quad_perm [1, 0, 3, 2]
    if constexpr (N >= 4) x = add_dpp<0x4E>(x);       // quad_perm [2, 3, 0, 1]
    if constexpr (N >= 8) x = add_dpp<0x141>(x);      // row_half_mirror
    if constexpr (N >= 16) x = add_dpp<0x140>(x);     // row_mirror
    if constexpr (N >= 32)
        x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));  // xor 16
    return x;
}

// 4 consecutive state values at element index i of a float32 or 16-bit state (float16, or
// bfloat16 with bf), widened to float32 ...
__device__ __forceinline__ f32x4 load_state4(const void *base, int64_t i, bool f16, bool bf = false) {
    if (f16) {
        if (bf) {
            const u16x4 h = *reinterpret_cast<const u16x4 *>(static_cast<const uint16_t *>(base) + i);
            return f32x4{bf16_bits_to_f32(h[0]), bf16_bits_to_f32(h[1]), bf16_bits_to_f32(h[2]), bf16_bits_to_f32(h[3])};
        }
        const f16x4 h = *reinterpret_cast<const f16x4 *>(static_cast<const _Float16 *>(base) + i);
        return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    }
    return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + i);
}

// ... and stored, float16 (bfloat16 with bf) rounded to nearest even.
__device__ __forceinline__ void store_state4(void *base, int64_t i, f32x4 v, bool f16, bool bf = false) {
    if (f16 && bf) {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<b4 *>(static_cast<__bf16 *>(base) + i) = b4{bf16_out(v[0]), bf16_out(v[1]), bf16_out(v[2]), bf16_out(v[3])};
    } else if (f16) {
        *reinterpret_cast<f16x4 *>(static_cast<_Float16 *>(base) + i) =
            f16x4{f16_out(v[0]), f16_out(v[1]), f16_out(v[2]), f16_out(v[3])};
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + i) = v;
    }
}

}  // namespace gdn
