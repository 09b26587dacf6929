// mfma_tiles.hpp -- register-level building blocks of the gfx950 MFMA tree
// kernels: bf16 conversions, the 16x16x32 / 16x16x16 bf16 MFMA wrappers, the
// LDS tile layout shared by the Gram and the blocked substitution, and the
// cross-lane regrouping of accumulator-layout blocks into K = 32 operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kD = 128;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float bf16_val(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 4 fp32 -> bf16 (RNE), two values per conversion instruction.
__device__ __forceinline__ s16x4 to_bf16x4(f32x4 x) {
    return __builtin_bit_cast(s16x4, __builtin_convertvector(x, bf16x4));
}

// 4 fp32 accumulator values -> bf16 hi part and bf16 lo part (x - hi).
__device__ __forceinline__ void split4(f32x4 x, s16x4& hi, s16x4& lo) {
    const bf16x4 h = __builtin_convertvector(x, bf16x4);
    hi = __builtin_bit_cast(s16x4, h);
    lo = to_bf16x4(x - __builtin_convertvector(h, f32x4));
}

// 8 fp32 -> bf16x8 (RNE).
__device__ __forceinline__ bf16x8 to_bf16x8(float4 a, float4 b) {
    bf16x8 r;
    r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)a.z; r[3] = (__bf16)a.w;
    r[4] = (__bf16)b.x; r[5] = (__bf16)b.y; r[6] = (__bf16)b.z; r[7] = (__bf16)b.w;
    return r;
}

// 16x16 bf16 tiles in LDS are stored as half of a 16x16x32 A operand: element
// (row, col) at 16-byte slot row + 16 (col / 8), position col % 8.  Two tiles
// stored back to back then form one 16 x 32 operand [T_0 | T_1]: lane l reads
// 16 bytes at slot l and holds row l % 16, columns 8 (l / 16) .. +7.
__device__ __forceinline__ int a32_pos(int row, int col) {
    return (row + 16 * (col >> 3)) * 8 + (col & 7);
}

// Two 16x16 blocks X, Y held in accumulator layout (lane (n, q): rows
// 4q .. 4q+3 of column n, as bf16) -> the stacked 32 x 16 matrix [X; Y] as a
// 16x16x32 B operand (lane (n, q): rows 8q .. 8q+7 of column n).  Read as an A
// operand the same registers are [X^T | Y^T].  Two cross-lane swaps: the
// 32-lane swap gives [X rows 0-7 | Y rows 0-7] and [X rows 8-15 | Y rows 8-15]
// by lane halves, the 16-lane swap interleaves them into 8-row runs.
__device__ __forceinline__ bf16x8 stack_pair(s16x4 x, s16x4 y) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 xv = __builtin_bit_cast(u32x2, x), yv = __builtin_bit_cast(u32x2, y);
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const auto w = __builtin_amdgcn_permlane32_swap(xv[h], yv[h], false, false);
        const auto v = __builtin_amdgcn_permlane16_swap(w[0], w[1], false, false);
        r[h] = v[0];
        r[2 + h] = v[1];
    }
    return __builtin_bit_cast(bf16x8, r);
}

}  // namespace gdn
