// Matrix-core operand helpers shared by the int8 GEMM kernels (gfx950).
//
// Lane layout of v_mfma_i32_32x32x32_i8 (and of the f16 / f32 32 x 32 forms
// used for scale products): lane l holds row (A operand) or column (B operand)
// l % 32, and K bytes 16 * (l / 32) .. + 16 of a 32-element block; the 32 x 32
// int32 result sits as column l % 32, rows mf_row_of(i, l / 32) for i < 16.
#pragma once
#include "kernels.h"

namespace moe {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int mf_row_of(int i, int half) { return (i >> 2) * 8 + half * 4 + (i & 3); }

// Q4_0 bytes (low nibble = element j, high nibble = element j + 16) widened to
// int8 (c - 8).  For a nibble c in each byte: c ^ 8 is c - 8 when c >= 8 and
// needs the sign bits 0xF0 when c < 8.
__device__ __forceinline__ uint32_t q4_widen(uint32_t nib) {
    const uint32_t v = nib ^ 0x08080808u;
    const uint32_t neg = (~nib) & 0x08080808u;
    return v | (neg * 0x1Eu);
}

// A binary16 scale as an f16 operand at k = 0 (the three other k slots zero).
__device__ __forceinline__ h4 scale_op(uint32_t d16) { return __builtin_bit_cast(h4, v2i{(int)d16, 0}); }

// the scale outer product: binary16 operands (exact in fp32), or fp32 operands
// (one k of v_mfma_f32_32x32x2_f32: lanes 0..31 carry the values, 32..63 zero)
__device__ __forceinline__ v16f scale_mfma(h4 a, h4 b) {
    return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, v16f{}, 0, 0, 0);
}
__device__ __forceinline__ v16f scale_mfma(float a, float b) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, v16f{}, 0, 0, 0);
}

}  // namespace moe
