// Device helpers of libmoe: binary16 bits, packed int8 dots, wave reductions and
// the Q8_1 block quantiser used by every kernel that produces activations.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    // v_cvt_f32_f16: exact for every binary16 value, subnormals included
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}

__device__ __forceinline__ uint32_t f2h_bits(float v) {
    // v_cvt_f16_f32: round to nearest even, gradual underflow
    return (uint32_t)__half_as_ushort(__float2half_rn(v));
}

__device__ __forceinline__ int dot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// sum of 16 int8 products
__device__ __forceinline__ int dot16(const v4i& w, const v4i& a) {
    int s = dot4(w.x, a.x, 0);
    s = dot4(w.y, a.y, s);
    s = dot4(w.z, a.z, s);
    return dot4(w.w, a.w, s);
}

// Q4_0 block (16 code bytes: element j in the low nibble of byte j, element j+16
// in the high nibble) against 32 int8 activations a_lo (elements 0..15) and
// a_hi (16..31): sum_j c_j a_j, codes unsigned 0..15.  The caller subtracts
// 8 * sum(a) to centre the codes.
__device__ __forceinline__ int dot_q4(const v4i& w, const v4i& a_lo, const v4i& a_hi) {
    const int m = 0x0F0F0F0F;
    int s = dot4(w.x & m, a_lo.x, 0);
    s = dot4(w.y & m, a_lo.y, s);
    s = dot4(w.z & m, a_lo.z, s);
    s = dot4(w.w & m, a_lo.w, s);
    s = dot4((w.x >> 4) & m, a_hi.x, s);
    s = dot4((w.y >> 4) & m, a_hi.y, s);
    s = dot4((w.z >> 4) & m, a_hi.z, s);
    return dot4((w.w >> 4) & m, a_hi.w, s);
}

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ int group_sum_i(int v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Q8_1 of 32 values held one per lane by a 32-lane group (lanes 0..31 of a
// half-wave; `l` is the lane index within the group).  Writes the 32 codes,
// the (d, s) binary16 pair and the exact code sum.
//   d = max|v| / 127 (correctly rounded fp32 divide), q = round-half-away(v/d),
//   q = 0 when d == 0, s = d * sum(q) in fp32.
__device__ __forceinline__ void quant_q8_1_32(float v, int l, int8_t* q32, uint32_t* ds,
                                              int32_t* sq) {
    float amax = fabsf(v);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    float d = amax / 127.0f;
    int q = 0;
    if (d != 0.0f) q = (int)__builtin_roundf(v / d);
    int s = group_sum_i<32>(q);
    q32[l] = (int8_t)q;
    if (l == 0) {
        // s is the fp32 product, rounded to binary16 afterwards; the empty asm
        // keeps the backend from fusing the two roundings into one
        // multiply-to-half (v_fma_mixlo_f16).
        float p = d * (float)s;
        asm volatile("" : "+v"(p));
        *ds = f2h_bits(d) | (f2h_bits(p) << 16);
        *sq = s;
    }
}

__device__ __forceinline__ v4i ld16(const void* p) {
    return *reinterpret_cast<const v4i*>(p);
}

}  // namespace moe
