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
// Q4_K sub-block b's 6-bit scale and min from a super-block's side data
// (scale bytes 0..3 in y, 4..7 in z, 8..11 in w): b < 4 takes the low 6 bits
// of bytes b and b + 4; b >= 4 the nibbles of byte b + 4 under the top two bits
// of bytes b - 4 (scale) and b (min).  Both forms are computed and one kept.
__device__ __forceinline__ void k4_scale_min(const v4i& sd, int b, int& sc, int& mn) {
    const int j = (b & 3) * 8;
    const uint32_t s0 = (uint32_t)sd.y >> j, s1 = (uint32_t)sd.z >> j, s2 = (uint32_t)sd.w >> j;
    const int lo_sc = (int)(s0 & 63u), lo_mn = (int)(s1 & 63u);
    const int hi_sc = (int)((s2 & 15u) | ((s0 >> 6) & 3u) << 4);
    const int hi_mn = (int)(((s2 >> 4) & 15u) | ((s1 >> 6) & 3u) << 4);
    sc = b < 4 ? lo_sc : hi_sc;
    mn = b < 4 ? lo_mn : hi_mn;
}

// Q3_K: the signed 6-bit scales of sub-blocks 2b and 2b + 1 (block b of a
// super-block) from the 12 scale bytes in s.x..s.z.  The low nibbles are bytes
// 2b, 2b + 1 (b < 4) or the high nibbles of bytes 2b - 8, 2b - 7; the top two
// bits of sub-block i are bits 2 * (i / 4) of byte 8 + i % 4; minus 32.
__device__ __forceinline__ void k3_scales(const v4i& s, int b, int& sc0, int& sc1) {
    const uint32_t wlo = (b & 2) ? (uint32_t)s.y : (uint32_t)s.x;
    const int sh = 16 * (b & 1) + (b < 4 ? 0 : 4);
    const uint32_t nib = (wlo >> sh) & 0x0F0Fu;
    const int i0 = 2 * b, i1 = i0 + 1;
    const uint32_t h0 = ((uint32_t)s.z >> (8 * (i0 & 3) + 2 * (i0 >> 2))) & 3u;
    const uint32_t h1 = ((uint32_t)s.z >> (8 * (i1 & 3) + 2 * (i1 >> 2))) & 3u;
    sc0 = (int)((nib & 0xFu) | h0 << 4) - 32;
    sc1 = (int)((nib >> 8) | h1 << 4) - 32;
}

// bits 0..3 of x moved to bit 4 of bytes 0..3 (bit i to byte i): the four
// copies x << 7i put bit i at bit 8i and nowhere else a byte starts
__device__ __forceinline__ int spread4(uint32_t x) {
    return (int)(((x * 0x00204081u) & 0x01010101u) << 4);
}

// Q5_1 block (16 nibble bytes w, fifth bits qh: element j at bit j) against
// Q8_1 codes: elements 0..15 in a_lo, 16..31 in a_hi; codes are 0..31
__device__ __forceinline__ int dot_q5(const v4i& w, uint32_t qh, const v4i& a_lo, const v4i& a_hi) {
    const int m = 0x0F0F0F0F;
    int s = dot4((w.x & m) | spread4(qh & 15u), a_lo.x, 0);
    s = dot4((w.y & m) | spread4((qh >> 4) & 15u), a_lo.y, s);
    s = dot4((w.z & m) | spread4((qh >> 8) & 15u), a_lo.z, s);
    s = dot4((w.w & m) | spread4((qh >> 12) & 15u), a_lo.w, s);
    s = dot4(((w.x >> 4) & m) | spread4((qh >> 16) & 15u), a_hi.x, s);
    s = dot4(((w.y >> 4) & m) | spread4((qh >> 20) & 15u), a_hi.y, s);
    s = dot4(((w.z >> 4) & m) | spread4((qh >> 24) & 15u), a_hi.z, s);
    return dot4(((w.w >> 4) & m) | spread4(qh >> 28), a_hi.w, s);
}

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

// NVFP4 (edge0-strata README, section "Changes from upstream Strata", NVFP4
// latent experts; the format read as FP4 E2M1 codes with an FP8 E4M3 scale per
// 16 elements and an fp32 scale per tensor).  Four codes, one per byte (0..15),
// become four int8 values 2 * e2m1(code): 0, 1, 2, 3, 4, 6, 8, 12 for the low
// three bits, negated when bit 3 is set.  v_perm looks the magnitude up in an
// 8-byte table (selector bytes 0..3 pick the low word, 4..7 the high word), a
// second lookup in the negated table gives the negative, and bit 3 selects.
__device__ __forceinline__ int e2m1x2_widen(uint32_t nib) {
    const uint32_t sel = nib & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sel);
    const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sel);
    const uint32_t m = ((nib >> 3) & 0x01010101u) * 0xFFu;
    return (int)((pos & ~m) | (neg & m));
}

// The two 16-element half sums of an NVFP4 chunk (byte j: element j in the low
// nibble, j + 16 in the high) against its Q8_1 codes: sum 2 * e2m1(c) * q_a.
__device__ __forceinline__ void dot_nv4(const v4i& w, const v4i& a_lo, const v4i& a_hi, int& s0, int& s1) {
    const uint32_t m = 0x0F0F0F0Fu;
    s0 = dot4(e2m1x2_widen((uint32_t)w.x & m), a_lo.x, 0);
    s0 = dot4(e2m1x2_widen((uint32_t)w.y & m), a_lo.y, s0);
    s0 = dot4(e2m1x2_widen((uint32_t)w.z & m), a_lo.z, s0);
    s0 = dot4(e2m1x2_widen((uint32_t)w.w & m), a_lo.w, s0);
    s1 = dot4(e2m1x2_widen(((uint32_t)w.x >> 4) & m), a_hi.x, 0);
    s1 = dot4(e2m1x2_widen(((uint32_t)w.y >> 4) & m), a_hi.y, s1);
    s1 = dot4(e2m1x2_widen(((uint32_t)w.z >> 4) & m), a_hi.z, s1);
    s1 = dot4(e2m1x2_widen(((uint32_t)w.w >> 4) & m), a_hi.w, s1);
}

// An FP8 E4M3 byte as float, exactly: bit 7 the sign, bits 6..3 the exponent
// (bias 7; 0 is subnormal, m * 2^-9), bits 2..0 the mantissa.  (0x7F / 0xFF,
// NaN in E4M3, decode as 480: non-finite input gives unspecified output.)
__device__ __forceinline__ float e4m3f(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -v : v;
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

// Sum over aligned groups of W lanes (W = 1..64), the result in every lane of
// the group: DPP quad permutes and row mirrors inside a 16-lane row, then the
// gfx950 row swaps (v_permlane16_swap / v_permlane32_swap) across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int W>
__device__ __forceinline__ float group_sum_fast(float v) {
    if constexpr (W >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
    if constexpr (W >= 16) v += dpp_mov<0x140>(v); // row_mirror
    if constexpr (W >= 32) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (W >= 64) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// fp64 value of another lane for one reduction step (STEP 0..5: xor 1, xor 2,
// mirror within 8, mirror within 16, the other row of a pair, the other half),
// through DPP and the gfx950 row swaps: no LDS round trip.
template <int STEP>
__device__ __forceinline__ double xlane_d(double v) {
    const long long b = __double_as_longlong(v);
    int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
    if constexpr (STEP < 4) {
        constexpr int CTRL = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
        lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xf, 0xf, false);
        hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xf, 0xf, false);
    } else if constexpr (STEP == 4) {
        auto a = __builtin_amdgcn_permlane16_swap((unsigned)lo, (unsigned)lo, false, false);
        auto c = __builtin_amdgcn_permlane16_swap((unsigned)hi, (unsigned)hi, false, false);
        const bool odd_row = (threadIdx.x & 16) != 0;
        lo = (int)(odd_row ? a[0] : a[1]);
        hi = (int)(odd_row ? c[0] : c[1]);
    } else {
        auto a = __builtin_amdgcn_permlane32_swap((unsigned)lo, (unsigned)lo, false, false);
        auto c = __builtin_amdgcn_permlane32_swap((unsigned)hi, (unsigned)hi, false, false);
        const bool upper = (threadIdx.x & 32) != 0;
        lo = (int)(upper ? a[0] : a[1]);
        hi = (int)(upper ? c[0] : c[1]);
    }
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Sum over the wave in a fixed order (every lane gets the same value: each
// step adds partner values that are equal across the partner pair).
__device__ __forceinline__ double wave_sum_d(double v) {
    v += xlane_d<0>(v);
    v += xlane_d<1>(v);
    v += xlane_d<2>(v);
    v += xlane_d<3>(v);
    v += xlane_d<4>(v);
    v += xlane_d<5>(v);
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

// A 16-byte load of data read once per call (expert and dense weight codes):
// marked non-temporal (streaming), which keeps it from displacing reused lines
// in the caches.  A single-launch read of 107 MB measured 6.1-6.4 TB/s with
// such loads against 5.5 TB/s with plain ones on MI355X.
__device__ __forceinline__ v4i ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

}  // namespace moe
