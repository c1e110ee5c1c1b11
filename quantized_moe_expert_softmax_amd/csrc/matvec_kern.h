// Matrix-vector kernels of libmoe: the decode path of the grouped expert FFN and
// the latent dense projections (device code, included by the per-format units).
//
// Prior art (Strata PR 24, SYCL port commits): the grouped expert kernels split
// each format into a once-per-weight part and a per-token part because a
// verify window routes one expert for up to 6 tokens; a handful of lanes per
// row beat a whole warp on short rows; 16-byte loads streamed faster than
// 4-byte ones.  Here, for gfx950:
//   * the workgroup stages the Q8_1 activations of its tokens in LDS once
//     (quantising fp32 rows on the way in when the producer left them fp32);
//   * a group of LPR lanes owns a weight row; lane sl loads the 16-byte chunks
//     c = j*LPR + sl (j < CPL), so each wave's loads are contiguous; one pass of
//     rows sits in registers while the next pass is already being loaded;
//   * each chunk is 16 int8 codes (half a Q8_0 block) or one Q4_0 / Q5_1 block
//     (Q5_1's fifth bits from the block's side data), dotted with v_dot4
//     against the LDS activations, scaled by d_w * d_a per block (plus Q5_1's
//     m_w * s_a);
//   * rows are reduced with DPP row ops and the gfx950 row swaps.
// Integer block sums are exact; scale products and row sums are fp32.
#pragma once
#include <algorithm>
#include <type_traits>

#include "matvec.h"
#include "select.h"

namespace moe {

struct __align__(16) K5SideMem {
    v4i s, qh0, qh1;
};
struct K5Side {
    v4i s, qh;
};

template <int FMT>
struct Fmt {
    static constexpr bool NIB = FMT != MOE_FMT_Q8_0;          // 16 nibble bytes per block
    static constexpr bool Q5 = FMT == MOE_FMT_Q5_1;
    static constexpr bool K5 = FMT == MOE_FMT_Q5_K;
    static constexpr bool K4 = FMT == MOE_FMT_Q4_K || K5;      // super-blocks of 256
    static constexpr bool K3 = FMT == MOE_FMT_Q3_K;            // super-blocks of 256
    static constexpr bool NV4 = FMT == MOE_FMT_NVFP4;          // two E4M3 scales per block
    static constexpr int QB = NIB ? 16 : 32;                  // code bytes per block of 32
    static constexpr int CPB = NIB ? 1 : 2;                   // chunks per block of 32
    static constexpr int SBLK = K4 || K3 ? 8 : 1;             // blocks of 32 per side-data unit
    static constexpr int CPSIDE = CPB * SBLK;                 // chunks per side-data unit
    // a unit's side data in memory and in registers: the binary16 d; for Q5_1
    // {d | m << 16, qh}; for a Q4_K super-block {d | dmin << 16, scale bytes
    // 0..11}; for Q5_K that and its 32 qh bytes (a chunk keeps its 16); for a
    // Q3_K super-block d in memory, {scale bytes 0..11, d} in registers
    using SideMem = std::conditional_t<
        K5, K5SideMem, std::conditional_t<K4, v4i, std::conditional_t<Q5, uint2, uint16_t>>>;
    using Side = std::conditional_t<
        K5, K5Side, std::conditional_t<K4 || K3, v4i, std::conditional_t<Q5, uint2, uint32_t>>>;
    // packed code bytes of a row of nb blocks (Q3_K: 108 per super-block)
    __host__ __device__ static constexpr size_t row_bytes(int nb) {
        return K3 ? (size_t)(nb / 8) * 108 : (size_t)nb * QB;
    }
};

// A Q3_K chunk: block c of the row, its 12 packed code bytes in w.x..w.z (two
// words of 2-bit codes, (word h >> 2m) & 0x03030303 being elements 16h + 4m ..
// + 3, and a word of high bits, element 4m + p at bit 8p + m) and the
// super-block's 12 scale bytes in s.x..s.z.  A code is low + 4 * high - 4:
// per byte, the low bits or'ed with 0xFC where the high bit is clear.  Returns
// the block's integer sum: each 16-element half's dot times its signed 6-bit
// sub-block scale (sub-blocks 2b, 2b + 1, b = c % 8).
__device__ __forceinline__ int k3_isum(const v4i& w, const v4i& s, int c, const int8_t* arow) {
    const v4i lo = *reinterpret_cast<const v4i*>(arow + c * 32);
    const v4i hi = *reinterpret_cast<const v4i*>(arow + c * 32 + 16);
    const uint32_t H = (uint32_t)w.z;
    int t0 = 0, t1 = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t n0 = ((H >> m) & 0x01010101u) ^ 0x01010101u;
        const uint32_t n1 = ((H >> (4 + m)) & 0x01010101u) ^ 0x01010101u;
        const int q0 = (int)((((uint32_t)w.x >> (2 * m)) & 0x03030303u) | (n0 * 0xFCu));
        const int q1 = (int)((((uint32_t)w.y >> (2 * m)) & 0x03030303u) | (n1 * 0xFCu));
        t0 = dot4(q0, lo[m], t0);
        t1 = dot4(q1, hi[m], t1);
    }
    int sc0, sc1;
    k3_scales(s, c & 7, sc0, sc1);
    return sc0 * t0 + sc1 * t1;
}

// A Q4_K chunk c (16 nibble bytes) of a row: super-block c / 8; within it
// nibble bytes 16 * (c % 8) .. + 16, i.e. elements 16 * (c % 2) .. + 16 of the
// sub-blocks 2g (low nibbles) and 2g + 1 (high nibbles), g = (c % 8) / 2.
// Its value against the LDS activations: the two scaled integer sums, and for
// the first half of each sub-block (c even) the min terms on the whole blocks'
// code sums.  isum0 / isum1 return the two integer sums (for taps).
// Q5_K (K5): qh holds the chunk's 16 qh bytes; bit b of qh byte i is the fifth
// bit of element i of sub-block b.
template <bool K5>
__device__ __forceinline__ float k4_chunk(const v4i& w, const v4i& sd, const v4i& qh, int c,
                                          bool valid, const int8_t* arow, const float* ad,
                                          const int32_t* asq, float acc, int& isum0, int& isum1) {
    const int sbk = c >> 3, cc = c & 7, g = cc >> 1, h = cc & 1;
    const int B0 = sbk * 8 + 2 * g, B1 = B0 + 1;
    const v4i a0 = *reinterpret_cast<const v4i*>(arow + B0 * 32 + 16 * h);
    const v4i a1 = *reinterpret_cast<const v4i*>(arow + B1 * 32 + 16 * h);
    const int m = 0x0F0F0F0F;
    v4i lo, hi;
    lo.x = w.x & m; lo.y = w.y & m; lo.z = w.z & m; lo.w = w.w & m;
    hi.x = (w.x >> 4) & m; hi.y = (w.y >> 4) & m; hi.z = (w.z >> 4) & m; hi.w = (w.w >> 4) & m;
    if constexpr (K5) {
        const int b0 = 2 * g, b1 = b0 + 1;
        lo.x |= (int)((((uint32_t)qh.x >> b0) & 0x01010101u) << 4);
        lo.y |= (int)((((uint32_t)qh.y >> b0) & 0x01010101u) << 4);
        lo.z |= (int)((((uint32_t)qh.z >> b0) & 0x01010101u) << 4);
        lo.w |= (int)((((uint32_t)qh.w >> b0) & 0x01010101u) << 4);
        hi.x |= (int)((((uint32_t)qh.x >> b1) & 0x01010101u) << 4);
        hi.y |= (int)((((uint32_t)qh.y >> b1) & 0x01010101u) << 4);
        hi.z |= (int)((((uint32_t)qh.z >> b1) & 0x01010101u) << 4);
        hi.w |= (int)((((uint32_t)qh.w >> b1) & 0x01010101u) << 4);
    }
    int i0 = dot4(lo.x, a0.x, 0);
    i0 = dot4(lo.y, a0.y, i0);
    i0 = dot4(lo.z, a0.z, i0);
    i0 = dot4(lo.w, a0.w, i0);
    int i1 = dot4(hi.x, a1.x, 0);
    i1 = dot4(hi.y, a1.y, i1);
    i1 = dot4(hi.z, a1.z, i1);
    i1 = dot4(hi.w, a1.w, i1);
    int sc0, mn0, sc1, mn1;
    k4_scale_min(sd, 2 * g, sc0, mn0);
    k4_scale_min(sd, 2 * g + 1, sc1, mn1);
    const float dd = h2f((uint32_t)sd.x), dmin = h2f((uint32_t)sd.x >> 16);
    const float da0 = ad[B0], da1 = ad[B1];
    acc = fmaf((float)i0, valid ? dd * (float)sc0 * da0 : 0.0f, acc);
    acc = fmaf((float)i1, valid ? dd * (float)sc1 * da1 : 0.0f, acc);
    const bool first = valid && h == 0;
    acc = fmaf((float)asq[B0], first ? -(dmin * (float)mn0 * da0) : 0.0f, acc);
    acc = fmaf((float)asq[B1], first ? -(dmin * (float)mn1 * da1) : 0.0f, acc);
    isum0 = i0;
    isum1 = i1;
    return acc;
}

// d of a block's side data
__device__ __forceinline__ uint32_t side_d(uint32_t s) { return s; }
__device__ __forceinline__ uint32_t side_d(uint2 s) { return s.x; }

// Q8_1 of one value per lane of a 32-lane group (see quant_q8_1_32), returned
// to every lane: code, (d, s) binary16 pair, code sum.
struct Q81 {
    int q;
    uint32_t ds;
    int sum;
};

__device__ __forceinline__ Q81 q8_1_lane(float v) {
    float amax = fabsf(v);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    float d = amax / 127.0f;
    int q = 0;
    if (d != 0.0f) q = (int)__builtin_roundf(v / d);
    int s = group_sum_i<32>(q);
    float p = d * (float)s;            // fp32 product, then binary16 (no fused rounding)
    asm volatile("" : "+v"(p));
    return Q81{q, f2h_bits(d) | (f2h_bits(p) << 16), s};
}

// ---------------------------------------------------------------------------
// LDS staging of the activation rows a workgroup works on.
//   s_q  int8  [n][K]
//   s_d  float [n][K/32]   the binary16 d of each block, as float
//   s_sq int   [n][K/32]   code sums (used by Q4_0 weights); with S_VAL the
//                          block's stored s as float bits instead (Q5_1 weights)
// src_row[i] is the row of the source buffer that becomes LDS row i.
template <bool S_VAL>
__device__ __forceinline__ void stage_q(const ActPtr& a, int K, const int32_t* src_row, int n,
                                        int8_t* s_q, float* s_d, int32_t* s_sq) {
    const int nb = K / QK, c16 = K / 16;
    for (int idx = threadIdx.x; idx < n * c16; idx += blockDim.x) {
        const int i = idx / c16, c = idx - i * c16;
        *reinterpret_cast<v4i*>(s_q + i * K + c * 16) = ld16(a.q + (size_t)src_row[i] * K + c * 16);
    }
    for (int idx = threadIdx.x; idx < n * nb; idx += blockDim.x) {
        const int i = idx / nb, b = idx - i * nb;
        const size_t g = (size_t)src_row[i] * nb + b;
        s_d[idx] = h2f(a.ds[g]);
        s_sq[idx] = S_VAL ? __float_as_int(h2f(a.ds[g] >> 16)) : a.sq[g];
    }
}

// fp32 rows quantised to Q8_1 straight into LDS; one 32-lane group per block.
// When `keep` has a q pointer the blocks are also written to it (row src_row[i]).
// (Loading several blocks' values before quantising the first measured no gain
// at one token and, inlined into every gate/up instance, took the 8-wave Q4_0
// kernel from 110 to 148 registers: half the occupancy at 32 tokens.)
template <bool S_VAL>
__device__ __forceinline__ void stage_f32(const float* src, int K, const int32_t* src_row, int n,
                                          int8_t* s_q, float* s_d, int32_t* s_sq, ActPtr keep) {
    const int nb = K / QK;
    const int ng = blockDim.x / 32, g = threadIdx.x / 32, l = threadIdx.x & 31;
    for (int blk = g; blk < n * nb; blk += ng) {
        const int i = blk / nb, b = blk - i * nb;
        const size_t row = src_row[i];
        const Q81 r = q8_1_lane(src[row * K + b * QK + l]);
        s_q[i * K + b * QK + l] = (int8_t)r.q;
        if (l == 0) {
            s_d[blk] = h2f(r.ds);
            s_sq[blk] = S_VAL ? __float_as_int(h2f(r.ds >> 16)) : r.sum;
        }
        if (keep.q) {
            keep.q[row * K + b * QK + l] = (int8_t)r.q;
            if (l == 0) {
                keep.ds[row * nb + b] = r.ds;
                keep.sq[row * nb + b] = r.sum;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The row-tile engine: for `rows` rows of a packed block matrix (codes at
// codes + r*rowb, side data at scl + r*nb/SBLK) and the n LDS activation rows,
// emit(i, r, W[r] . act[i]) from lane 0 of each row's lane group.
// Loads are unconditional (a chunk index past the row is clamped to the last
// chunk and its contribution masked later), and the scale stays as raw binary16
// bits until it is used, so no load waits on another.  STREAM loads the code
// bytes non-temporal, right for rows that a call reads once (every decode
// kernel here: one token, or an expert bucket that fits one chunk of staged
// tokens), as the caches then keep what is reused; the side data always loads
// plainly.  Measured on MI355X against plain loads: one-token layers 40.2 ->
// 37.9 us, six-token 158.2 -> 144.6 us; a row that its workgroup re-reads for a
// later chunk of tokens lost (the 32-token latent D in four-token chunks, 67 ->
// 75 us) and should load plainly.
// An empty asm that the compiler must assume rewrites a weight row's side data
// in place: a value computed from it cannot move above this point.
__device__ __forceinline__ void opaque_side(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque_side(uint2& v) {
    asm volatile("" : "+v"(v.x));
    asm volatile("" : "+v"(v.y));
}
__device__ __forceinline__ void opaque_side(v4i& v) {
    int x = v.x, y = v.y, z = v.z, w = v.w;
    asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
    v = v4i{x, y, z, w};
}
__device__ __forceinline__ void opaque_side(K5Side& v) {
    opaque_side(v.s);
    opaque_side(v.qh);
}

template <int FMT, int LPR, int CPL, bool STREAM>
__device__ __forceinline__ void load_row(const uint8_t* row, const typename Fmt<FMT>::SideMem* rscl,
                                         int sl, int NCH, v4i (&wq)[CPL],
                                         typename Fmt<FMT>::Side (&wsc)[CPL]) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = min(j * LPR + sl, NCH - 1);
        if constexpr (F::K3) {
            // the block's 12 code bytes and the super-block's scale bytes (4-byte
            // aligned), its d from the side data
            const uint8_t* u = row + (size_t)(c >> 3) * 108;
            const uint32_t* cw = reinterpret_cast<const uint32_t*>(u + (c & 7) * 12);
            const uint32_t* sw = reinterpret_cast<const uint32_t*>(u + 96);
            wq[j] = v4i{(int)cw[0], (int)cw[1], (int)cw[2], 0};
            wsc[j] = v4i{(int)sw[0], (int)sw[1], (int)sw[2], (int)rscl[c >> 3]};
            continue;
        }
        wq[j] = STREAM ? ld16_stream(row + (size_t)c * 16) : ld16(row + (size_t)c * 16);
        if constexpr (F::K5) {
            // the super-block's scales and the qh half of this chunk
            const v4i* u = reinterpret_cast<const v4i*>(rscl + c / F::CPSIDE);
            wsc[j].s = u[0];
            wsc[j].qh = u[1 + (c & 1)];
        } else {
            wsc[j] = rscl[c / F::CPSIDE];
        }
    }
}

template <int FMT>
__device__ __forceinline__ int chunk_isum_lds(const v4i& wq, const typename Fmt<FMT>::Side& side,
                                              const int8_t* arow, const int32_t* asq, int c) {
    if constexpr (FMT == MOE_FMT_Q4_K || FMT == MOE_FMT_Q5_K) {
        return 0;   // (K-quant chunks go through k4_chunk)
    } else if constexpr (FMT == MOE_FMT_Q5_1) {
        const v4i lo = *reinterpret_cast<const v4i*>(arow + c * 32);
        const v4i hi = *reinterpret_cast<const v4i*>(arow + c * 32 + 16);
        return dot_q5(wq, side.y, lo, hi);
    } else if constexpr (FMT == MOE_FMT_Q4_0) {
        const v4i lo = *reinterpret_cast<const v4i*>(arow + c * 32);
        const v4i hi = *reinterpret_cast<const v4i*>(arow + c * 32 + 16);
        return dot_q4(wq, lo, hi) - 8 * asq[c];
    } else {
        const v4i a = *reinterpret_cast<const v4i*>(arow + c * 16);
        return dot16(wq, a);
    }
}

// One pass: the rows of this pass (weights in wq/wsc) against the n staged rows.
template <int FMT, int LPR, int CPL, bool TAP, class Emit, class EmitIsum>
__device__ __forceinline__ void pass_dot(const v4i (&wq)[CPL], const typename Fmt<FMT>::Side (&wsc)[CPL], int r,
                                         int sl, int NCH, int nb, int n, int K,
                                         const int8_t* s_q, const float* s_d,
                                         const int32_t* s_sq, Emit& emit, EmitIsum& emit_isum,
                                         bool tap) {
    using F = Fmt<FMT>;
#pragma unroll 1
    for (int i = 0; i < n; ++i) {
        const int8_t* arow = s_q + i * K;
        const float* ad = s_d + i * nb;
        const int32_t* asq = s_sq + i * nb;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const bool valid = j * LPR + sl < NCH;
            const int c = min(j * LPR + sl, NCH - 1);
            if constexpr (F::K3) {
                const int is = k3_isum(wq[j], wsc[j], c, arow);
                acc = fmaf((float)is, valid ? h2f((uint32_t)wsc[j].w) * ad[c] : 0.0f, acc);
                if constexpr (TAP) {
                    if (tap && valid) emit_isum(i, r, c, is);
                }
            } else if constexpr (F::K4) {
                int i0, i1;
                if constexpr (F::K5)
                    acc = k4_chunk<true>(wq[j], wsc[j].s, wsc[j].qh, c, valid, arow, ad, asq, acc, i0, i1);
                else
                    acc = k4_chunk<false>(wq[j], wsc[j], wsc[j], c, valid, arow, ad, asq, acc, i0, i1);
                if constexpr (TAP) {
                    if (tap) {
                        // the two halves of each sub-block sit in lanes sl, sl ^ 1
                        const int f0 = i0 + __shfl_xor(i0, 1, 64), f1 = i1 + __shfl_xor(i1, 1, 64);
                        const int B0 = (c >> 3) * 8 + 2 * ((c & 7) >> 1);
                        if (valid && (sl & 1) == 0) {
                            emit_isum(i, r, B0, f0);
                            emit_isum(i, r, B0 + 1, f1);
                        }
                    }
                }
            } else if constexpr (F::NV4) {
                // the two halves' sums times their E4M3 scales, times d_a / 2
                const v4i lo = *reinterpret_cast<const v4i*>(arow + c * 32);
                const v4i hi = *reinterpret_cast<const v4i*>(arow + c * 32 + 16);
                int i0, i1;
                dot_nv4(wq[j], lo, hi, i0, i1);
                const float dh = valid ? 0.5f * ad[c] : 0.0f;
                acc = fmaf((float)i0, e4m3f(wsc[j] & 0xFFu) * dh, acc);
                acc = fmaf((float)i1, e4m3f((wsc[j] >> 8) & 0xFFu) * dh, acc);
                if constexpr (TAP) {
                    if (tap && valid) emit_isum(i, r, c, (int)(((uint32_t)i0 & 0xFFFFu) | ((uint32_t)i1 << 16)));
                }
            } else {
                const int blk = c / F::CPB;
                const int is = chunk_isum_lds<FMT>(wq[j], wsc[j], arow, asq, c);
                acc = fmaf((float)is, valid ? h2f(side_d(wsc[j])) * ad[blk] : 0.0f, acc);
                if constexpr (F::Q5) {
                    // min term: m_w times the activation block's stored s
                    acc = fmaf(valid ? h2f(wsc[j].x >> 16) : 0.0f, __int_as_float(asq[blk]), acc);
                }
                if constexpr (TAP) {
                    if (tap) {
                        int full = is;
                        if constexpr (F::CPB == 2) full += __shfl_xor(is, 1, 64);
                        if (valid && (F::CPB == 1 || (sl & 1) == 0)) emit_isum(i, r, blk, full);
                    }
                }
            }
        }
        const float v = group_sum_fast<LPR>(acc);
        if (sl == 0) emit(i, r, v);
    }
}

// All passes of a row tile.  Two register buffers alternate (A: even passes,
// B: odd passes) so the next pass is always in flight while one is dotted and
// no register copy forces a wait.  A load past the last pass re-reads the last
// pass's rows (it is never used) so that every load is unconditional.  On
// entry A must hold pass 0 when `a_loaded`.
template <int FMT, int LPR, int CPL, int NW, bool TAP, bool STREAM, int PASSES = 0, bool FENCE = true,
          class Emit, class EmitIsum>
__device__ __forceinline__ void row_tile(const uint8_t* codes, const typename Fmt<FMT>::SideMem* scl,
                                         size_t rowb,
                                         int nb, int rows, int n, int K, const int8_t* s_q,
                                         const float* s_d, const int32_t* s_sq, Emit emit,
                                         EmitIsum emit_isum, bool tap, v4i (&wA)[CPL],
                                         typename Fmt<FMT>::Side (&sA)[CPL], bool a_loaded) {
    using F = Fmt<FMT>;
    constexpr int RPW = 64 / LPR;
    const int NCH = nb * F::CPB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sl = lane % LPR, rg = lane / LPR;
    const int passes = PASSES ? PASSES : rows / (NW * RPW);
    // (opaque_side before each dot of buffer A keeps the scale conversions of
    // rows loaded before the staging from being hoisted above it, where the
    // staging would wait for them; placed after the next pass's loads are out.
    // Measured on several passes: the gate/up slabs gain (latent_q4 at 32
    // tokens 80.1 -> 76.5 us), the per-bucket rows lose (48.7 -> 58.3 us) and
    // take FENCE = false)
    if constexpr (PASSES == 1) {
        // a single pass: one buffer
        const int r = wave * RPW + rg;
        if (!a_loaded) load_row<FMT, LPR, CPL, STREAM>(codes + r * rowb, scl + (size_t)r * (nb / F::SBLK), sl, NCH, wA, sA);
#pragma unroll
        for (int j = 0; j < CPL; ++j) opaque_side(sA[j]);
        pass_dot<FMT, LPR, CPL, TAP>(wA, sA, r, sl, NCH, nb, n, K, s_q, s_d, s_sq, emit, emit_isum,
                                     tap);
        return;
    }
    auto row_of = [&](int p) { return (min(p, passes - 1) * NW + wave) * RPW + rg; };
    v4i wB[CPL];
    typename F::Side sB[CPL];
    if (!a_loaded) {
        const int r = row_of(0);
        load_row<FMT, LPR, CPL, STREAM>(codes + r * rowb, scl + (size_t)r * (nb / F::SBLK), sl, NCH, wA, sA);
    }
    for (int p = 0; p < passes; p += 2) {
        {
            const int r = row_of(p + 1);
            load_row<FMT, LPR, CPL, STREAM>(codes + r * rowb, scl + (size_t)r * (nb / F::SBLK), sl, NCH, wB, sB);
        }
        if constexpr (FENCE) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) opaque_side(sA[j]);
        }
        pass_dot<FMT, LPR, CPL, TAP>(wA, sA, row_of(p), sl, NCH, nb, n, K, s_q, s_d, s_sq, emit,
                                     emit_isum, tap);
        {
            const int r = row_of(p + 2);
            load_row<FMT, LPR, CPL, STREAM>(codes + r * rowb, scl + (size_t)r * (nb / F::SBLK), sl, NCH, wA, sA);
        }
        if (p + 1 < passes)
            pass_dot<FMT, LPR, CPL, TAP>(wB, sB, row_of(p + 1), sl, NCH, nb, n, K, s_q, s_d, s_sq,
                                         emit, emit_isum, tap);
    }
}



// One token's routing result, published by the workgroup that selected it (NT
// threads): ids and weights (threads j < k hold w_j) in rank order, and the
// buckets: every expert's count (0 or 1), the one assignment a = j at the head
// of its expert's list, the active experts in id order.
template <int NT>
__device__ __forceinline__ void publish_route(const RouteOut& R, int k, int E, const RouteLds& S,
                                              float w) {
    const int tid = threadIdx.x;
    if (tid < k) {
        const int id = S.sel[tid];
        int below = 0;
        for (int j = 0; j < k; ++j) below += (int)(S.sel[j] < id);
        R.ids[tid] = id;
        R.wts[tid] = w;
        R.lists[id] = tid;
        R.active[below] = id;
    }
    for (int e = tid; e < E; e += NT) {
        int c = 0;
        for (int j = 0; j < k; ++j) c |= (int)(S.sel[j] == e);
        R.counts[e] = c;
    }
    if (tid == 0) R.ctrl[CW_N_ACTIVE] = (uint32_t)k;
}

// (the second launch bound is the minimum number of waves per SIMD: 3 lets
// three 4-wave workgroups share a CU)
// (ALL: a slab of at most four passes has all of them in registers at once, see
// below; an instance of its own because the registers cost the occupancy that
// the windows of several tokens need)
template <int FMT, int LPR, int CPL, int NW>
constexpr bool gu_all_passes_ok() {
    constexpr int PASSES = 64 / (NW * (64 / LPR));
    constexpr int SIDE_DW = (int)(sizeof(typename Fmt<FMT>::Side) / 4);
    return PASSES > 1 && PASSES <= 4 && PASSES * CPL * (4 + SIDE_DW) <= (NW == 4 ? 100 : 128);
}

template <int FMT, int LPR, int CPL, int NW, bool TAP, bool ALL = false>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 3 : 2) void k_gate_up_mv(GUArgs A) {
    constexpr bool STREAM = true;   // an expert's tokens fit one chunk at decode sizes
    constexpr int PASSES = 64 / (NW * (64 / LPR));
    extern __shared__ __align__(16) char smem[];
    const int FB = A.F / QK;
    const int slot = blockIdx.x / FB, fb = blockIdx.x - slot * FB;
    const int K = A.K, nb = K / QK, TCH = A.tch;
    // With ALL (one token, a slab of a few passes: the short latent rows) every
    // pass of weights is requested at once and kept in registers, so the
    // workgroup waits for memory once instead of once per pass (latent_q8
    // one-token gate/up 15.9 -> 12.5 us; with several tokens the lost occupancy
    // made latent_q4 at 32 tokens 166 -> 225 us per layer, hence an instance of
    // its own).  In the 8-wave instances an fp32 input row (latent z) is then
    // requested first, before the routing ids and the weights: the loads
    // complete in order, so its quantisation waits for it alone (one token,
    // gate/up: latent_q4 11.1 -> 9.8 us, latent_q3_k 11.3 -> 10.3 us; the
    // 4-wave latent_q8 instance went from 13.6 to 15.7 us with it and does not).
    constexpr bool ALLP = ALL && gu_all_passes_ok<FMT, LPR, CPL, NW>();
    constexpr int ZPT = 4;      // fp32 input values per thread (K <= 2048)
    constexpr bool ZPRE = ALLP && NW == 8;
    float zv[ZPRE ? ZPT : 1];
    const bool zpre = ZPRE && A.ain_f32 && K <= ZPT * NW * 64;
    if constexpr (ZPRE) {
        if (zpre) {
#pragma unroll
            for (int i = 0; i < ZPT; ++i) {
                const int idx = threadIdx.x + i * NW * 64;
                zv[i] = idx < K ? A.ain_f32[idx] : 0.0f;     // token 0
            }
        }
    }
    int8_t* s_q = reinterpret_cast<int8_t*>(smem);
    float* s_d = reinterpret_cast<float*>(smem + (size_t)TCH * K);
    int32_t* s_sq = reinterpret_cast<int32_t*>(smem + (size_t)TCH * K + (size_t)TCH * nb * 4);
    float* s_gu = reinterpret_cast<float*>(smem + stage_bytes(TCH, K));
    int32_t* s_a = reinterpret_cast<int32_t*>(s_gu + TCH * 64);
    int32_t* s_t = s_a + TCH;
    int e, cnt;
    const int32_t* lst = nullptr;
    // one token whose activations are already quantised (the plain layer's
    // Q8_1(x)): its row is loaded before the routing, so that its loads overlap
    // the logits' instead of following the first weights
    const bool prestaged = A.route.part && !A.ain_f32 && K / 16 <= NW * 64;
    v4i xq = v4i{0, 0, 0, 0};
    uint32_t xds = 0u;
    int32_t xsq = 0;
    if (prestaged) {
        // (registers now, LDS once the selection is done: the loads are then
        // in flight together with the logits')
        if ((int)threadIdx.x < K / 16) xq = ld16(A.ain.q + threadIdx.x * 16);
        if ((int)threadIdx.x < nb) {
            xds = A.ain.ds[threadIdx.x];
            xsq = A.ain.sq[threadIdx.x];
        }
    }
    if (A.route.part) {
        // one token: the workgroup selects the experts (workgroup 0 also the
        // weights, and publishes the routing); slot j serves the rank-j expert,
        // whose one assignment is a = j
        const size_t route_off = (stage_bytes(TCH, K) + (size_t)TCH * (64 * 4 + 8) + 15) & ~(size_t)15;
        RouteLds& S = *reinterpret_cast<RouteLds*>(smem + route_off);
        SelectArgs sa = A.route;
        if (blockIdx.x != 0) sa.logits_tap = nullptr;
        float wt = 0.0f;
        select_wg<NW * 64>(sa, S, blockIdx.x == 0, &wt);
        if (blockIdx.x == 0) publish_route<NW * 64>(A.rout, A.k, A.route.E, S, wt);
        e = __builtin_amdgcn_readfirstlane(S.sel[slot]);
        cnt = 1;
        if (prestaged) {
            if (threadIdx.x == 0) {
                s_a[0] = slot;
                s_t[0] = 0;
            }
            if ((int)threadIdx.x < K / 16) *reinterpret_cast<v4i*>(s_q + threadIdx.x * 16) = xq;
            if ((int)threadIdx.x < nb) {
                asm volatile("" : "+v"(xds));   // (no conversion above the selection)
                s_d[threadIdx.x] = h2f(xds);
                s_sq[threadIdx.x] = Fmt<FMT>::Q5 ? __float_as_int(h2f(xds >> 16)) : xsq;
            }
        }
    } else if (A.ids_direct) {
        // one token routed by the launch before: slot j serves the rank-j
        // expert, whose one assignment is a = j
        e = __builtin_amdgcn_readfirstlane(A.b.ids[slot]);
        cnt = 1;
    } else if (A.ids_slots) {
        // a few tokens, no buckets: from the T * k routing ids, slot j serves the
        // j-th smallest distinct expert, whose assignments are listed in order
        // (the bucketing kernel's active / counts / lists, for this slot only):
        // counts per expert in LDS, then ballots and per-wave totals
        constexpr int NT = NW * 64;
        __shared__ int s_cnt[2 * NT], s_lst[DECODE_T * 32], s_wc[3][NW];
        __shared__ int s_e;
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, nA = A.T * A.k;
        const unsigned long long lt = (1ull << lane) - 1ull;
        const int id = tid < nA ? A.b.ids[tid] : -1;
        s_cnt[tid] = 0;
        s_cnt[tid + NT] = 0;
        if (tid == 0) s_e = -1;
        __syncthreads();
        if (id >= 0) atomicAdd(&s_cnt[id], 1);
        __syncthreads();
        // expert ids tid (pass 0) and tid + NT (pass 1); rank = active ids below
        unsigned long long bal[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            bal[m] = __ballot(s_cnt[tid + m * NT] > 0);
            if (lane == 0) s_wc[m][wave] = __popcll(bal[m]);
        }
        __syncthreads();
        int base = 0;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            for (int w = 0; w < NW; ++w) base += w < wave ? s_wc[m][w] : 0;
            if ((bal[m] >> lane) & 1ull) {
                if (base + __popcll(bal[m] & lt) == slot) s_e = tid + m * NT;
            }
            for (int w = wave; w < NW; ++w) base += s_wc[m][w];
        }
        __syncthreads();
        e = s_e;
        if (e < 0) return;              // (uniform) no expert for this slot
        const bool mine = id == e;
        const unsigned long long bm = __ballot(mine);
        if (lane == 0) s_wc[2][wave] = __popcll(bm);
        __syncthreads();
        if (mine) {
            int pos = __popcll(bm & lt);
            for (int w = 0; w < wave; ++w) pos += s_wc[2][w];
            s_lst[pos] = tid;
        }
        cnt = s_cnt[e];
        __syncthreads();
        lst = s_lst;
    } else {
        if (slot >= (int)A.b.ctrl[CW_N_ACTIVE]) return;
        e = A.b.active[slot];
        cnt = A.b.counts[e];
        lst = A.b.lists + (size_t)e * A.T;
    }
    const size_t rowb = Fmt<FMT>::row_bytes(nb);
    const uint8_t* ebase = expert_pack(A.experts, A.etab, e, A.eb);
    const uint8_t* codes = ebase + (size_t)fb * 64 * rowb;
    float tsg = 1.0f, tsu = 1.0f;
    if constexpr (Fmt<FMT>::NV4) {
        tsg = reinterpret_cast<const float*>(ebase + A.ts_off)[0];
        tsu = reinterpret_cast<const float*>(ebase + A.ts_off)[1];
    }
    using SM = typename Fmt<FMT>::SideMem;
    const SM* scl = reinterpret_cast<const SM*>(ebase + A.gu_scales_off) + (size_t)fb * 64 * (nb / Fmt<FMT>::SBLK);

    // the first pass of weights (with ALL: every pass) is requested before the
    // activations are staged (a one-token row of quantised activations: staged
    // in the prologue already)
    constexpr int RPW = 64 / LPR;
    constexpr int NBUF = ALLP ? PASSES : 1;
    const int sl = (threadIdx.x & 63) % LPR;
    auto row_of = [&](int p) { return (p * NW + (int)(threadIdx.x >> 6)) * RPW + (int)(threadIdx.x & 63) / LPR; };
    v4i wP[NBUF][CPL];
    typename Fmt<FMT>::Side sP[NBUF][CPL];
#pragma unroll
    for (int p = 0; p < NBUF; ++p) {
        const int r = row_of(p);
        load_row<FMT, LPR, CPL, STREAM>(codes + r * rowb, scl + (size_t)r * (nb / Fmt<FMT>::SBLK), sl,
                                        nb * Fmt<FMT>::CPB, wP[p], sP[p]);
    }
    for (int i0 = 0; i0 < cnt; i0 += TCH) {
        const int n = min(TCH, cnt - i0);
        if (prestaged) {
            __syncthreads();        // (the row staged after the selection)
        } else {
        if (threadIdx.x < n) {
            const int a = lst ? lst[i0 + threadIdx.x] : slot;
            s_a[threadIdx.x] = a;
            s_t[threadIdx.x] = a / A.k;
        }
        __syncthreads();
        if (ZPRE && zpre) {
            // the prefetched row: 32-lane groups hold whole blocks
            const ActPtr keep = fb == 0 ? A.keep : ActPtr{};
#pragma unroll
            for (int i = 0; i < ZPT; ++i) {
                const int idx = threadIdx.x + i * NW * 64, blk = idx / QK;
                if (idx < K) {
                    const Q81 r = q8_1_lane(zv[i]);
                    s_q[idx] = (int8_t)r.q;
                    if ((threadIdx.x & 31) == 0) {
                        s_d[blk] = h2f(r.ds);
                        s_sq[blk] = Fmt<FMT>::Q5 ? __float_as_int(h2f(r.ds >> 16)) : r.sum;
                    }
                    if (keep.q) {
                        keep.q[idx] = (int8_t)r.q;
                        if ((threadIdx.x & 31) == 0) {
                            keep.ds[blk] = r.ds;
                            keep.sq[blk] = r.sum;
                        }
                    }
                }
            }
        } else if (A.ain_f32)
            stage_f32<Fmt<FMT>::Q5>(A.ain_f32, K, s_t, n, s_q, s_d, s_sq, fb == 0 ? A.keep : ActPtr{});
        else
            stage_q<Fmt<FMT>::Q5>(A.ain, K, s_t, n, s_q, s_d, s_sq);
        __syncthreads();
        }
        const bool tap = TAP && A.taps.isum_gu;
        auto emit = [&](int i, int r, float v) {
            // NVFP4: the gate (rows 0..31 of the slab) or up tensor scale
            s_gu[i * 64 + r] = Fmt<FMT>::NV4 ? v * (r < 32 ? tsg : tsu) : v;
        };
        auto emit_isum = [&](int i, int r, int blk, int v) {
            if (s_t[i] < A.taps.tap_tokens) {
                const int row = r < 32 ? fb * 32 + r : A.F + fb * 32 + (r - 32);
                A.taps.isum_gu[((size_t)s_a[i] * 2 * A.F + row) * nb + blk] = v;
            }
        };
        if constexpr (ALLP) {
            // (the scale conversions would otherwise be hoisted above the
            // staging, which then waits for half of the weights first)
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
#pragma unroll
                for (int j = 0; j < CPL; ++j) opaque_side(sP[p][j]);
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
                pass_dot<FMT, LPR, CPL, TAP>(wP[p], sP[p], row_of(p), sl, nb * Fmt<FMT>::CPB, nb, n, K, s_q,
                                             s_d, s_sq, emit, emit_isum, tap);
        } else {
            row_tile<FMT, LPR, CPL, NW, TAP, STREAM, PASSES>(codes, scl, rowb, nb, 64, n, K, s_q, s_d, s_sq,
                                                             emit, emit_isum, tap, wP[0], sP[0], i0 == 0);
        }
        __syncthreads();
        // SwiGLU and Q8_1: one 32-lane group per token, lane = output f
        for (int ii = threadIdx.x / 32; ii < n; ii += NW * 2) {
            const int f = threadIdx.x & 31;
            const float g = s_gu[ii * 64 + f], u = s_gu[ii * 64 + 32 + f];
            const float h = g / (1.0f + expf(-g)) * u;
            const int a = s_a[ii];
            const Q81 r = q8_1_lane(h);
            A.hq.q[(size_t)a * A.F + fb * 32 + f] = (int8_t)r.q;
            if (f == 0) {
                A.hq.ds[(size_t)a * FB + fb] = r.ds;
                A.hq.sq[(size_t)a * FB + fb] = r.sum;
            }
            if constexpr (TAP) {
                if (A.taps.h) A.taps.h[(size_t)a * A.F + fb * 32 + f] = h;
            }
        }
        __syncthreads();
    }
}


// (SEL: the dense one-token form with the selection workgroup; an instance of
// its own, as the selection's registers cost the expert rows kernels occupancy.
// ONE: a tile of one pass, known when compiled (the dense one-token D and U),
// so that no second buffer re-requests the same rows; as a runtime case in
// the general instance it cost the per-bucket rows at 20 and 32 tokens 10-20%)
template <int FMT, int LPR, int CPL, int NW, bool TAP, bool SEL = false, bool ONE = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void k_rows_mv(RowsArgs A) {
    constexpr bool STREAM = true;   // one token (dense) or one bucket chunk (experts)
    extern __shared__ __align__(16) char smem[];
    int bid = blockIdx.x;
    if constexpr (SEL) {
        // dense mode, one token: workgroup 0 selects the token's experts (its
        // LDS holds only the selection), the others are the row tiles
        if (bid == 0) {
            RouteLds& S = *reinterpret_cast<RouteLds*>(smem);
            float wt = 0.0f;
            select_wg<NW * 64>(A.route, S, true, &wt);
            publish_route<NW * 64>(A.rout, A.k, A.route.E, S, wt);
            return;
        }
        --bid;
    }
    const int NRT = A.rows / A.rt;
    const int g = bid / NRT, rt = bid - g * NRT;
    const uint8_t* mat;
    const int32_t* lst = nullptr;
    int cnt;
    if (A.b.ctrl) {
        if (g >= (int)A.b.ctrl[CW_N_ACTIVE]) return;
        const int e = A.b.active[g];
        mat = expert_pack(A.base, A.etab, e, A.group_stride);
        cnt = A.b.counts[e];
        lst = A.b.lists + (size_t)e * A.T;
    } else {
        mat = A.base;
        cnt = A.T;
    }
    const int K = A.K, nb = K / QK, TCH = A.tch;
    const size_t rowb = Fmt<FMT>::row_bytes(nb);
    const uint8_t* codes = mat + A.codes_off + (size_t)rt * A.rt * rowb;
    // NVFP4 expert mode: the matrix's tensor scale
    const float tsr = Fmt<FMT>::NV4 && A.ts_off ? *reinterpret_cast<const float*>(mat + A.ts_off) : 1.0f;
    using SM = typename Fmt<FMT>::SideMem;
    const SM* scl = reinterpret_cast<const SM*>(mat + A.scales_off) + (size_t)rt * A.rt * (nb / Fmt<FMT>::SBLK);
    int8_t* s_q = reinterpret_cast<int8_t*>(smem);
    float* s_d = reinterpret_cast<float*>(smem + (size_t)TCH * K);
    int32_t* s_sq = reinterpret_cast<int32_t*>(smem + (size_t)TCH * K + (size_t)TCH * nb * 4);
    int32_t* s_s = reinterpret_cast<int32_t*>(smem + stage_bytes(TCH, K));

    // the first pass of weights is requested before the activations are staged
    v4i wA[CPL];
    typename Fmt<FMT>::Side sA[CPL];
    {
        constexpr int RPW = 64 / LPR;
        const int lane = threadIdx.x & 63;
        const int r = (threadIdx.x >> 6) * RPW + lane / LPR;
        load_row<FMT, LPR, CPL, STREAM>(codes + r * rowb, scl + (size_t)r * (nb / Fmt<FMT>::SBLK), lane % LPR,
                                nb * Fmt<FMT>::CPB, wA, sA);
    }
    for (int i0 = 0; i0 < cnt; i0 += TCH) {
        const int n = min(TCH, cnt - i0);
        if (threadIdx.x < n) s_s[threadIdx.x] = lst ? lst[i0 + threadIdx.x] : i0 + threadIdx.x;
        __syncthreads();
        if (A.ain_f32)
            stage_f32<Fmt<FMT>::Q5>(A.ain_f32, K, s_s, n, s_q, s_d, s_sq, rt == 0 ? A.keep : ActPtr{});
        else
            stage_q<Fmt<FMT>::Q5>(A.ain, K, s_s, n, s_q, s_d, s_sq);
        __syncthreads();
        const int r0 = rt * A.rt;
        auto emit = [&](int i, int r, float v) { A.out[(size_t)s_s[i] * A.rows + r0 + r] = v * tsr; };
        auto emit_isum = [&](int i, int r, int blk, int v) {
            if (s_s[i] / A.tap_div < A.tap_tokens)
                A.isum_tap[((size_t)s_s[i] * A.rows + r0 + r) * nb + blk] = v;
        };
        row_tile<FMT, LPR, CPL, NW, TAP, STREAM, ONE ? 1 : 0, false>(codes, scl, rowb, nb, A.rt, n, K, s_q, s_d,
                                                                     s_sq, emit, emit_isum, TAP && A.isum_tap, wA,
                                                                     sA, i0 == 0);
        __syncthreads();
    }
}


// The down kernels' epilogue: rows rt * RT .. + RT of token t combined in rank
// order from s_y.  With outq (a latent layer's y_lat, quantised once for the U
// projection): a 32-row tile is one Q8_1 block, quantised here; a 16-row tile is
// half of one, and the second of the block's two tiles to finish quantises it.
// That hand-off has no wait: each tile stores its rows with agent-scope stores
// (written through to the device-coherent level), waits for their completion,
// then counts itself in on the block's arrival counter (A.arrive, zero on
// entry); the tile that finds the other one there reads the 32 rows with
// agent-scope loads, writes the block and clears the counter for the next call.
template <bool TAP, int RT, int KMAX>
__device__ __forceinline__ void down_combine(const DownTokArgs& A, int t, int rt,
                                             const float (&s_y)[KMAX][RT]) {
    const int nbk = A.Kout / QK;
    const bool half = RT < QK && A.outq.q != nullptr;
    if (threadIdx.x < RT) {
        const int r = threadIdx.x;
        float o = 0.0f;
        for (int j = 0; j < A.k; ++j) {
            const int a = t * A.k + j;
            o = fmaf(A.b.wts[a], s_y[j][r], o);
            if constexpr (TAP) {
                if (A.taps.y) A.taps.y[(size_t)a * A.Kout + rt * RT + r] = s_y[j][r];
            }
        }
        float* dst = A.out + (size_t)t * A.Kout + rt * RT + r;
        if (half)
            __hip_atomic_store(dst, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            *dst = o;
        if constexpr (RT == QK) {
            // lanes 0..31 of wave 0: the tile's block
            const Q81 q = q8_1_lane(o);
            A.outq.q[(size_t)t * A.Kout + rt * RT + r] = (int8_t)q.q;
            if (r == 0) {
                A.outq.ds[(size_t)t * nbk + rt] = q.ds;
                A.outq.sq[(size_t)t * nbk + rt] = q.sum;
            }
        }
    }
    if constexpr (RT < QK) {
        if (!half) return;                  // (uniform)
        __shared__ int s_last;
        const int blk = rt * RT / QK;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(A.arrive + (size_t)t * nbk + blk, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(QK / RT - 1);
        __syncthreads();
        if (s_last && threadIdx.x < QK) {
            const size_t i = (size_t)t * A.Kout + (size_t)blk * QK + threadIdx.x;
            const float v = __hip_atomic_load(A.out + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const Q81 q = q8_1_lane(v);
            A.outq.q[i] = (int8_t)q.q;
            if (threadIdx.x == 0) {
                A.outq.ds[(size_t)t * nbk + blk] = q.ds;
                A.outq.sq[(size_t)t * nbk + blk] = q.sum;
                A.arrive[(size_t)t * nbk + blk] = 0u;
            }
        }
    }
}

// (TABLE: the packs are found through A.etab; a separate instance, so that the
// array form's rank loop carries no table load and no wait for it.  RT: output
// rows per workgroup; 32-row tiles also write Q8_1 of the combined rows)
template <int FMT, int LPR, int CPL, bool TAP, bool TABLE = false, int RT = DT_RT>
__global__ __launch_bounds__(DT_NW * 64, 2) void k_down_tok_mv(DownTokArgs A) {
    constexpr bool STREAM = true;
    using F = Fmt<FMT>;
    constexpr int RPW = 64 / LPR;
    constexpr int NA = F::CPB == 1 ? 2 : 1;     // 16-byte activation pieces per chunk
    __shared__ float s_y[DT_KMAX][RT];
    const int NRT = A.Kout / RT;
    const int t = blockIdx.x / NRT, rt = blockIdx.x - t * NRT;
    const int nb = A.F / QK;
    const int NCH = nb * F::CPB;
    const size_t rowb = F::row_bytes(nb);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sl = lane % LPR, rg = lane / LPR;
    const bool tap = TAP && t < A.taps.tap_tokens && A.taps.isum_dn;
    constexpr int PASSES = RT / RPW;
    for (int j = wave; j < A.k; j += DT_NW) {
        const int a = t * A.k + j;
        const int e = A.b.ids[a];
        const uint8_t* ebase = TABLE ? expert_pack(nullptr, A.etab, e, 0) : A.experts + (size_t)e * A.eb;
        const uint8_t* mat = ebase + A.dn_off;
        const uint8_t* codes = mat + (size_t)rt * RT * rowb;
        // NVFP4: the down matrix's tensor scale
        const float tsd = F::NV4 ? *reinterpret_cast<const float*>(ebase + A.ts_off) : 1.0f;
        using SM = typename F::SideMem;
        const SM* scl = reinterpret_cast<const SM*>(mat + A.dn_scales_off) + (size_t)rt * RT * (nb / F::SBLK);
        v4i wq[CPL], wn[CPL];
        typename F::Side wsc[CPL], wsn[CPL];
        load_row<FMT, LPR, CPL, STREAM>(codes + rg * rowb, scl + (size_t)rg * (nb / F::SBLK), sl, NCH, wq, wsc);
        // this rank's activation chunks, the same for every row
        v4i act[CPL][NA];
        int asq[CPL];
        const int8_t* arow = A.hq.q + (size_t)a * A.F;
        uint32_t ads[CPL];
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) {
            const int c = min(jj * LPR + sl, NCH - 1);
#pragma unroll
            for (int h = 0; h < NA; ++h) act[jj][h] = ld16(arow + c * 16 * NA + h * 16);
            asq[jj] = F::CPB == 1 && !F::Q5 ? A.hq.sq[(size_t)a * nb + c] : 0;
            ads[jj] = A.hq.ds[(size_t)a * nb + c / F::CPB];
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = p * RPW + rg;
            if (p + 1 < PASSES)
                load_row<FMT, LPR, CPL, STREAM>(codes + (r + RPW) * rowb, scl + (size_t)(r + RPW) * (nb / F::SBLK), sl,
                                        NCH, wn, wsn);
            float acc = 0.0f;
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                const int c = jj * LPR + sl;
                const bool valid = c < NCH;
                int is;
                if constexpr (F::NV4) {
                    // two halves, each with its E4M3 scale, times d_a / 2; the
                    // tap holds both sums (half 0 in the low 16 bits)
                    int i0, i1;
                    dot_nv4(wq[jj], act[jj][0], act[jj][NA - 1], i0, i1);
                    const float dh = valid ? 0.5f * h2f(ads[jj]) : 0.0f;
                    acc = fmaf((float)i0, e4m3f(wsc[jj] & 0xFFu) * dh, acc);
                    acc = fmaf((float)i1, e4m3f((wsc[jj] >> 8) & 0xFFu) * dh, acc);
                    is = (int)(((uint32_t)i0 & 0xFFFFu) | ((uint32_t)i1 << 16));
                } else {
                    if constexpr (F::Q5)
                        is = dot_q5(wq[jj], wsc[jj].y, act[jj][0], act[jj][NA - 1]);
                    else if constexpr (F::CPB == 1)
                        is = dot_q4(wq[jj], act[jj][0], act[jj][NA - 1]) - 8 * asq[jj];
                    else
                        is = dot16(wq[jj], act[jj][0]);
                    acc = fmaf((float)is, valid ? h2f(side_d(wsc[jj])) * h2f(ads[jj]) : 0.0f, acc);
                }
                if constexpr (F::Q5) {
                    // min term: m_w times the block's stored s
                    acc = fmaf(valid ? h2f(wsc[jj].x >> 16) : 0.0f, h2f(ads[jj] >> 16), acc);
                }
                if constexpr (TAP) {
                    if (tap) {
                        int full = is;
                        if constexpr (F::CPB == 2) full += __shfl_xor(is, 1, 64);
                        if (valid && (F::CPB == 1 || (sl & 1) == 0))
                            A.taps.isum_dn[((size_t)a * A.Kout + rt * RT + r) * nb + c / F::CPB] = full;
                    }
                }
            }
            const float y = group_sum_fast<LPR>(acc);
            if (sl == 0) s_y[j][r] = F::NV4 ? y * tsd : y;
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                wq[jj] = wn[jj];
                wsc[jj] = wsn[jj];
            }
        }
    }
    __syncthreads();
    down_combine<TAP, RT>(A, t, rt, s_y);
}

// The same for K-quant experts (Q4_K, Q5_K, Q3_K), whose chunk dots read the
// activations from LDS: the token's k rows of Q8_1(h) are staged once for every
// wave (after each wave has requested its first pass of weights), then wave j
// runs rank j's rows through the row-tile dot and the tile is combined in rank
// order as above.  Dynamic LDS: k * (F + 8 * F/32) bytes.
template <int FMT, int LPR, int CPL, bool TAP, int RT = DT_RT>
__global__ __launch_bounds__(DT_NW * 64, 2) void k_down_tok_kq(DownTokArgs A) {
    constexpr bool STREAM = true;
    using F = Fmt<FMT>;
    using SM = typename F::SideMem;
    constexpr int RPW = 64 / LPR;
    constexpr int PASSES = RT / RPW;
    extern __shared__ __align__(16) char smem[];
    __shared__ float s_y[DT_KMAX][RT];
    __shared__ int32_t s_src[DT_KMAX];
    const int NRT = A.Kout / RT;
    const int t = blockIdx.x / NRT, rt = blockIdx.x - t * NRT;
    const int K = A.F, nb = K / QK, NCH = nb * F::CPB;
    const size_t rowb = F::row_bytes(nb);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sl = lane % LPR, rg = lane / LPR;
    const bool tap = TAP && t < A.taps.tap_tokens && A.taps.isum_dn;
    int8_t* s_q = reinterpret_cast<int8_t*>(smem);
    float* s_d = reinterpret_cast<float*>(smem + (size_t)A.k * K);
    int32_t* s_sq = reinterpret_cast<int32_t*>(smem + (size_t)A.k * K + (size_t)A.k * nb * 4);

    const uint8_t* codes = nullptr;
    const SM* scl = nullptr;
    auto locate = [&](int j) {
        const int e = A.b.ids[t * A.k + j];
        const uint8_t* mat = expert_pack(A.experts, A.etab, e, A.eb) + A.dn_off;
        codes = mat + (size_t)rt * RT * rowb;
        scl = reinterpret_cast<const SM*>(mat + A.dn_scales_off) + (size_t)rt * RT * (nb / F::SBLK);
    };
    v4i wq[CPL], wn[CPL];
    typename F::Side wsc[CPL], wsn[CPL];
    if (wave < A.k) {
        locate(wave);
        load_row<FMT, LPR, CPL, STREAM>(codes + rg * rowb, scl + (size_t)rg * (nb / F::SBLK), sl, NCH, wq, wsc);
    }
    if ((int)threadIdx.x < A.k) s_src[threadIdx.x] = t * A.k + threadIdx.x;
    __syncthreads();
    stage_q<F::Q5>(A.hq, K, s_src, A.k, s_q, s_d, s_sq);
    __syncthreads();
    for (int j = wave; j < A.k; j += DT_NW) {
        const int a = t * A.k + j;
        if (j != wave) {
            locate(j);
            load_row<FMT, LPR, CPL, STREAM>(codes + rg * rowb, scl + (size_t)rg * (nb / F::SBLK), sl, NCH, wq, wsc);
        }
        auto emit = [&](int, int r, float v) { s_y[j][r] = v; };
        auto emit_isum = [&](int, int r, int blk, int v) {
            A.taps.isum_dn[((size_t)a * A.Kout + rt * RT + r) * nb + blk] = v;
        };
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = p * RPW + rg;
            if (p + 1 < PASSES)
                load_row<FMT, LPR, CPL, STREAM>(codes + (r + RPW) * rowb, scl + (size_t)(r + RPW) * (nb / F::SBLK), sl,
                                        NCH, wn, wsn);
            pass_dot<FMT, LPR, CPL, TAP>(wq, wsc, r, sl, NCH, nb, 1, K, s_q + (size_t)j * K, s_d + j * nb,
                                         s_sq + j * nb, emit, emit_isum, tap);
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                wq[jj] = wn[jj];
                wsc[jj] = wsn[jj];
            }
        }
    }
    __syncthreads();
    down_combine<TAP, RT>(A, t, rt, s_y);
}

// ---------------------------------------------------------------------------
// configuration choice and dispatch

// lanes per row and 16-byte chunks per lane for a row of nch chunks

#define MOE_LPR_CPL_SWITCH(LPR_, CPL_, CALL)                                      \
    switch (LPR_ * 16 + CPL_) {                                                    \
        case 8 * 16 + 1: { constexpr int L = 8, C = 1; CALL; break; }             \
        case 8 * 16 + 2: { constexpr int L = 8, C = 2; CALL; break; }             \
        case 8 * 16 + 3: { constexpr int L = 8, C = 3; CALL; break; }             \
        case 8 * 16 + 4: { constexpr int L = 8, C = 4; CALL; break; }             \
        case 8 * 16 + 5: { constexpr int L = 8, C = 5; CALL; break; }             \
        case 8 * 16 + 6: { constexpr int L = 8, C = 6; CALL; break; }             \
        case 8 * 16 + 7: { constexpr int L = 8, C = 7; CALL; break; }             \
        case 8 * 16 + 8: { constexpr int L = 8, C = 8; CALL; break; }             \
        case 16 * 16 + 1: { constexpr int L = 16, C = 1; CALL; break; }           \
        case 16 * 16 + 2: { constexpr int L = 16, C = 2; CALL; break; }           \
        case 16 * 16 + 3: { constexpr int L = 16, C = 3; CALL; break; }           \
        case 16 * 16 + 4: { constexpr int L = 16, C = 4; CALL; break; }           \
        case 16 * 16 + 5: { constexpr int L = 16, C = 5; CALL; break; }           \
        case 16 * 16 + 6: { constexpr int L = 16, C = 6; CALL; break; }           \
        case 16 * 16 + 7: { constexpr int L = 16, C = 7; CALL; break; }           \
        case 16 * 16 + 8: { constexpr int L = 16, C = 8; CALL; break; }           \
        case 32 * 16 + 1: { constexpr int L = 32, C = 1; CALL; break; }           \
        case 32 * 16 + 2: { constexpr int L = 32, C = 2; CALL; break; }           \
        case 32 * 16 + 3: { constexpr int L = 32, C = 3; CALL; break; }           \
        case 32 * 16 + 4: { constexpr int L = 32, C = 4; CALL; break; }           \
        case 32 * 16 + 5: { constexpr int L = 32, C = 5; CALL; break; }           \
        case 32 * 16 + 6: { constexpr int L = 32, C = 6; CALL; break; }           \
        case 32 * 16 + 7: { constexpr int L = 32, C = 7; CALL; break; }           \
        case 32 * 16 + 8: { constexpr int L = 32, C = 8; CALL; break; }           \
        case 64 * 16 + 1: { constexpr int L = 64, C = 1; CALL; break; }           \
        case 64 * 16 + 2: { constexpr int L = 64, C = 2; CALL; break; }           \
        case 64 * 16 + 3: { constexpr int L = 64, C = 3; CALL; break; }           \
        case 64 * 16 + 4: { constexpr int L = 64, C = 4; CALL; break; }           \
        case 64 * 16 + 5: { constexpr int L = 64, C = 5; CALL; break; }           \
        case 64 * 16 + 6: { constexpr int L = 64, C = 6; CALL; break; }           \
        case 64 * 16 + 7: { constexpr int L = 64, C = 7; CALL; break; }           \
        case 64 * 16 + 8: { constexpr int L = 64, C = 8; CALL; break; }           \
        default: return hipErrorInvalidConfiguration;                              \
    }

template <int FMT, bool TAP>
hipError_t gate_up_fmt(int lpr, int cpl, dim3 grid, size_t lds, const GUArgs& a,
                              hipStream_t st, const KEvents& ev) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        constexpr int NW = gu_waves_c(L, FMT);
        // (one token: 8 waves, whose registers hold every pass at once)
        if constexpr (64 % (8 * (64 / L)) == 0 && gu_all_passes_ok<FMT, L, C, 8>()) {
            if (a.T == 1) {
                launch_k(k_gate_up_mv<FMT, L, C, 8, TAP, true>, grid, dim3(8 * 64), lds, st, ev, a);
                break;
            }
        }
        launch_k(k_gate_up_mv<FMT, L, C, NW, TAP>, grid, dim3(NW * 64), lds, st, ev, a);
    }));
    return hipGetLastError();
}

template <int FMT, bool TAP>
hipError_t rows_fmt(int lpr, int cpl, dim3 grid, size_t lds, const RowsArgs& a,
                           hipStream_t st) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        // one pass of rows per tile in the dense one-token form
        const bool one = !a.b.ctrl && a.T == 1 && a.rt == ROWS_NW * (64 / L);
        if (a.route.part) {
            if constexpr (FMT == MOE_FMT_Q8_0 || FMT == MOE_FMT_Q4_0) {
                if (one)
                    hipLaunchKernelGGL((k_rows_mv<FMT, L, C, ROWS_NW, TAP, true, true>), grid, dim3(ROWS_NW * 64),
                                       lds, st, a);
                else
                    hipLaunchKernelGGL((k_rows_mv<FMT, L, C, ROWS_NW, TAP, true>), grid, dim3(ROWS_NW * 64), lds,
                                       st, a);
            } else {
                return hipErrorInvalidValue;      // (the dense formats only)
            }
        } else if (one) {
            if constexpr (FMT == MOE_FMT_Q8_0 || FMT == MOE_FMT_Q4_0)
                hipLaunchKernelGGL((k_rows_mv<FMT, L, C, ROWS_NW, TAP, false, true>), grid, dim3(ROWS_NW * 64),
                                   lds, st, a);
            else
                hipLaunchKernelGGL((k_rows_mv<FMT, L, C, ROWS_NW, TAP>), grid, dim3(ROWS_NW * 64), lds, st, a);
        } else {
            hipLaunchKernelGGL((k_rows_mv<FMT, L, C, ROWS_NW, TAP>), grid, dim3(ROWS_NW * 64), lds, st, a);
        }
    }));
    return hipGetLastError();
}

template <int FMT, bool TAP>
hipError_t down_tok_fmt(int lpr, int cpl, int T, const DownTokArgs& a, hipStream_t st) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        if constexpr (DT_RT % (64 / L) == 0) {
            dim3 grid(T * (a.Kout / DT_RT));
            if (a.outq.q && !a.arrive)
                hipLaunchKernelGGL((k_down_tok_mv<FMT, L, C, TAP, false, QK>), dim3(T * (a.Kout / QK)),
                                   dim3(DT_NW * 64), 0, st, a);
            else if (a.outq.q && DT_RT_ONE % (64 / L) == 0)
                hipLaunchKernelGGL((k_down_tok_mv<FMT, L, C, TAP, false, DT_RT_ONE % (64 / L) == 0 ? DT_RT_ONE : DT_RT>),
                                   dim3(T * (a.Kout / DT_RT_ONE)), dim3(DT_NW * 64), 0, st, a);
            else if (a.etab)
                hipLaunchKernelGGL((k_down_tok_mv<FMT, L, C, false, true>), grid, dim3(DT_NW * 64), 0, st, a);
            else
                hipLaunchKernelGGL((k_down_tok_mv<FMT, L, C, TAP>), grid, dim3(DT_NW * 64), 0, st, a);
        } else {
            return hipErrorInvalidConfiguration;
        }
    }));
    return hipGetLastError();
}

template <int FMT, bool TAP>
hipError_t down_tok_kq_fmt(int lpr, int cpl, int T, size_t lds, const DownTokArgs& a, hipStream_t st) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        if constexpr (DT_RT % (64 / L) == 0) {
            dim3 grid(T * (a.Kout / DT_RT));
            if (a.outq.q && !a.arrive)
                hipLaunchKernelGGL((k_down_tok_kq<FMT, L, C, TAP, QK>), dim3(T * (a.Kout / QK)),
                                   dim3(DT_NW * 64), lds, st, a);
            else if (a.outq.q && DT_RT_ONE % (64 / L) == 0)
                hipLaunchKernelGGL((k_down_tok_kq<FMT, L, C, TAP, DT_RT_ONE % (64 / L) == 0 ? DT_RT_ONE : DT_RT>),
                                   dim3(T * (a.Kout / DT_RT_ONE)), dim3(DT_NW * 64), lds, st, a);
            else
                hipLaunchKernelGGL((k_down_tok_kq<FMT, L, C, TAP>), grid, dim3(DT_NW * 64), lds, st, a);
        } else {
            return hipErrorInvalidConfiguration;
        }
    }));
    return hipGetLastError();
}

// Explicit instances of one format's launch functions.
#define MOE_MV_INSTANCES(F)                                                                     \
    template hipError_t gate_up_fmt<F, false>(int, int, dim3, size_t, const GUArgs&, hipStream_t, \
                                              const KEvents&);                                  \
    template hipError_t gate_up_fmt<F, true>(int, int, dim3, size_t, const GUArgs&, hipStream_t,  \
                                             const KEvents&);                                   \
    template hipError_t rows_fmt<F, false>(int, int, dim3, size_t, const RowsArgs&, hipStream_t); \
    template hipError_t rows_fmt<F, true>(int, int, dim3, size_t, const RowsArgs&, hipStream_t);
#define MOE_MV_DOWN_TOK_INSTANCES(F)                                                           \
    template hipError_t down_tok_fmt<F, false>(int, int, int, const DownTokArgs&, hipStream_t); \
    template hipError_t down_tok_fmt<F, true>(int, int, int, const DownTokArgs&, hipStream_t);
#define MOE_MV_DOWN_TOK_KQ_INSTANCES(F)                                                              \
    template hipError_t down_tok_kq_fmt<F, false>(int, int, int, size_t, const DownTokArgs&, hipStream_t); \
    template hipError_t down_tok_kq_fmt<F, true>(int, int, int, size_t, const DownTokArgs&, hipStream_t);

}  // namespace moe
