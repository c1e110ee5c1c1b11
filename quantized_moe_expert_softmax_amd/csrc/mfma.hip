// Grouped int8 matrix-core GEMM of libmoe: the many-token (prefill) path of
// the expert FFN and of the latent dense projections.
//
// Prior art: the Strata pages run prefill through a chunked grouped path and
// note that an integer matrix lane pays off once an expert sees about a hundred
// rows or more (Strata PR 24, SYCL port commits; "Q8 0 support", section "GPU
// expert kernels").  Here, for gfx950:
//   * one v_mfma_i32_32x32x32_i8 covers exactly one 32-element block along K,
//     so its int32 result is the exact block sum of 32 weight rows against 32
//     token columns; the block is then scaled by d_w * d_a in fp32 and added to
//     an fp32 accumulator (the block sums are never merged across blocks);
//   * the 32 x 32 scale products d_w[row] * d_a[token] of a block come from an
//     f16 matrix-core outer product (v_mfma_f32_32x32x16_f16 with one non-zero
//     k), exact in fp32 because two binary16 significands need 22 bits; so the
//     vector ALU spends one convert and one FMA per block result;
//   * weights are the row operand, tokens the column operand, so a lane holds
//     one token and 16 weight rows: the 32 outputs of one Q8_1 block of h sit in
//     one lane pair, which makes the SwiGLU + requantisation epilogue local;
//   * a workgroup computes 128 weight rows x 64 tokens, staging 4 blocks of K
//     at a time in LDS (double-buffered, rows padded by 16 bytes against bank
//     conflicts); Q4_0 codes are widened to int8 (c - 8) while staged, so the
//     inner loop is the same for both formats;
//   * the token tiles of all active experts are numbered by the bucketing
//     kernel (tile_map); block ids are spread so that one XCD works on
//     consecutive token tiles of the same weight rows, which then hit its L2.
#include <algorithm>

#include "kernels.h"

namespace moe {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int MF_MT = GEMM_TILE_M;        // token columns per workgroup
constexpr int MF_NT = 128;                // weight rows per workgroup
constexpr int MF_KB = 4;                  // blocks of 32 per LDS stage
constexpr int MF_ROWB = MF_KB * QK + 16;  // LDS bytes per staged row (padded)
constexpr int MF_THREADS = 256;
// binary16 scales of a stage: [block][MF_NT + 32] and [block][MF_MT + 32]; the
// last 32 entries of each row stay zero (the f16 outer product reads them in
// lanes 32..63)
constexpr int MF_SWR = MF_NT + 32, MF_SAR = MF_MT + 32;

struct MfArgs {
    const uint8_t* base;          // expert packs (group mode) or the dense matrix
    size_t group_stride;          // bytes per expert
    size_t codes_off, scales_off; // of the matrix inside an expert pack
    int rows, K, T;               // weight rows, elements per row, tokens
    int max_tiles;                // token tiles covered by the grid
    int act_div;                  // activation row = list entry / act_div
    Buckets b;                    // b.ctrl == nullptr: dense mode (tokens 0..T-1)
    const int32_t* tile_map;      // group mode: tile -> expert | (tile of expert << 16)
    ActPtr ain;                   // activation rows, Q8_1
    int F;                        // gate/up: intermediate width (SwiGLU epilogue)
    ActPtr hq;                    // gate/up output
    float* out;                   // store epilogue: [output row][rows]
    float* tap_h;                 // [A][F]
    int32_t* tap_isum;            // [output row][canonical row][K/32]
    int tap_tokens, tap_div;      // token of output row o = o / tap_div
};

__device__ __forceinline__ int mf_row_of(int i, int half) { return (i >> 2) * 8 + half * 4 + (i & 3); }

// Q4_0 bytes (low nibble = element j, high nibble = element j + 16) widened to
// int8 (c - 8).  For a nibble c in each byte: c ^ 8 is c - 8 when c >= 8 and
// needs the sign bits 0xF0 when c < 8.
__device__ __forceinline__ uint32_t q4_widen(uint32_t nib) {
    const uint32_t v = nib ^ 0x08080808u;
    const uint32_t neg = (~nib) & 0x08080808u;
    return v | (neg * 0x1Eu);
}

template <int FMT, bool SWIGLU, bool TAP>
__global__ __launch_bounds__(MF_THREADS, 2) void k_mfma(MfArgs A) {
    constexpr int QB = FMT == MOE_FMT_Q4_0 ? 16 : 32;   // code bytes per block
    constexpr int WBYTES = MF_NT * MF_ROWB, XBYTES = MF_MT * MF_ROWB;
    constexpr int STAGE = WBYTES + XBYTES + MF_KB * MF_SWR * 2 + MF_KB * MF_SAR * 2;
    __shared__ __align__(16) char smem[2 * STAGE];
    __shared__ int s_row[MF_MT], s_orow[MF_MT];

    // block id -> (row tile, token tile); consecutive ids of one XCD share row tiles
    const int nb_all = gridDim.x;
    const int lid = (blockIdx.x & 7) * (nb_all >> 3) + (blockIdx.x >> 3);
    const int NTI = A.rows / MF_NT;
    const int nt = lid / A.max_tiles, g = lid - nt * A.max_tiles;
    if (nt >= NTI) return;
    const uint8_t* mat;
    const int32_t* lst = nullptr;
    int cnt, m0;
    if (A.b.ctrl) {
        if (g >= (int)A.b.ctrl[CW_N_TILES]) return;
        const int tm = A.tile_map[g];
        const int e = tm & 0xffff;
        m0 = (tm >> 16) * MF_MT;
        cnt = A.b.counts[e];
        lst = A.b.lists + (size_t)e * A.T;
        mat = A.base + (size_t)e * A.group_stride;
    } else {
        m0 = g * MF_MT;
        if (m0 >= A.T) return;
        cnt = A.T;
        mat = A.base;
    }
    const int ncol = min(MF_MT, cnt - m0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    {
        // zero tails of the scale rows, both stage buffers
        const int buf = tid >> 7, kb = (tid >> 5) & 3, z = tid & 31;
        uint16_t* sdw = reinterpret_cast<uint16_t*>(smem + buf * STAGE + WBYTES + XBYTES);
        sdw[kb * MF_SWR + MF_NT + z] = 0;
        sdw[MF_KB * MF_SWR + kb * MF_SAR + MF_MT + z] = 0;
    }
    if (tid < MF_MT) {
        const int c = min(tid, ncol - 1);
        const int o = lst ? lst[m0 + c] : m0 + c;
        s_orow[tid] = o;
        s_row[tid] = o / A.act_div;
    }
    __syncthreads();

    const int K = A.K, nb = K / QK;
    const size_t rowb = (size_t)nb * QB;
    const uint8_t* codes = mat + A.codes_off + (size_t)nt * MF_NT * rowb;
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(mat + A.scales_off) + (size_t)nt * MF_NT * nb;

    // ---- global -> registers -> LDS staging of one stage (blocks kb0 .. kb0+MF_KB)
    constexpr int WCH = FMT == MOE_FMT_Q4_0 ? 2 : 4;   // 16-byte weight chunks per thread
    constexpr int WCPR = MF_KB * QB / 16;            // chunks per weight row per stage
    v4i rw[WCH];
    v4i rx[2];
    uint2 rdw;
    v4i rda;
    auto gload = [&](int kb0) {
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int r = ch / WCPR, p = ch - r * WCPR;
            rw[j] = ld16(codes + (size_t)r * rowb + (size_t)kb0 * QB + p * 16);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int c = ch >> 3, p = ch & 7;
            rx[j] = ld16(A.ain.q + (size_t)s_row[c] * K + (size_t)kb0 * QK + p * 16);
        }
        if (tid < MF_NT) {
            rdw = *reinterpret_cast<const uint2*>(scl + (size_t)tid * nb + kb0);
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
            rda = *reinterpret_cast<const v4i*>(A.ain.ds + (size_t)s_row[c] * nb + kb0);
        }
    };
    auto lstore = [&](int buf) {
        char* st = smem + buf * STAGE;
        int8_t* sw = reinterpret_cast<int8_t*>(st);
        int8_t* sx = reinterpret_cast<int8_t*>(st + WBYTES);
        uint16_t* sdw = reinterpret_cast<uint16_t*>(st + WBYTES + XBYTES);
        uint16_t* sda = sdw + MF_KB * MF_SWR;
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int r = ch / WCPR, p = ch - r * WCPR;
            if constexpr (FMT == MOE_FMT_Q4_0) {
                // one Q4_0 block (16 bytes) -> 32 int8: elements 0..15, then 16..31
                v4i lo, hi;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t w = (uint32_t)rw[j][d];
                    lo[d] = (int)q4_widen(w & 0x0F0F0F0Fu);
                    hi[d] = (int)q4_widen((w >> 4) & 0x0F0F0F0Fu);
                }
                *reinterpret_cast<v4i*>(sw + r * MF_ROWB + p * 32) = lo;
                *reinterpret_cast<v4i*>(sw + r * MF_ROWB + p * 32 + 16) = hi;
            } else {
                *reinterpret_cast<v4i*>(sw + r * MF_ROWB + p * 16) = rw[j];
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int c = ch >> 3, p = ch & 7;
            *reinterpret_cast<v4i*>(sx + c * MF_ROWB + p * 16) = rx[j];
        }
        if (tid < MF_NT) {
            sdw[0 * MF_SWR + tid] = (uint16_t)(rdw.x & 0xffffu);
            sdw[1 * MF_SWR + tid] = (uint16_t)(rdw.x >> 16);
            sdw[2 * MF_SWR + tid] = (uint16_t)(rdw.y & 0xffffu);
            sdw[3 * MF_SWR + tid] = (uint16_t)(rdw.y >> 16);
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
            const bool ok = c < ncol;      // columns past the tile's tokens get d_a = 0
#pragma unroll
            for (int q = 0; q < MF_KB; ++q)
                sda[q * MF_SAR + c] = ok ? (uint16_t)((uint32_t)rda[q] & 0xffffu) : (uint16_t)0;
        }
    };

    // ---- the wave's tile: rows wr*64 + [0,32) and + [32,64), token columns wc*32 + [0,32)
    const int wr = wave & 1, wc = wave >> 1;
    const int half = lane >> 5, l32 = lane & 31;
    // scale entries of this lane (the zero tails in lanes 32..63)
    const int o_w0 = half ? MF_NT + l32 : wr * 64 + l32;
    const int o_w1 = half ? MF_NT + l32 : wr * 64 + 32 + l32;
    const int o_a = half ? MF_MT + l32 : wc * 32 + l32;
    // a wave whose 32 token columns are all past the tile's tokens only stages
    const bool busy = wc * 32 < ncol;
    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.0f;

    const int stages = nb / MF_KB;
    auto compute = [&](int buf, int s) {
        if (!busy) return;
        const char* st = smem + buf * STAGE;
        const int8_t* sw = reinterpret_cast<const int8_t*>(st);
        const int8_t* sx = reinterpret_cast<const int8_t*>(st + WBYTES);
        const uint16_t* sdw = reinterpret_cast<const uint16_t*>(st + WBYTES + XBYTES);
        const uint16_t* sda = sdw + MF_KB * MF_SWR;
        // block kb's products are issued one block ahead of their rescale
        auto frag = [&](int kb, v4i& a0, v4i& a1, v4i& bx) {
            a0 = *reinterpret_cast<const v4i*>(sw + (wr * 64 + l32) * MF_ROWB + kb * QK + half * 16);
            a1 = *reinterpret_cast<const v4i*>(sw + (wr * 64 + 32 + l32) * MF_ROWB + kb * QK + half * 16);
            bx = *reinterpret_cast<const v4i*>(sx + (wc * 32 + l32) * MF_ROWB + kb * QK + half * 16);
        };
        // scale operands: lanes 0..31 give row / column l32 its binary16 d at k = 0
        auto sfrag = [&](int kb, h8& d0, h8& d1, h8& dc) {
            const v4i w0 = {(int)sdw[kb * MF_SWR + o_w0], 0, 0, 0};
            const v4i w1 = {(int)sdw[kb * MF_SWR + o_w1], 0, 0, 0};
            const v4i c0 = {(int)sda[kb * MF_SAR + o_a], 0, 0, 0};
            d0 = __builtin_bit_cast(h8, w0);
            d1 = __builtin_bit_cast(h8, w1);
            dc = __builtin_bit_cast(h8, c0);
        };
        v4i a0, a1, bx;
        h8 d0, d1, dc;
        frag(0, a0, a1, bx);
        sfrag(0, d0, d1, dc);
        v16i i0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bx, v16i{}, 0, 0, 0);
        v16i i1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bx, v16i{}, 0, 0, 0);
        v16f s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(d0, dc, v16f{}, 0, 0, 0);
        v16f s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(d1, dc, v16f{}, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < MF_KB; ++kb) {
            v16i n0, n1;
            v16f t0, t1;
            if (kb + 1 < MF_KB) {
                frag(kb + 1, a0, a1, bx);
                sfrag(kb + 1, d0, d1, dc);
                n0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bx, v16i{}, 0, 0, 0);
                n1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bx, v16i{}, 0, 0, 0);
                t0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(d0, dc, v16f{}, 0, 0, 0);
                t1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(d1, dc, v16f{}, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc0[i] = fmaf((float)i0[i], s0[i], acc0[i]);
                acc1[i] = fmaf((float)i1[i], s1[i], acc1[i]);
            }
            if constexpr (TAP) {
                const int c = wc * 32 + l32;
                const int o = s_orow[c];
                if (A.tap_isum && c < ncol && o / A.tap_div < A.tap_tokens) {
                    const int blk = s * MF_KB + kb;
                    for (int i = 0; i < 16; ++i) {
                        for (int t = 0; t < 2; ++t) {
                            const int pr = nt * MF_NT + wr * 64 + t * 32 + mf_row_of(i, half);
                            // canonical row: gate/up rows are stored as 32 gate + 32 up per slab
                            const int cr = SWIGLU ? ((pr & 63) < 32 ? (pr >> 6) * 32 + (pr & 31)
                                                                    : A.F + (pr >> 6) * 32 + (pr & 31))
                                                  : pr;
                            A.tap_isum[((size_t)o * A.rows + cr) * nb + blk] = t ? i1[i] : i0[i];
                        }
                    }
                }
            }
            if (kb + 1 < MF_KB) {
                i0 = n0;
                i1 = n1;
                s0 = t0;
                s1 = t1;
            }
            // the block's rescale happens here, not sunk past later stores
#pragma unroll
            for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(acc0[i]), "+v"(acc1[i]));
            // keep the two-deep pipeline: no hoisting of later blocks' reads
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    gload(0);
    lstore(0);
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s + 1 < stages; ++s) {
        gload((s + 1) * MF_KB);
        compute(s & 1, s);
        lstore((s + 1) & 1);
        __syncthreads();
    }
    compute((stages - 1) & 1, stages - 1);

    // ---- epilogue
    const int c = wc * 32 + l32;
    const bool valid = c < ncol;
    const int o = s_orow[c];
    if constexpr (SWIGLU) {
        // rows wr*64 + [0,32) are gate rows f, + [32,64) the up rows of the same f
        const int fb = nt * 2 + wr;     // Q8_1 block of h along F
        float h[16];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float gg = acc0[i], uu = acc1[i];
            h[i] = gg / (1.0f + expf(-gg)) * uu;
            amax = fmaxf(amax, fabsf(h[i]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const float d = amax / 127.0f;
        int qs[16];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            qs[i] = d != 0.0f ? (int)__builtin_roundf(h[i] / d) : 0;
            sum += qs[i];
        }
        sum += __shfl_xor(sum, 32, 64);
        float p = d * (float)sum;          // fp32 product, then binary16 (no fused rounding)
        asm volatile("" : "+v"(p));
        if (valid) {
            int8_t* qrow = A.hq.q + (size_t)o * A.F + fb * QK + half * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t pk = (uint32_t)(qs[4 * q] & 0xff) | ((uint32_t)(qs[4 * q + 1] & 0xff) << 8) |
                                    ((uint32_t)(qs[4 * q + 2] & 0xff) << 16) |
                                    ((uint32_t)(qs[4 * q + 3] & 0xff) << 24);
                *reinterpret_cast<uint32_t*>(qrow + q * 8) = pk;
            }
            if (half == 0) {
                const int FB = A.F / QK;
                A.hq.ds[(size_t)o * FB + fb] = f2h_bits(d) | (f2h_bits(p) << 16);
                A.hq.sq[(size_t)o * FB + fb] = sum;
            }
            if (TAP && A.tap_h) {
                float* hrow = A.tap_h + (size_t)o * A.F + fb * QK + half * 4;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4*>(hrow + q * 8) =
                        make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
            }
        }
    } else {
        if (valid) {
            float* orow = A.out + (size_t)o * A.rows + nt * MF_NT + wr * 64 + half * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<float4*>(orow + q * 8) =
                    make_float4(acc0[4 * q], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]);
                *reinterpret_cast<float4*>(orow + 32 + q * 8) =
                    make_float4(acc1[4 * q], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
bool mfma_config_ok(int rows, int K) { return rows % MF_NT == 0 && K % (MF_KB * QK) == 0; }


template <int FMT, bool SWIGLU>
static hipError_t mfma_launch(const MfArgs& a, bool tap, hipStream_t st, const KEvents& ev) {
    long blocks = (long)(a.rows / MF_NT) * a.max_tiles;
    blocks = (blocks + 7) & ~7L;
    if (blocks == 0) return hipSuccess;
    if (tap)
        launch_k(k_mfma<FMT, SWIGLU, true>, dim3((unsigned)blocks), dim3(MF_THREADS), 0, st, ev, a);
    else
        launch_k(k_mfma<FMT, SWIGLU, false>, dim3((unsigned)blocks), dim3(MF_THREADS), 0, st, ev, a);
    return hipGetLastError();
}

template <bool SWIGLU>
static hipError_t mfma_fmt(int fmt, const MfArgs& a, bool tap, hipStream_t st,
                           const KEvents& ev = KEvents{}) {
    if (!mfma_config_ok(a.rows, a.K)) return hipErrorInvalidConfiguration;
    if (fmt == MOE_FMT_Q4_0) return mfma_launch<MOE_FMT_Q4_0, SWIGLU>(a, tap, st, ev);
    return mfma_launch<MOE_FMT_Q8_0, SWIGLU>(a, tap, st, ev);
}

hipError_t launch_gate_up_mfma(const Dims& m, int T, const uint8_t* experts, ActPtr ain,
                               const Buckets& b, const int32_t* tile_map, ActPtr hq,
                               const Taps& taps, hipStream_t st, const KEvents& ev) {
    MfArgs a{};
    a.base = experts;
    a.group_stride = m.expert_bytes;
    a.codes_off = m.gu.codes_off;
    a.scales_off = m.gu.scales_off;
    a.rows = 2 * m.F; a.K = m.kin; a.T = T;
    a.max_tiles = gemm_max_tiles(T, m.k, m.E);
    a.act_div = m.k;
    a.b = b; a.tile_map = tile_map;
    a.ain = ain;
    a.F = m.F; a.hq = hq;
    a.tap_h = taps.h; a.tap_isum = taps.isum_gu; a.tap_tokens = taps.tap_tokens; a.tap_div = m.k;
    return mfma_fmt<true>(m.fmt, a, taps.h || taps.isum_gu, st, ev);
}

hipError_t launch_down_mfma(const Dims& m, int T, const uint8_t* experts, ActPtr hq,
                            const Buckets& b, const int32_t* tile_map, float* y, const Taps& taps,
                            hipStream_t st) {
    MfArgs a{};
    a.base = experts;
    a.group_stride = m.expert_bytes;
    a.codes_off = m.dn_off + m.dn.codes_off;
    a.scales_off = m.dn_off + m.dn.scales_off;
    a.rows = m.kout; a.K = m.F; a.T = T;
    a.max_tiles = gemm_max_tiles(T, m.k, m.E);
    a.act_div = 1;
    a.b = b; a.tile_map = tile_map;
    a.ain = hq;
    a.out = y;
    a.tap_isum = taps.isum_dn; a.tap_tokens = taps.tap_tokens; a.tap_div = m.k;
    return mfma_fmt<false>(m.fmt, a, taps.isum_dn != nullptr, st);
}

hipError_t launch_dense_mfma(const MatLayout& W, const uint8_t* base, int T, ActPtr ain, float* out,
                             int32_t* isum_tap, int tap_tokens, hipStream_t st) {
    MfArgs a{};
    a.base = base;
    a.codes_off = W.codes_off;
    a.scales_off = W.scales_off;
    a.rows = W.rows; a.K = W.nblk * QK; a.T = T;
    a.max_tiles = (T + MF_MT - 1) / MF_MT;
    a.act_div = 1;
    a.b = Buckets{};
    a.ain = ain;
    a.out = out;
    a.tap_isum = isum_tap; a.tap_tokens = tap_tokens; a.tap_div = 1;
    return mfma_fmt<false>(W.fmt, a, isum_tap != nullptr, st);
}

}  // namespace moe
