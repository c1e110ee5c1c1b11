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
//     f16 matrix-core outer product (v_mfma_f32_32x32x8f16 with one non-zero
//     k), exact in fp32 because two binary16 significands need 22 bits; so the
//     vector ALU spends one convert and one FMA per block result;
//   * weights are the row operand, tokens the column operand, so a lane holds
//     one token and 16 weight rows: the 32 outputs of one Q8_1 block of h sit in
//     one lane pair, which makes the SwiGLU + requantisation epilogue local;
//   * a workgroup computes 128 weight rows x 64 tokens, 4 blocks of K per LDS
//     stage.  Q8_0 weights stream into a three-stage LDS ring with direct
//     global->LDS loads (no registers, two stages in flight behind the one in
//     use; rows XOR-swizzled against bank conflicts).  Q4_0 weights go through
//     registers into two padded LDS stages, widened to int8 (c - 8) on the way,
//     so the inner loop is the same for both formats;
//   * the token tiles of all active experts are numbered by the bucketing
//     kernel (tile_map); block ids are spread so that one XCD works on
//     consecutive token tiles of the same weight rows, which then hit its L2.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "mfma_ops.h"

namespace moe {

constexpr int MF_MT = GEMM_TILE_M;        // token columns per workgroup
constexpr int MF_NT = 128;                // weight rows per workgroup
constexpr int MF_KB = 4;                  // blocks of 32 per LDS stage
constexpr int MF_THREADS = 256;

struct MfArgs {
    const uint8_t* base;          // expert packs (group mode) or the dense matrix
    size_t group_stride;          // bytes per expert
    const uint8_t* const* etab;   // group mode: expert pack addresses, or null (base + e * stride)
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
    size_t ts_off;                // NVFP4 group mode: tensor scales (gate, up, down fp32) in a pack
};

// ---------------------------------------------------------------------------
// Shared pieces of both kernels.

// The workgroup's tile: block id -> (row tile nt, token tile); the rows of its
// token columns go to s_row (activation rows) and s_orow (output rows).
// Returns false when the workgroup has no tile.  Consecutive ids of one XCD
// (ids are dealt to the 8 XCDs round-robin) get consecutive token tiles of the
// same row tile.
struct MfTile {
    const uint8_t* mat;
    int nt, m0, ncol;
};

__device__ __forceinline__ bool mf_tile(const MfArgs& A, MfTile& t, int* s_row, int* s_orow) {
    const int nb_all = gridDim.x;
    const int lid = (blockIdx.x & 7) * (nb_all >> 3) + (blockIdx.x >> 3);
    t.nt = lid / A.max_tiles;
    const int g = lid - t.nt * A.max_tiles;
    if (t.nt >= A.rows / MF_NT) return false;
    const int32_t* lst = nullptr;
    int cnt;
    if (A.b.ctrl) {
        if (g >= (int)A.b.ctrl[CW_N_TILES]) return false;
        const int tm = A.tile_map[g];
        const int e = tm & 0xffff;
        t.m0 = (tm >> 16) * MF_MT;
        cnt = A.b.counts[e];
        lst = A.b.lists + (size_t)e * A.T;
        t.mat = expert_pack(A.base, A.etab, e, A.group_stride);
    } else {
        t.m0 = g * MF_MT;
        if (t.m0 >= A.T) return false;
        cnt = A.T;
        t.mat = A.base;
    }
    t.ncol = min(MF_MT, cnt - t.m0);
    if ((int)threadIdx.x < MF_MT) {
        const int c = min((int)threadIdx.x, t.ncol - 1);   // columns past the tokens repeat the last
        const int o = lst ? lst[t.m0 + c] : t.m0 + c;
        s_orow[threadIdx.x] = o;
        s_row[threadIdx.x] = o / A.act_div;
    }
    return true;
}

// The wave's place in the tile: rows wr*64 + [0,32) (accumulator 0) and
// + [32,64) (accumulator 1), token columns wc*32 + [0,32).
struct MfWave {
    int wr, wc, half, l32;
};

// One stage (MF_KB blocks) of a wave: frag(kb, a0, a1, bx) fetches the code
// operands of block kb, sfrag(kb, d0, d1, dc) the binary16 scale operands
// (row / column l32's d at k = 0 in lanes 0..31, zero elsewhere; a zero-
// extended 16-bit load gives the first register, the second is zero).  Block
// kb+1's products are issued before block kb is rescaled.
template <bool SWIGLU, bool TAP, class SOp = h4, bool NEG = false, bool NV4 = false, class Frag,
          class SFrag>
__device__ __forceinline__ void mf_stage(const MfArgs& A, const MfTile& t, const MfWave& w, int s,
                                         const int* s_orow, Frag frag, SFrag sfrag,
                                         float (&acc0)[16], float (&acc1)[16]) {
    v4i a0, a1, bx;
    SOp d0, d1, dc;
    frag(0, a0, a1, bx);
    sfrag(0, d0, d1, dc);
    v16i i0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bx, v16i{}, 0, 0, 0);
    v16i i1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bx, v16i{}, 0, 0, 0);
    v16f s0 = scale_mfma(d0, dc);
    v16f s1 = scale_mfma(d1, dc);
#pragma unroll
    for (int kb = 0; kb < MF_KB; ++kb) {
        v16i n0, n1;
        v16f t0, t1;
        if (kb + 1 < MF_KB) {
            frag(kb + 1, a0, a1, bx);
            sfrag(kb + 1, d0, d1, dc);
            n0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bx, v16i{}, 0, 0, 0);
            n1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bx, v16i{}, 0, 0, 0);
            t0 = scale_mfma(d0, dc);
            t1 = scale_mfma(d1, dc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc0[i] = fmaf((float)i0[i], s0[i], acc0[i]);
            acc1[i] = fmaf((float)i1[i], s1[i], acc1[i]);
        }
        if constexpr (TAP) {
            const int c = w.wc * 32 + w.l32;
            const int o = s_orow[c];
            if (A.tap_isum && c < t.ncol && o / A.tap_div < A.tap_tokens) {
                const int nb = A.K / QK;
                const int blk = s * MF_KB + kb;
                for (int i = 0; i < 16; ++i) {
                    for (int q = 0; q < 2; ++q) {
                        const int pr = t.nt * MF_NT + w.wr * 64 + q * 32 + mf_row_of(i, w.half);
                        // canonical row: gate/up rows are stored as 32 gate + 32 up per slab
                        const int cr = SWIGLU ? ((pr & 63) < 32 ? (pr >> 6) * 32 + (pr & 31)
                                                                : A.F + (pr >> 6) * 32 + (pr & 31))
                                              : pr;
                        // (NEG: the staged codes were negated, so the sum is too)
                        const int v = q ? i1[i] : i0[i];
                        if constexpr (NV4) {
                            // staged block blk is half blk & 1 of block blk / 2: the
                            // tap holds the two half sums as 16-bit halves
                            reinterpret_cast<int16_t*>(A.tap_isum + ((size_t)o * A.rows + cr) * nb +
                                                       (blk >> 1))[blk & 1] = (int16_t)v;
                        } else {
                            A.tap_isum[((size_t)o * A.rows + cr) * nb + blk] = NEG ? -v : v;
                        }
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
}

// Epilogue: SwiGLU + Q8_1 of h (gate/up), or the fp32 rows (down, dense).
template <bool SWIGLU, bool TAP>
__device__ __forceinline__ void mf_epilogue(const MfArgs& A, const MfTile& t, const MfWave& w,
                                            const int* s_orow, const float (&acc0)[16],
                                            const float (&acc1)[16]) {
    const int c = w.wc * 32 + w.l32;
    const bool valid = c < t.ncol;
    const int o = s_orow[c];
    const int half = w.half;
    if constexpr (SWIGLU) {
        // rows wr*64 + [0,32) are gate rows f, + [32,64) the up rows of the same f
        const int fb = t.nt * 2 + w.wr;     // Q8_1 block of h along F
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
            float* orow = A.out + (size_t)o * A.rows + t.nt * MF_NT + w.wr * 64 + half * 4;
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
// Q8_0: three-stage LDS ring filled by direct global->LDS loads.
//
// Stage layout (bytes): codes W [128 rows][128] at 0, codes X [64 tokens][128]
// at 16384, d_w [128 rows][4 x binary16] at 24576, d_a [64 tokens][4 x u32
// (d16 | s16 << 16)] at 25600.  A load instruction writes 64 lanes x 16 bytes
// (x 4 bytes for d_w) contiguously, so the code rows cannot be padded; the
// 16-byte chunk c of row r sits in slot c ^ mf_swz(r) instead.  mf_swz gives
// distinct slots to rows 0..7 (and 8..15), and to the even and the odd rows of
// 0..15, so the fragment reads (16 lanes = rows r..r+15 of one chunk) hit
// distinct banks with either 32 or 64 LDS banks.
constexpr int MD_W = 0, MD_X = MF_NT * 128, MD_DW = MD_X + MF_MT * 128, MD_DA = MD_DW + MF_NT * 8;
constexpr int MD_STAGE = MD_DA + MF_MT * 16;   // 26624
constexpr int MD_NS = 3;                       // stages in the ring

__device__ __forceinline__ int mf_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef __attribute__((address_space(3))) char lds_char;

// Direct global->LDS loads: lane i writes its 16 (4) bytes at LDS address
// lds + 16 i (4 i).  Issued from asm so that the compiler does not add its own
// wait for all such loads before every later LDS read (it cannot tell the
// ring's stages apart); the kernel's wait_stage() is the only wait.  The loads
// write no registers: the address registers are read when the load issues.
__device__ __forceinline__ uint32_t lds_addr(const char* l) {
    return (uint32_t)(uintptr_t)(const lds_char*)l;
}
// reads at an LDS byte address
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ v4i lds_ld16(uint32_t a) { return *(const lds_v4i*)(uintptr_t)a; }
__device__ __forceinline__ uint32_t lds_ldu16(uint32_t a) { return *(const lds_u16*)(uintptr_t)a; }
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lds), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(lds), "v"(g) : "memory", "m0");
}

template <bool SWIGLU, bool TAP>
__global__ __launch_bounds__(MF_THREADS, 2) void k_mfma_dma(MfArgs A) {
    __shared__ __align__(16) char ring[MD_NS * MD_STAGE];
    __shared__ __align__(16) char zero16[16];
    __shared__ int s_row[MF_MT], s_orow[MF_MT];

    MfTile t;
    if (!mf_tile(A, t, s_row, s_orow)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < 4) reinterpret_cast<uint32_t*>(zero16)[tid] = 0u;
    __syncthreads();

    const int K = A.K, nb = K / QK;
    const size_t rowb = (size_t)nb * 32;
    const uint8_t* codes = t.mat + A.codes_off + (size_t)t.nt * MF_NT * rowb;
    const uint8_t* scl = t.mat + A.scales_off + (size_t)t.nt * MF_NT * nb * 2;

    // this wave's loads of a stage, as per-lane sources at stage 0 (a stage
    // advances codes by 128 bytes, d_w by 8 and d_a by 16):
    //   codes W: instructions 4*wave .. 4*wave+3, rows 8i + lane/8, chunk (lane%8) ^ swz
    //   codes X: instructions 2*wave, 2*wave+1, token rows 8i + lane/8
    //   d_w:     instruction wave, rows 32*wave + lane/2, 4 bytes (lane%2)
    //   d_a:     wave 0, token lane, 16 bytes
    const uint8_t* srcW[4];
    const int8_t* srcX[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (4 * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ mf_swz(r);
        srcW[j] = codes + (size_t)r * rowb + c * 16;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 8 * (2 * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ mf_swz(r);
        srcX[j] = A.ain.q + (size_t)s_row[r] * K + c * 16;
    }
    const uint8_t* srcDW = scl + ((size_t)(32 * wave + (lane >> 1)) * nb) * 2 + (lane & 1) * 4;
    const uint32_t* srcDA = A.ain.ds + (size_t)s_row[lane] * nb;
    const uint32_t ring0 = lds_addr(ring);
    const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int s) {
        const uint32_t st = ring0 + (uint32_t)(s % MD_NS) * MD_STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(srcW[j] + s * 128, st + MD_W + (4 * wv + j) * 1024);
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(srcX[j] + s * 128, st + MD_X + (2 * wv + j) * 1024);
        dma4(srcDW + s * 8, st + MD_DW + wv * 256);
        if (wv == 0) dma16(srcDA + s * MF_KB, st + MD_DA);
    };
    // wait until this wave's loads of the stage about to be used have landed
    // (at most one later stage of loads may stay in flight), then a barrier so
    // that every wave's loads have, and every wave is done with the buffer the
    // next loads refill: a wave issues 8 (wave 0) or 7 loads per stage.  The
    // tapped kernel also stores inside the loop, so it drains every time.
    auto wait_stage = [&](bool later) {
        if (TAP || !later) {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else if (wave == 0) {
            asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };

    MfWave w{wave & 1, wave >> 1, lane >> 5, lane & 31};
    const bool busy = w.wc * 32 < t.ncol;   // a wave past the tile's tokens only loads
    // chunk c = 2kb + half of row r sits in slot c ^ swz(r): byte offset
    // (2kb * 16) ^ ((half ^ swz(r)) * 16) within the row
    const int ra = w.wr * 64 + w.l32, rb = w.wc * 32 + w.l32;
    const int fa = (w.half ^ mf_swz(ra)) * 16, fbx = (w.half ^ mf_swz(rb)) * 16;
    int offA[MF_KB], offB[MF_KB];
#pragma unroll
    for (int kb = 0; kb < MF_KB; ++kb) {
        offA[kb] = lds_addr(ring) + MD_W + ra * 128 + ((kb * 32) ^ fa);
        offB[kb] = lds_addr(ring) + MD_X + rb * 128 + ((kb * 32) ^ fbx);
    }
    // scale entries: lanes 32..63 read zeros
    const uint32_t oW0 = w.half ? lds_addr(zero16) : lds_addr(ring) + MD_DW + ra * 8;
    const uint32_t oW1 = w.half ? lds_addr(zero16) : lds_addr(ring) + MD_DW + (ra + 32) * 8;
    const uint32_t oDA = w.half ? lds_addr(zero16) : lds_addr(ring) + MD_DA + rb * 16;
    const int kw2 = w.half ? 0 : 2, kw4 = w.half ? 0 : 4;   // per-block steps of those entries
    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.0f;

    // stage s of the ring buffer B (= s % MD_NS, a constant in each copy)
    auto stage = [&](int s, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        const int stages = nb / MF_KB;
        wait_stage(s + 1 < stages);
        if (s + 2 < stages) issue(s + 2);
        if (!busy) return;
        const uint32_t sb = (uint32_t)B * MD_STAGE;                     // buffer base
        const uint32_t sbz = w.half ? 0u : sb;                          // zero entries stay put
        auto frag = [&](int kb, v4i& a0, v4i& a1, v4i& bx) {
            a0 = lds_ld16(offA[kb] + sb);
            a1 = lds_ld16(offA[kb] + sb + 32 * 128);
            bx = lds_ld16(offB[kb] + sb);
        };
        auto sfrag = [&](int kb, h4& d0, h4& d1, h4& dc) {
            d0 = scale_op(lds_ldu16(oW0 + sbz + kb * kw2));
            d1 = scale_op(lds_ldu16(oW1 + sbz + kb * kw2));
            dc = scale_op(lds_ldu16(oDA + sbz + kb * kw4));
        };
        mf_stage<SWIGLU, TAP>(A, t, w, s, s_orow, frag, sfrag, acc0, acc1);
    };

    const int stages = nb / MF_KB;
    issue(0);
    if (stages > 1) issue(1);
    for (int s = 0; s < stages; s += MD_NS) {
        stage(s, std::integral_constant<int, 0>{});
        if (s + 1 < stages) stage(s + 1, std::integral_constant<int, 1>{});
        if (s + 2 < stages) stage(s + 2, std::integral_constant<int, 2>{});
    }
    mf_epilogue<SWIGLU, TAP>(A, t, w, s_orow, acc0, acc1);
}

// ---------------------------------------------------------------------------
// Q4_0: two padded LDS stages filled through registers, codes widened to int8.
constexpr int MS_ROWB = MF_KB * QK + 16;  // LDS bytes per staged row (padded)
// binary16 scales of a stage: [block][MF_NT + 32] and [block][MF_MT + 32]; the
// last 32 entries of each row stay zero (the f16 outer product reads them in
// lanes 32..63)
constexpr int MS_SWR = MF_NT + 32, MS_SAR = MF_MT + 32;

// Q5_1 (FMT): the fifth bits come from each block's side data {d | m << 16, qh},
// the codes widen to int8 0..31, and each stage adds the min terms
// sum_b m_w[r][b] * s_a[t][b] with one more f16 outer product per row tile:
// the four blocks' m and s in the k slots 0..3 of lanes 0..31.
// Q3_K (FMT): a stage of four blocks is half a super-block.  Each element
// widens to w = -(code * scale) of its 16-element sub-block, in [-128, 124]
// (the code in [-4, 3], the scale in [-32, 31]), by a byte lookup (v_perm) in
// the sub-block's table (4 - v) * scale over v = code + 4; the block's matrix-
// core sum is then minus its integer sum, exact, and the rows' scale operand
// is -d (a sign flip of the binary16 d).
template <bool SWIGLU, bool TAP, int FMT>
__global__ __launch_bounds__(MF_THREADS, 2) void k_mfma_q4(MfArgs A) {
    constexpr bool Q5 = FMT == MOE_FMT_Q5_1;
    constexpr bool K3 = FMT == MOE_FMT_Q3_K;
    constexpr int QB = 16;                                // code bytes per Q4_0 / Q5_1 block
    constexpr int WBYTES = MF_NT * MS_ROWB, XBYTES = MF_MT * MS_ROWB;
    constexpr int SCB = MF_KB * MS_SWR * 2 + MF_KB * MS_SAR * 2;
    constexpr int MINB = Q5 ? (MF_NT + MF_MT) * MF_KB * 2 : 0;   // m_w [row][4], s_a [col][4]
    constexpr int STAGE = WBYTES + XBYTES + SCB + MINB;
    __shared__ __align__(16) char smem[2 * STAGE];
    __shared__ int s_row[MF_MT], s_orow[MF_MT];

    MfTile t;
    if (!mf_tile(A, t, s_row, s_orow)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    {
        // zero tails of the scale rows, both stage buffers
        const int buf = tid >> 7, kb = (tid >> 5) & 3, z = tid & 31;
        uint16_t* sdw = reinterpret_cast<uint16_t*>(smem + buf * STAGE + WBYTES + XBYTES);
        sdw[kb * MS_SWR + MF_NT + z] = 0;
        sdw[MF_KB * MS_SWR + kb * MS_SAR + MF_MT + z] = 0;
    }
    __syncthreads();

    const int K = A.K, nb = K / QK, nsb = nb / 8;
    const size_t rowb = K3 ? (size_t)nsb * 108 : (size_t)nb * QB;
    const uint8_t* codes = t.mat + A.codes_off + (size_t)t.nt * MF_NT * rowb;
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(t.mat + A.scales_off) + (size_t)t.nt * MF_NT * nb;
    const uint2* side = reinterpret_cast<const uint2*>(t.mat + A.scales_off) + (size_t)t.nt * MF_NT * nb;
    // Q3_K: one binary16 d per row and super-block
    const uint16_t* sbd = reinterpret_cast<const uint16_t*>(t.mat + A.scales_off) + (size_t)t.nt * MF_NT * nsb;

    // ---- global -> registers -> LDS staging of one stage (blocks kb0 .. kb0+MF_KB)
    constexpr int WCH = 2;                     // 16-byte chunks (= blocks) per thread
    constexpr int WCPR = MF_KB * QB / 16;      // chunks per weight row per stage
    v4i rw[WCH];
    uint32_t rq[WCH];                          // Q5_1: qh of each chunk's block
    v4i rx[2];
    uint2 rdw;
    v4i rsd[2];                                // Q5_1: the row's side data, 4 blocks
    v4i rda;
    v4i rs3[WCH];                              // Q3_K: each chunk's super-block scale bytes
    uint32_t rd3 = 0;                          // Q3_K: the row's d (this stage's super-block)
    auto gload = [&](int kb0) {
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int r = ch / WCPR, p = ch - r * WCPR;
            if constexpr (K3) {
                // block kb0 + p: 12 code bytes, and the super-block's 12 scale bytes
                const int blk = kb0 + p;
                const uint8_t* u = codes + (size_t)r * rowb + (size_t)(blk >> 3) * 108;
                const uint32_t* cw = reinterpret_cast<const uint32_t*>(u + (blk & 7) * 12);
                const uint32_t* sw = reinterpret_cast<const uint32_t*>(u + 96);
                rw[j] = v4i{(int)cw[0], (int)cw[1], (int)cw[2], 0};
                rs3[j] = v4i{(int)sw[0], (int)sw[1], (int)sw[2], 0};
            } else {
                rw[j] = ld16(codes + (size_t)r * rowb + (size_t)kb0 * QB + p * 16);
            }
            if constexpr (Q5) rq[j] = side[(size_t)r * nb + kb0 + p].y;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int c = ch >> 3, p = ch & 7;
            rx[j] = ld16(A.ain.q + (size_t)s_row[c] * K + (size_t)kb0 * QK + p * 16);
        }
        if (tid < MF_NT) {
            if constexpr (K3) {
                rd3 = sbd[(size_t)tid * nsb + (kb0 >> 3)];
            } else if constexpr (Q5) {
                rsd[0] = ld16(side + (size_t)tid * nb + kb0);
                rsd[1] = ld16(side + (size_t)tid * nb + kb0 + 2);
            } else {
                rdw = *reinterpret_cast<const uint2*>(scl + (size_t)tid * nb + kb0);
            }
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
            rda = *reinterpret_cast<const v4i*>(A.ain.ds + (size_t)s_row[c] * nb + kb0);
        }
    };
    auto lstore = [&](int buf, int kb0w) {
        char* st = smem + buf * STAGE;
        int8_t* sw = reinterpret_cast<int8_t*>(st);
        int8_t* sx = reinterpret_cast<int8_t*>(st + WBYTES);
        uint16_t* sdw = reinterpret_cast<uint16_t*>(st + WBYTES + XBYTES);
        uint16_t* sda = sdw + MF_KB * MS_SWR;
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int r = ch / WCPR, p = ch - r * WCPR;
            // one block (16 bytes) -> 32 int8: elements 0..15, then 16..31
            v4i lo, hi;
            if constexpr (K3) {
                int sc0, sc1;
                k3_scales(rs3[j], (kb0w + p) & 7, sc0, sc1);
                // byte tables (4 - v) * scale, v = 0..7: low word v < 4, high word v >= 4
                auto table = [](int sc, uint32_t& tlo, uint32_t& thi) {
                    tlo = (uint32_t)(4 * sc & 0xFF) | (uint32_t)(3 * sc & 0xFF) << 8 |
                          (uint32_t)(2 * sc & 0xFF) << 16 | (uint32_t)(sc & 0xFF) << 24;
                    thi = (uint32_t)(-sc & 0xFF) << 8 | (uint32_t)(-2 * sc & 0xFF) << 16 |
                          (uint32_t)(-3 * sc & 0xFF) << 24;
                };
                uint32_t t0lo, t0hi, t1lo, t1hi;
                table(sc0, t0lo, t0hi);
                table(sc1, t1lo, t1hi);
                const uint32_t H = (uint32_t)rw[j].z;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t v0 = (((uint32_t)rw[j].x >> (2 * m)) & 0x03030303u) |
                                        (((H >> m) & 0x01010101u) << 2);
                    const uint32_t v1 = (((uint32_t)rw[j].y >> (2 * m)) & 0x03030303u) |
                                        (((H >> (4 + m)) & 0x01010101u) << 2);
                    lo[m] = (int)__builtin_amdgcn_perm(t0hi, t0lo, v0);
                    hi[m] = (int)__builtin_amdgcn_perm(t1hi, t1lo, v1);
                }
                *reinterpret_cast<v4i*>(sw + r * MS_ROWB + p * 32) = lo;
                *reinterpret_cast<v4i*>(sw + r * MS_ROWB + p * 32 + 16) = hi;
                continue;
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t x = (uint32_t)rw[j][d];
                if constexpr (Q5) {
                    lo[d] = (int)(x & 0x0F0F0F0Fu) | spread4((rq[j] >> (4 * d)) & 15u);
                    hi[d] = (int)((x >> 4) & 0x0F0F0F0Fu) | spread4((rq[j] >> (16 + 4 * d)) & 15u);
                } else {
                    lo[d] = (int)q4_widen(x & 0x0F0F0F0Fu);
                    hi[d] = (int)q4_widen((x >> 4) & 0x0F0F0F0Fu);
                }
            }
            *reinterpret_cast<v4i*>(sw + r * MS_ROWB + p * 32) = lo;
            *reinterpret_cast<v4i*>(sw + r * MS_ROWB + p * 32 + 16) = hi;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int c = ch >> 3, p = ch & 7;
            *reinterpret_cast<v4i*>(sx + c * MS_ROWB + p * 16) = rx[j];
        }
        if (tid < MF_NT) {
            if constexpr (K3) {
                const uint16_t nd = (uint16_t)(rd3 ^ 0x8000u);     // -d
#pragma unroll
                for (int q = 0; q < MF_KB; ++q) sdw[q * MS_SWR + tid] = nd;
            } else if constexpr (Q5) {
                // side words: {d | m << 16, qh} per block; blocks 0,1 in rsd[0], 2,3 in rsd[1]
                const uint32_t dm[4] = {(uint32_t)rsd[0].x, (uint32_t)rsd[0].z, (uint32_t)rsd[1].x,
                                        (uint32_t)rsd[1].z};
                uint16_t* smw = sda + MF_KB * MS_SAR;
#pragma unroll
                for (int q = 0; q < MF_KB; ++q) sdw[q * MS_SWR + tid] = (uint16_t)(dm[q] & 0xffffu);
                *reinterpret_cast<uint2*>(smw + tid * MF_KB) =
                    uint2{(dm[0] >> 16) | (dm[1] & 0xffff0000u), (dm[2] >> 16) | (dm[3] & 0xffff0000u)};
            } else {
                sdw[0 * MS_SWR + tid] = (uint16_t)(rdw.x & 0xffffu);
                sdw[1 * MS_SWR + tid] = (uint16_t)(rdw.x >> 16);
                sdw[2 * MS_SWR + tid] = (uint16_t)(rdw.y & 0xffffu);
                sdw[3 * MS_SWR + tid] = (uint16_t)(rdw.y >> 16);
            }
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
#pragma unroll
            for (int q = 0; q < MF_KB; ++q) sda[q * MS_SAR + c] = (uint16_t)((uint32_t)rda[q] & 0xffffu);
            if constexpr (Q5) {
                // the activation blocks' stored s (high halves of ds)
                uint16_t* sas = sda + MF_KB * MS_SAR + MF_NT * MF_KB;
                *reinterpret_cast<uint2*>(sas + c * MF_KB) =
                    uint2{((uint32_t)rda[0] >> 16) | ((uint32_t)rda[1] & 0xffff0000u),
                          ((uint32_t)rda[2] >> 16) | ((uint32_t)rda[3] & 0xffff0000u)};
            }
        }
    };

    MfWave w{wave & 1, wave >> 1, lane >> 5, lane & 31};
    // scale entries of this lane (the zero tails in lanes 32..63)
    const int o_w0 = w.half ? MF_NT + w.l32 : w.wr * 64 + w.l32;
    const int o_w1 = w.half ? MF_NT + w.l32 : w.wr * 64 + 32 + w.l32;
    const int o_a = w.half ? MF_MT + w.l32 : w.wc * 32 + w.l32;
    const bool busy = w.wc * 32 < t.ncol;   // a wave past the tile's tokens only stages
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
        const uint16_t* sda = sdw + MF_KB * MS_SWR;
        auto frag = [&](int kb, v4i& a0, v4i& a1, v4i& bx) {
            a0 = *reinterpret_cast<const v4i*>(sw + (w.wr * 64 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
            a1 = *reinterpret_cast<const v4i*>(sw + (w.wr * 64 + 32 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
            bx = *reinterpret_cast<const v4i*>(sx + (w.wc * 32 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
        };
        auto sfrag = [&](int kb, h4& d0, h4& d1, h4& dc) {
            d0 = scale_op(sdw[kb * MS_SWR + o_w0]);
            d1 = scale_op(sdw[kb * MS_SWR + o_w1]);
            dc = scale_op(sda[kb * MS_SAR + o_a]);
        };
        mf_stage<SWIGLU, TAP, h4, K3>(A, t, w, s, s_orow, frag, sfrag, acc0, acc1);
        if constexpr (Q5) {
            // min terms of the stage's four blocks (k slots 0..3; lanes 32..63 zero)
            const uint16_t* smw = sda + MF_KB * MS_SAR;
            const uint16_t* sas = smw + MF_NT * MF_KB;
            const h4 z{};
            const h4 m0 = *reinterpret_cast<const h4*>(smw + (w.wr * 64 + w.l32) * MF_KB);
            const h4 m1 = *reinterpret_cast<const h4*>(smw + (w.wr * 64 + 32 + w.l32) * MF_KB);
            const h4 sv = *reinterpret_cast<const h4*>(sas + (w.wc * 32 + w.l32) * MF_KB);
            const v16f p0 = __builtin_amdgcn_mfma_f32_32x32x8f16(w.half ? z : m0, w.half ? z : sv,
                                                                 v16f{}, 0, 0, 0);
            const v16f p1 = __builtin_amdgcn_mfma_f32_32x32x8f16(w.half ? z : m1, w.half ? z : sv,
                                                                 v16f{}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc0[i] += p0[i];
                acc1[i] += p1[i];
            }
        }
    };
    gload(0);
    lstore(0, 0);
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s + 1 < stages; ++s) {
        gload((s + 1) * MF_KB);
        compute(s & 1, s);
        lstore((s + 1) & 1, (s + 1) * MF_KB);
        __syncthreads();
    }
    compute((stages - 1) & 1, stages - 1);
    mf_epilogue<SWIGLU, TAP>(A, t, w, s_orow, acc0, acc1);
}

// ---------------------------------------------------------------------------
// NVFP4 (edge0-strata README, section "Changes from upstream Strata", NVFP4
// latent experts; read as FP4 E2M1 codes, an FP8 E4M3 scale per 16 elements and
// an fp32 scale per tensor).  Each 16-element half of a block is staged as a
// block of its own: the half's codes widened to int8 2 * e2m1 (v_perm table
// lookups, as in the matrix-vector kernels) and then 16 zero bytes, the matching
// activation half beside them; so one int8 MFMA gives the half's exact sum, and
// its scale operand is e4m3(s) / 2 in binary16 (exact) against d_a.  A stage of
// MF_KB staged blocks covers two blocks.  The tensor scales multiply the fp32
// accumulators before the epilogue.
template <bool SWIGLU, bool TAP>
__global__ __launch_bounds__(MF_THREADS, 2) void k_mfma_nv4(MfArgs A) {
    constexpr int WBYTES = MF_NT * MS_ROWB, XBYTES = MF_MT * MS_ROWB;
    constexpr int SCB = MF_KB * MS_SWR * 2 + MF_KB * MS_SAR * 2;
    constexpr int STAGE = WBYTES + XBYTES + SCB;
    __shared__ __align__(16) char smem[2 * STAGE];
    __shared__ int s_row[MF_MT], s_orow[MF_MT];

    MfTile t;
    if (!mf_tile(A, t, s_row, s_orow)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    {
        // zero tails of the scale rows, both stage buffers
        const int buf = tid >> 7, kb = (tid >> 5) & 3, z = tid & 31;
        uint16_t* sdw = reinterpret_cast<uint16_t*>(smem + buf * STAGE + WBYTES + XBYTES);
        sdw[kb * MS_SWR + MF_NT + z] = 0;
        sdw[MF_KB * MS_SWR + kb * MS_SAR + MF_MT + z] = 0;
        // the upper 16 bytes of every staged weight block stay zero (both buffers):
        // 2 x 128 rows x 4 blocks
        for (int i = tid; i < 2 * MF_NT * MF_KB; i += MF_THREADS) {
            const int b = i / (MF_NT * MF_KB), r = (i / MF_KB) % MF_NT, q = i % MF_KB;
            *reinterpret_cast<v4i*>(smem + b * STAGE + r * MS_ROWB + q * QK + 16) = v4i{0, 0, 0, 0};
        }
    }
    __syncthreads();

    const int K = A.K, nb = K / QK;
    const size_t rowb = (size_t)nb * 16;
    const uint8_t* codes = t.mat + A.codes_off + (size_t)t.nt * MF_NT * rowb;
    // two E4M3 bytes per block (half 0 low)
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(t.mat + A.scales_off) + (size_t)t.nt * MF_NT * nb;

    // stage s holds blocks 2s and 2s + 1 (staged blocks 4s .. 4s + 3)
    v4i rw, rx;
    uint32_t rdw = 0;
    uint2 rda = uint2{0u, 0u};
    auto gload = [&](int s) {
        const int b0 = 2 * s;
        {
            const int r = tid >> 1, p = tid & 1;               // 128 rows x 2 blocks
            rw = ld16(codes + (size_t)r * rowb + (size_t)(b0 + p) * 16);
        }
        {
            const int c = tid >> 2, p = tid & 3;               // 64 tokens x 4 halves
            rx = ld16(A.ain.q + (size_t)s_row[c] * K + (size_t)b0 * QK + p * 16);
        }
        if (tid < MF_NT) {
            rdw = *reinterpret_cast<const uint32_t*>(scl + (size_t)tid * nb + b0);
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
            rda = *reinterpret_cast<const uint2*>(A.ain.ds + (size_t)s_row[c] * nb + b0);
        }
    };
    auto lstore = [&](int buf) {
        char* st = smem + buf * STAGE;
        int8_t* sw = reinterpret_cast<int8_t*>(st);
        int8_t* sx = reinterpret_cast<int8_t*>(st + WBYTES);
        uint16_t* sdw = reinterpret_cast<uint16_t*>(st + WBYTES + XBYTES);
        uint16_t* sda = sdw + MF_KB * MS_SWR;
        {
            // block p of the row: low nibbles = half 0 -> staged block 2p, high -> 2p + 1
            const int r = tid >> 1, p = tid & 1;
            v4i lo, hi;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t x = (uint32_t)rw[d];
                lo[d] = e2m1x2_widen(x & 0x0F0F0F0Fu);
                hi[d] = e2m1x2_widen((x >> 4) & 0x0F0F0F0Fu);
            }
            *reinterpret_cast<v4i*>(sw + r * MS_ROWB + (2 * p) * QK) = lo;
            *reinterpret_cast<v4i*>(sw + r * MS_ROWB + (2 * p + 1) * QK) = hi;
        }
        {
            // half p & 1 of block p / 2 of the token = staged block p
            const int c = tid >> 2, p = tid & 3;
            *reinterpret_cast<v4i*>(sx + c * MS_ROWB + p * QK) = rx;
        }
        if (tid < MF_NT) {
#pragma unroll
            for (int q = 0; q < MF_KB; ++q)
                sdw[q * MS_SWR + tid] = (uint16_t)f2h_bits(0.5f * e4m3f((rdw >> (8 * q)) & 0xFFu));
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
#pragma unroll
            for (int q = 0; q < MF_KB; ++q)
                sda[q * MS_SAR + c] = (uint16_t)(((q >> 1) ? rda.y : rda.x) & 0xffffu);
        }
    };

    MfWave w{wave & 1, wave >> 1, lane >> 5, lane & 31};
    const int o_w0 = w.half ? MF_NT + w.l32 : w.wr * 64 + w.l32;
    const int o_w1 = w.half ? MF_NT + w.l32 : w.wr * 64 + 32 + w.l32;
    const int o_a = w.half ? MF_MT + w.l32 : w.wc * 32 + w.l32;
    const bool busy = w.wc * 32 < t.ncol;   // a wave past the tile's tokens only stages
    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.0f;

    const int stages = nb / 2;
    auto compute = [&](int buf, int s) {
        if (!busy) return;
        const char* st = smem + buf * STAGE;
        const int8_t* sw = reinterpret_cast<const int8_t*>(st);
        const int8_t* sx = reinterpret_cast<const int8_t*>(st + WBYTES);
        const uint16_t* sdw = reinterpret_cast<const uint16_t*>(st + WBYTES + XBYTES);
        const uint16_t* sda = sdw + MF_KB * MS_SWR;
        auto frag = [&](int kb, v4i& a0, v4i& a1, v4i& bx) {
            a0 = *reinterpret_cast<const v4i*>(sw + (w.wr * 64 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
            a1 = *reinterpret_cast<const v4i*>(sw + (w.wr * 64 + 32 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
            bx = *reinterpret_cast<const v4i*>(sx + (w.wc * 32 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
        };
        auto sfrag = [&](int kb, h4& d0, h4& d1, h4& dc) {
            d0 = scale_op(sdw[kb * MS_SWR + o_w0]);
            d1 = scale_op(sdw[kb * MS_SWR + o_w1]);
            dc = scale_op(sda[kb * MS_SAR + o_a]);
        };
        mf_stage<SWIGLU, TAP, h4, false, true>(A, t, w, s, s_orow, frag, sfrag, acc0, acc1);
    };
    gload(0);
    lstore(0);
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s + 1 < stages; ++s) {
        gload(s + 1);
        compute(s & 1, s);
        lstore((s + 1) & 1);
        __syncthreads();
    }
    compute((stages - 1) & 1, stages - 1);
    if (A.ts_off) {
        // gate rows (acc0) and up rows (acc1) of the slab, or the down rows
        const float* ts = reinterpret_cast<const float*>(t.mat + A.ts_off);
        const float s0 = SWIGLU ? ts[0] : ts[2], s1 = SWIGLU ? ts[1] : ts[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc0[i] *= s0;
            acc1[i] *= s1;
        }
    }
    mf_epilogue<SWIGLU, TAP>(A, t, w, s_orow, acc0, acc1);
}

// ---------------------------------------------------------------------------
// Q4_K / Q5_K (FMT): a stage of four blocks is half a super-block.  Its 64
// nibble bytes widen to int8 (plus Q5_K's fifth bits from qh): nibble byte
// 32g' + i of the stage gives element i of stage block 2g' (low nibble) and of
// 2g' + 1 (high nibble).  A row's scale for stage block q is d * scale_b and
// its min product dmin * min_b (b = the sub-block), both exact in fp32 and
// taken to the matrix cores as fp32 (v_mfma_f32_32x32x2_f32): the rescale uses
// d * scale_b x d_a, and each stage subtracts sum_q dmin*min_q[r] x d_a*sum(q_a)[t]
// with two more fp32 outer products (two blocks each, in the two k slots).
template <bool SWIGLU, bool TAP, int FMT>
__global__ __launch_bounds__(MF_THREADS, 2) void k_mfma_kq(MfArgs A) {
    constexpr bool K5 = FMT == MOE_FMT_Q5_K;
    constexpr int SIDE = K5 ? 48 : 16;                   // side bytes per super-block
    constexpr int WBYTES = MF_NT * MS_ROWB, XBYTES = MF_MT * MS_ROWB;
    constexpr int SW32 = MF_KB * MS_SWR * 4, SA32 = MF_KB * MS_SAR * 4;
    constexpr int MW32 = MF_KB * MF_NT * 4, MA32 = MF_KB * MF_MT * 4;
    constexpr int STAGE = WBYTES + XBYTES + SW32 + SA32 + MW32 + MA32;
    __shared__ __align__(16) char smem[2 * STAGE];
    __shared__ int s_row[MF_MT], s_orow[MF_MT];

    MfTile t;
    if (!mf_tile(A, t, s_row, s_orow)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    {
        // zero tails of the fp32 scale rows, both stage buffers
        const int buf = tid >> 7, kb = (tid >> 5) & 3, z = tid & 31;
        float* sdw = reinterpret_cast<float*>(smem + buf * STAGE + WBYTES + XBYTES);
        sdw[kb * MS_SWR + MF_NT + z] = 0.0f;
        sdw[MF_KB * MS_SWR + kb * MS_SAR + MF_MT + z] = 0.0f;
    }
    __syncthreads();

    const int K = A.K, nb = K / QK, nsb = nb / 8;
    const size_t rowb = (size_t)nb * 16;
    const uint8_t* codes = t.mat + A.codes_off + (size_t)t.nt * MF_NT * rowb;
    const uint8_t* side = t.mat + A.scales_off + (size_t)t.nt * MF_NT * nsb * SIDE;

    constexpr int WCH = 2;                      // 16-byte chunks per thread (4 per row per stage)
    v4i rw[WCH], rqh[WCH];
    v4i rx[2];
    v4i rsd, rda, rsq;
    auto gload = [&](int kb0) {
        const int sbk = kb0 >> 3;
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int r = ch >> 2, p = ch & 3;
            rw[j] = ld16(codes + (size_t)r * rowb + (size_t)kb0 * 16 + p * 16);
            if constexpr (K5) rqh[j] = ld16(side + ((size_t)r * nsb + sbk) * SIDE + 16 + 16 * (p & 1));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int c = ch >> 3, p = ch & 7;
            rx[j] = ld16(A.ain.q + (size_t)s_row[c] * K + (size_t)kb0 * QK + p * 16);
        }
        if (tid < MF_NT) {
            rsd = ld16(side + ((size_t)tid * nsb + sbk) * SIDE);
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
            rda = *reinterpret_cast<const v4i*>(A.ain.ds + (size_t)s_row[c] * nb + kb0);
            rsq = *reinterpret_cast<const v4i*>(A.ain.sq + (size_t)s_row[c] * nb + kb0);
        }
    };
    auto lstore = [&](int buf, int kb0) {
        const int half = (kb0 >> 2) & 1;                  // which half of the super-block
        char* st = smem + buf * STAGE;
        int8_t* sw = reinterpret_cast<int8_t*>(st);
        int8_t* sx = reinterpret_cast<int8_t*>(st + WBYTES);
        float* sdw = reinterpret_cast<float*>(st + WBYTES + XBYTES);
        float* sda = sdw + MF_KB * MS_SWR;
        float* smw = sda + MF_KB * MS_SAR;
        float* sas = smw + MF_KB * MF_NT;
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int r = ch >> 2, p = ch & 3;
            const int q0 = 2 * (p >> 1), h = p & 1;       // stage blocks q0 (low), q0 + 1 (high)
            const int gb = 4 * half + q0;                 // the low nibbles' sub-block
            v4i lo, hi;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t x = (uint32_t)rw[j][d];
                uint32_t l = x & 0x0F0F0F0Fu, hh = (x >> 4) & 0x0F0F0F0Fu;
                if constexpr (K5) {
                    const uint32_t qb = (uint32_t)rqh[j][d];
                    l |= ((qb >> gb) & 0x01010101u) << 4;
                    hh |= ((qb >> (gb + 1)) & 0x01010101u) << 4;
                }
                lo[d] = (int)l;
                hi[d] = (int)hh;
            }
            *reinterpret_cast<v4i*>(sw + r * MS_ROWB + q0 * QK + 16 * h) = lo;
            *reinterpret_cast<v4i*>(sw + r * MS_ROWB + (q0 + 1) * QK + 16 * h) = hi;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = tid + j * MF_THREADS;
            const int c = ch >> 3, p = ch & 7;
            *reinterpret_cast<v4i*>(sx + c * MS_ROWB + p * 16) = rx[j];
        }
        if (tid < MF_NT) {
            const float dd = h2f((uint32_t)rsd.x), dmin = h2f((uint32_t)rsd.x >> 16);
#pragma unroll
            for (int q = 0; q < MF_KB; ++q) {
                int sc, mn;
                k4_scale_min(rsd, 4 * half + q, sc, mn);
                sdw[q * MS_SWR + tid] = dd * (float)sc;
                smw[q * MF_NT + tid] = dmin * (float)mn;
            }
        } else if (tid < MF_NT + MF_MT) {
            const int c = tid - MF_NT;
#pragma unroll
            for (int q = 0; q < MF_KB; ++q) {
                const float da = h2f((uint32_t)rda[q]);
                sda[q * MS_SAR + c] = da;
                sas[q * MF_MT + c] = da * (float)rsq[q];
            }
        }
    };

    MfWave w{wave & 1, wave >> 1, lane >> 5, lane & 31};
    const int o_w0 = w.half ? MF_NT + w.l32 : w.wr * 64 + w.l32;
    const int o_w1 = w.half ? MF_NT + w.l32 : w.wr * 64 + 32 + w.l32;
    const int o_a = w.half ? MF_MT + w.l32 : w.wc * 32 + w.l32;
    const bool busy = w.wc * 32 < t.ncol;
    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.0f;

    const int stages = nb / MF_KB;
    auto compute = [&](int buf, int s) {
        if (!busy) return;
        const char* st = smem + buf * STAGE;
        const int8_t* sw = reinterpret_cast<const int8_t*>(st);
        const int8_t* sx = reinterpret_cast<const int8_t*>(st + WBYTES);
        const float* sdw = reinterpret_cast<const float*>(st + WBYTES + XBYTES);
        const float* sda = sdw + MF_KB * MS_SWR;
        const float* smw = sda + MF_KB * MS_SAR;
        const float* sas = smw + MF_KB * MF_NT;
        auto frag = [&](int kb, v4i& a0, v4i& a1, v4i& bx) {
            a0 = *reinterpret_cast<const v4i*>(sw + (w.wr * 64 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
            a1 = *reinterpret_cast<const v4i*>(sw + (w.wr * 64 + 32 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
            bx = *reinterpret_cast<const v4i*>(sx + (w.wc * 32 + w.l32) * MS_ROWB + kb * QK + w.half * 16);
        };
        auto sfrag = [&](int kb, float& d0, float& d1, float& dc) {
            d0 = sdw[kb * MS_SWR + o_w0];
            d1 = sdw[kb * MS_SWR + o_w1];
            dc = sda[kb * MS_SAR + o_a];
        };
        mf_stage<SWIGLU, TAP, float>(A, t, w, s, s_orow, frag, sfrag, acc0, acc1);
        // min terms: blocks (0, 1) then (2, 3), one per k slot (lane half)
        v16f p0 = v16f{}, p1 = v16f{};
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const int q = 2 * pr + w.half;
            const float m0 = smw[q * MF_NT + w.wr * 64 + w.l32];
            const float m1 = smw[q * MF_NT + w.wr * 64 + 32 + w.l32];
            const float sv = sas[q * MF_MT + w.wc * 32 + w.l32];
            p0 = __builtin_amdgcn_mfma_f32_32x32x2f32(m0, sv, p0, 0, 0, 0);
            p1 = __builtin_amdgcn_mfma_f32_32x32x2f32(m1, sv, p1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc0[i] -= p0[i];
            acc1[i] -= p1[i];
        }
    };
    gload(0);
    lstore(0, 0);
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s + 1 < stages; ++s) {
        gload((s + 1) * MF_KB);
        compute(s & 1, s);
        lstore((s + 1) & 1, (s + 1) * MF_KB);
        __syncthreads();
    }
    compute((stages - 1) & 1, stages - 1);
    mf_epilogue<SWIGLU, TAP>(A, t, w, s_orow, acc0, acc1);
}

// ---------------------------------------------------------------------------
bool mfma_config_ok(int rows, int K) { return rows % MF_NT == 0 && K % (MF_KB * QK) == 0; }

template <bool SWIGLU>
static hipError_t mfma_fmt(int fmt, const MfArgs& a, bool tap, hipStream_t st,
                           const KEvents& ev = KEvents{}) {
    if (!mfma_config_ok(a.rows, a.K)) return hipErrorInvalidConfiguration;
    long blocks = (long)(a.rows / MF_NT) * a.max_tiles;
    blocks = (blocks + 7) & ~7L;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(MF_THREADS);
    if (fmt == MOE_FMT_Q4_0) {
        if (tap)
            launch_k(k_mfma_q4<SWIGLU, true, MOE_FMT_Q4_0>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_q4<SWIGLU, false, MOE_FMT_Q4_0>, grid, block, 0, st, ev, a);
    } else if (fmt == MOE_FMT_Q5_1) {
        if (tap)
            launch_k(k_mfma_q4<SWIGLU, true, MOE_FMT_Q5_1>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_q4<SWIGLU, false, MOE_FMT_Q5_1>, grid, block, 0, st, ev, a);
    } else if (fmt == MOE_FMT_Q3_K) {
        if (tap)
            launch_k(k_mfma_q4<SWIGLU, true, MOE_FMT_Q3_K>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_q4<SWIGLU, false, MOE_FMT_Q3_K>, grid, block, 0, st, ev, a);
    } else if (fmt == MOE_FMT_Q4_K) {
        if (tap)
            launch_k(k_mfma_kq<SWIGLU, true, MOE_FMT_Q4_K>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_kq<SWIGLU, false, MOE_FMT_Q4_K>, grid, block, 0, st, ev, a);
    } else if (fmt == MOE_FMT_Q5_K) {
        if (tap)
            launch_k(k_mfma_kq<SWIGLU, true, MOE_FMT_Q5_K>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_kq<SWIGLU, false, MOE_FMT_Q5_K>, grid, block, 0, st, ev, a);
    } else if (fmt == MOE_FMT_NVFP4) {
        if (tap)
            launch_k(k_mfma_nv4<SWIGLU, true>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_nv4<SWIGLU, false>, grid, block, 0, st, ev, a);
    } else if (fmt != MOE_FMT_Q8_0) {
        return hipErrorInvalidValue;   // (no matrix-core path for this format)
    } else {
        if (tap)
            launch_k(k_mfma_dma<SWIGLU, true>, grid, block, 0, st, ev, a);
        else
            launch_k(k_mfma_dma<SWIGLU, false>, grid, block, 0, st, ev, a);
    }
    return hipGetLastError();
}

hipError_t launch_gate_up_mfma(const Dims& m, int T, ExpertSrc experts, ActPtr ain,
                               const Buckets& b, const int32_t* tile_map, ActPtr hq,
                               const Taps& taps, hipStream_t st, const KEvents& ev) {
    MfArgs a{};
    a.base = experts.base;
    a.etab = experts.table;
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
    a.ts_off = m.ts_off;
    return mfma_fmt<true>(m.fmt, a, taps.h || taps.isum_gu, st, ev);
}

hipError_t launch_down_mfma(const Dims& m, int T, ExpertSrc experts, ActPtr hq,
                            const Buckets& b, const int32_t* tile_map, float* y, const Taps& taps,
                            hipStream_t st) {
    MfArgs a{};
    a.base = experts.base;
    a.etab = experts.table;
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
    a.ts_off = m.ts_off;
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
