// Matrix-vector kernels of libmoe: the decode path of the grouped expert FFN and
// the latent dense projections.
//
// Prior art (Strata PR 24, SYCL port commits): the grouped expert kernels split
// each format into a once-per-weight part and a per-token part because a
// verify window routes one expert for up to 6 tokens, and a handful of lanes per
// row beat a full warp on short rows; 16-byte loads streamed faster than
// 4-byte ones.  Here, for gfx950:
//   * a lane group of LPR lanes owns one weight row; lane sl of the group loads
//     16-byte chunks c = j*LPR + sl (j < CPL), so a wave's loads are contiguous;
//   * the weights are loaded once into registers and reused for every token of
//     the expert's bucket; the Q8_1 activation chunks are read per token;
//   * each chunk is 16 int8 codes (half a Q8_0 block) or one Q4_0 block, dotted
//     with packed int8 dot products; the row is reduced across the group.
// The per-block integer sums are exact; the scale products and the row sums are
// fp32.
#include <algorithm>

#include "kernels.h"

namespace moe {

template <int FMT>
struct Fmt {
    static constexpr int QB = FMT == MOE_FMT_Q4_0 ? 16 : 32;  // code bytes per block
    static constexpr int CPB = FMT == MOE_FMT_Q4_0 ? 1 : 2;   // 16-byte chunks per block
};

// Integer sum of chunk c (of a weight row held in wq) against activation row
// `arow` (K int8 codes, sums asq).  Q8_0: half a block; Q4_0: a whole block.
template <int FMT>
__device__ __forceinline__ int chunk_isum(const v4i& wq, const int8_t* arow, const int32_t* asq,
                                          int c) {
    if constexpr (FMT == MOE_FMT_Q4_0) {
        v4i lo = ld16(arow + c * 32);
        v4i hi = ld16(arow + c * 32 + 16);
        return dot_q4(wq, lo, hi) - 8 * asq[c];
    } else {
        v4i a = ld16(arow + c * 16);
        return dot16(wq, a);
    }
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU + Q8_1 requantisation.  Workgroup = (slot, fb): the 64-row
// slab of gate rows fb*32.. and up rows fb*32.. of the slot's expert, for every
// token routed to it.  Output: hq rows a = t*k + j, 32 codes of block fb.
struct GUArgs {
    const uint8_t* experts;
    size_t eb, gu_scales_off;
    int K, F, k, T;
    ActPtr ain;
    Buckets b;
    ActPtr hq;
    Taps taps;
};

constexpr int GU_TCH = 32;  // tokens buffered in LDS before the SwiGLU epilogue

template <int FMT, int LPR, int CPL>
__device__ __forceinline__ void load_row_chunks(const uint8_t* row, const uint16_t* rscl, int sl,
                                                int NCH, v4i (&wq)[CPL], float (&wsc)[CPL]) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = j * LPR + sl;
        if (c < NCH) {
            wq[j] = ld16(row + (size_t)c * 16);
            wsc[j] = h2f(rscl[c / F::CPB]);
        } else {
            wq[j] = v4i{0, 0, 0, 0};
            wsc[j] = 0.0f;
        }
    }
}

template <int FMT, int LPR, int CPL, int NW, bool TAP>
__global__ __launch_bounds__(NW * 64) void k_gate_up_mv(GUArgs A) {
    using F = Fmt<FMT>;
    constexpr int RPW = 64 / LPR;
    constexpr int PASSES = 64 / (NW * RPW);
    static_assert(PASSES >= 1 && PASSES * NW * RPW == 64, "64 rows per workgroup");
    __shared__ float gu_s[GU_TCH][64];

    const int FB = A.F / QK;
    const int slot = blockIdx.x / FB, fb = blockIdx.x - slot * FB;
    if (slot >= (int)A.b.ctrl[CW_N_ACTIVE]) return;
    const int e = A.b.active[slot];
    const int cnt = A.b.counts[e];
    const int32_t* lst = A.b.lists + (size_t)e * A.T;
    const int nb = A.K / QK;
    const int NCH = nb * F::CPB;
    const size_t rowb = (size_t)nb * F::QB;
    const uint8_t* ebase = A.experts + (size_t)e * A.eb;
    const uint8_t* codes = ebase + (size_t)fb * 64 * rowb;
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(ebase + A.gu_scales_off) + (size_t)fb * 64 * nb;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sl = lane % LPR, rg = lane / LPR;

    for (int i0 = 0; i0 < cnt; i0 += GU_TCH) {
        const int n = min(GU_TCH, cnt - i0);
        // one pass = one row per lane group; the next pass's row is loaded
        // while this one is dotted with the tokens
        v4i wq[CPL];
        float wsc[CPL];
        {
            const int r = wave * RPW + rg;
            load_row_chunks<FMT, LPR, CPL>(codes + r * rowb, scl + (size_t)r * nb, sl, NCH, wq, wsc);
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = (p * NW + wave) * RPW + rg;
            v4i wn[CPL];
            float wsn[CPL];
            if (p + 1 < PASSES) {
                const int rn = ((p + 1) * NW + wave) * RPW + rg;
                load_row_chunks<FMT, LPR, CPL>(codes + rn * rowb, scl + (size_t)rn * nb, sl, NCH, wn, wsn);
            }
#pragma unroll 1
            for (int i = 0; i < n; ++i) {
                const int a = lst[i0 + i];
                const int t = a / A.k;
                const int8_t* arow = A.ain.q + (size_t)t * A.K;
                const uint32_t* ads = A.ain.ds + (size_t)t * nb;
                const int32_t* asq = A.ain.sq + (size_t)t * nb;
                const bool tap = TAP && A.taps.isum_gu && t < A.taps.tap_tokens;
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = j * LPR + sl;
                    const bool valid = c < NCH;
                    const int blk = c / F::CPB;
                    const int is = valid ? chunk_isum<FMT>(wq[j], arow, asq, c) : 0;
                    acc += (float)is * (wsc[j] * (valid ? h2f(ads[blk]) : 0.0f));
                    if constexpr (TAP) {
                        if (tap) {
                            int full = is;
                            if constexpr (F::CPB == 2) full += __shfl_xor(is, 1, 64);
                            if (valid && (F::CPB == 1 || (sl & 1) == 0)) {
                                const int row = r < 32 ? fb * 32 + r : A.F + fb * 32 + (r - 32);
                                A.taps.isum_gu[((size_t)a * 2 * A.F + row) * nb + blk] = full;
                            }
                        }
                    }
                }
                const float v = group_sum<LPR>(acc);
                if (sl == 0) gu_s[i][r] = v;
            }
            if (p + 1 < PASSES) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    wq[j] = wn[j];
                    wsc[j] = wsn[j];
                }
            }
        }
        __syncthreads();
        // SwiGLU and Q8_1: one 32-lane group per token, lane = output f
        for (int ii = threadIdx.x / 32; ii < n; ii += NW * 2) {
            const int f = threadIdx.x & 31;
            const float g = gu_s[ii][f], u = gu_s[ii][32 + f];
            const float h = g / (1.0f + expf(-g)) * u;
            const int a = lst[i0 + ii];
            const size_t hb = (size_t)a * FB + fb;
            quant_q8_1_32(h, f, A.hq.q + (size_t)a * A.F + fb * 32, A.hq.ds + hb, A.hq.sq + hb);
            if constexpr (TAP) {
                if (A.taps.h) A.taps.h[(size_t)a * A.F + fb * 32 + f] = h;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Rows kernel: out[s][r] = W_g[r] . act[s] for the rows of a block matrix and a
// list of activation rows.  Expert mode (b.ctrl != nullptr): group = slot, W_g =
// the down matrix of expert active[slot], rows of act/out = the expert's
// assignments.  Dense mode: one matrix, act/out rows 0..T-1.
struct RowsArgs {
    const uint8_t* base;
    size_t group_stride, codes_off, scales_off;
    int rows, K, T;
    Buckets b;                 // b.ctrl == nullptr: dense mode
    ActPtr ain;
    float* out;                // [act row][rows]
    int tap_div;               // token of act row s = s / tap_div
    int32_t* isum_tap;         // [act row][rows][K/32]
    int tap_tokens;
};

template <int FMT, int LPR, int CPL, int NW, bool TAP>
__global__ __launch_bounds__(NW * 64) void k_rows_mv(RowsArgs A) {
    using F = Fmt<FMT>;
    constexpr int RPW = 64 / LPR;
    constexpr int RT = NW * RPW;
    const int NRT = A.rows / RT;
    const int g = blockIdx.x / NRT, rt = blockIdx.x - g * NRT;
    const uint8_t* mat;
    const int32_t* lst = nullptr;
    int cnt;
    if (A.b.ctrl) {
        if (g >= (int)A.b.ctrl[CW_N_ACTIVE]) return;
        const int e = A.b.active[g];
        mat = A.base + (size_t)e * A.group_stride;
        cnt = A.b.counts[e];
        lst = A.b.lists + (size_t)e * A.T;
    } else {
        mat = A.base;
        cnt = A.T;
    }
    const int nb = A.K / QK;
    const int NCH = nb * F::CPB;
    const size_t rowb = (size_t)nb * F::QB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sl = lane % LPR, rg = lane / LPR;
    const int r = rt * RT + wave * RPW + rg;
    const uint8_t* codes = mat + A.codes_off + (size_t)r * rowb;
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(mat + A.scales_off) + (size_t)r * nb;

    v4i wq[CPL];
    float wsc[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = j * LPR + sl;
        if (c < NCH) {
            wq[j] = ld16(codes + (size_t)c * 16);
            wsc[j] = h2f(scl[c / F::CPB]);
        } else {
            wq[j] = v4i{0, 0, 0, 0};
            wsc[j] = 0.0f;
        }
    }
    for (int i = 0; i < cnt; ++i) {
        const int s = lst ? lst[i] : i;
        const int8_t* arow = A.ain.q + (size_t)s * A.K;
        const uint32_t* ads = A.ain.ds + (size_t)s * nb;
        const int32_t* asq = A.ain.sq + (size_t)s * nb;
        const bool tap = TAP && A.isum_tap && s / A.tap_div < A.tap_tokens;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = j * LPR + sl;
            const bool valid = c < NCH;
            const int blk = c / F::CPB;
            const int is = valid ? chunk_isum<FMT>(wq[j], arow, asq, c) : 0;
            acc += (float)is * (wsc[j] * (valid ? h2f(ads[blk]) : 0.0f));
            if constexpr (TAP) {
                if (tap) {
                    int full = is;
                    if constexpr (F::CPB == 2) full += __shfl_xor(is, 1, 64);
                    if (valid && (F::CPB == 1 || (sl & 1) == 0))
                        A.isum_tap[((size_t)s * A.rows + r) * nb + blk] = full;
                }
            }
        }
        const float v = group_sum<LPR>(acc);
        if (sl == 0) A.out[(size_t)s * A.rows + r] = v;
    }
}

// ---------------------------------------------------------------------------
// Down projection with the combine fused, one workgroup per (token, row tile):
// out[t][r] = sum_j w[t][j] * (W_down[e_j][r] . hq[t*k+j]), rank order.
struct DownTokArgs {
    const uint8_t* experts;
    size_t eb, dn_off, dn_scales_off;
    int F, Kout, k;
    ActPtr hq;
    Buckets b;
    float* out;
    Taps taps;
};

template <int FMT, int LPR, int CPL, int NW, bool TAP>
__global__ __launch_bounds__(NW * 64) void k_down_tok_mv(DownTokArgs A) {
    using F = Fmt<FMT>;
    constexpr int RPW = 64 / LPR;
    constexpr int RT = NW * RPW;
    const int NRT = A.Kout / RT;
    const int t = blockIdx.x / NRT, rt = blockIdx.x - t * NRT;
    const int nb = A.F / QK;
    const int NCH = nb * F::CPB;
    const size_t rowb = (size_t)nb * F::QB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sl = lane % LPR, rg = lane / LPR;
    const int r = rt * RT + wave * RPW + rg;
    const bool tap = TAP && t < A.taps.tap_tokens;
    float o = 0.0f;
    for (int j = 0; j < A.k; ++j) {
        const int a = t * A.k + j;
        const int e = A.b.ids[a];
        const float wj = A.b.wts[a];
        const uint8_t* mat = A.experts + (size_t)e * A.eb + A.dn_off;
        const uint8_t* codes = mat + (size_t)r * rowb;
        const uint16_t* scl = reinterpret_cast<const uint16_t*>(mat + A.dn_scales_off) + (size_t)r * nb;
        const int8_t* arow = A.hq.q + (size_t)a * A.F;
        const uint32_t* ads = A.hq.ds + (size_t)a * nb;
        const int32_t* asq = A.hq.sq + (size_t)a * nb;
        v4i wq[CPL];
        float wsc[CPL];
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) {
            const int c = jj * LPR + sl;
            if (c < NCH) {
                wq[jj] = ld16(codes + (size_t)c * 16);
                wsc[jj] = h2f(scl[c / F::CPB]);
            } else {
                wq[jj] = v4i{0, 0, 0, 0};
                wsc[jj] = 0.0f;
            }
        }
        float acc = 0.0f;
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) {
            const int c = jj * LPR + sl;
            const bool valid = c < NCH;
            const int blk = c / F::CPB;
            const int is = valid ? chunk_isum<FMT>(wq[jj], arow, asq, c) : 0;
            acc += (float)is * (wsc[jj] * (valid ? h2f(ads[blk]) : 0.0f));
            if constexpr (TAP) {
                if (tap && A.taps.isum_dn) {
                    int full = is;
                    if constexpr (F::CPB == 2) full += __shfl_xor(is, 1, 64);
                    if (valid && (F::CPB == 1 || (sl & 1) == 0))
                        A.taps.isum_dn[((size_t)a * A.Kout + r) * nb + blk] = full;
                }
            }
        }
        const float y = group_sum<LPR>(acc);
        o = fmaf(wj, y, o);
        if constexpr (TAP) {
            if (sl == 0 && A.taps.y) A.taps.y[(size_t)a * A.Kout + r] = y;
        }
    }
    if (sl == 0) A.out[(size_t)t * A.Kout + r] = o;
}

// ---------------------------------------------------------------------------
// configuration choice and dispatch

// lanes per row and 16-byte chunks per lane for a row of nch chunks, with at
// most max_regs chunks held per lane when `passes` rows share a lane group.
static bool pick(int nch, int& lpr, int& cpl) {
    for (int c = 8; c >= 1; --c)
        for (int l = 8; l <= 64; l *= 2)
            if (l * c == nch) { lpr = l; cpl = c; return true; }
    if (nch <= 512) { lpr = 64; cpl = (nch + 63) / 64; return true; }
    return false;
}

#define MOE_LPR_CPL_SWITCH(LPR_, CPL_, CALL)                                      \
    switch (LPR_ * 16 + CPL_) {                                                    \
        case 8 * 16 + 1: { constexpr int L = 8, C = 1; CALL; break; }          \
        case 8 * 16 + 2: { constexpr int L = 8, C = 2; CALL; break; }          \
        case 8 * 16 + 3: { constexpr int L = 8, C = 3; CALL; break; }          \
        case 8 * 16 + 4: { constexpr int L = 8, C = 4; CALL; break; }          \
        case 8 * 16 + 5: { constexpr int L = 8, C = 5; CALL; break; }          \
        case 8 * 16 + 6: { constexpr int L = 8, C = 6; CALL; break; }          \
        case 8 * 16 + 7: { constexpr int L = 8, C = 7; CALL; break; }          \
        case 8 * 16 + 8: { constexpr int L = 8, C = 8; CALL; break; }          \
        case 16 * 16 + 1: { constexpr int L = 16, C = 1; CALL; break; }        \
        case 16 * 16 + 2: { constexpr int L = 16, C = 2; CALL; break; }        \
        case 16 * 16 + 3: { constexpr int L = 16, C = 3; CALL; break; }        \
        case 16 * 16 + 4: { constexpr int L = 16, C = 4; CALL; break; }        \
        case 16 * 16 + 5: { constexpr int L = 16, C = 5; CALL; break; }        \
        case 16 * 16 + 6: { constexpr int L = 16, C = 6; CALL; break; }        \
        case 16 * 16 + 7: { constexpr int L = 16, C = 7; CALL; break; }        \
        case 16 * 16 + 8: { constexpr int L = 16, C = 8; CALL; break; }        \
        case 32 * 16 + 1: { constexpr int L = 32, C = 1; CALL; break; }        \
        case 32 * 16 + 2: { constexpr int L = 32, C = 2; CALL; break; }        \
        case 32 * 16 + 3: { constexpr int L = 32, C = 3; CALL; break; }        \
        case 32 * 16 + 4: { constexpr int L = 32, C = 4; CALL; break; }        \
        case 32 * 16 + 5: { constexpr int L = 32, C = 5; CALL; break; }        \
        case 32 * 16 + 6: { constexpr int L = 32, C = 6; CALL; break; }        \
        case 32 * 16 + 7: { constexpr int L = 32, C = 7; CALL; break; }        \
        case 32 * 16 + 8: { constexpr int L = 32, C = 8; CALL; break; }        \
        case 64 * 16 + 1: { constexpr int L = 64, C = 1; CALL; break; }        \
        case 64 * 16 + 2: { constexpr int L = 64, C = 2; CALL; break; }        \
        case 64 * 16 + 3: { constexpr int L = 64, C = 3; CALL; break; }        \
        case 64 * 16 + 4: { constexpr int L = 64, C = 4; CALL; break; }        \
        case 64 * 16 + 5: { constexpr int L = 64, C = 5; CALL; break; }        \
        case 64 * 16 + 6: { constexpr int L = 64, C = 6; CALL; break; }        \
        case 64 * 16 + 7: { constexpr int L = 64, C = 7; CALL; break; }        \
        case 64 * 16 + 8: { constexpr int L = 64, C = 8; CALL; break; }        \
        default: return hipErrorInvalidConfiguration;                              \
    }

// Chunks per row of a Kin-wide row, and the (lanes, chunks) pair the kernels use.
static int nchunks(int K, int fmt) { return fmt == MOE_FMT_Q4_0 ? K / 32 : K / 16; }

// gate/up: one pass of rows in registers plus the prefetched next pass, so at
// most 5 chunks per lane when there is more than one pass.
constexpr int GU_NW = 8;   // waves per gate/up workgroup

static bool pick_gu(int nch, int& lpr, int& cpl) {
    for (int l = 64; l >= 8; l /= 2)
        for (int c = 8; c >= 1; --c) {
            int passes = 64 / (GU_NW * (64 / l));
            if (l * c == nch && (passes == 1 || c <= 5)) { lpr = l; cpl = c; return true; }
        }
    return false;
}

bool mv_config_ok(int K, int fmt, bool gate_up) {
    int l, c;
    if (gate_up ? !pick_gu(nchunks(K, fmt), l, c) : !pick(nchunks(K, fmt), l, c)) return false;
    return c >= 1 && c <= 8 && (l == 8 || l == 16 || l == 32 || l == 64);
}

template <int FMT, bool TAP>
static hipError_t gate_up_fmt(int lpr, int cpl, dim3 grid, const GUArgs& a, hipStream_t st) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        constexpr int NW = GU_NW;
        constexpr int PASSES = 64 / (NW * (64 / L));
        if constexpr (PASSES == 1 || C <= 5)
            hipLaunchKernelGGL((k_gate_up_mv<FMT, L, C, NW, TAP>), grid, dim3(NW * 64), 0, st, a);
        else
            return hipErrorInvalidConfiguration;
    }));
    return hipGetLastError();
}

hipError_t launch_gate_up_mv(const Dims& m, int T, const uint8_t* experts, ActPtr ain,
                             const Buckets& b, ActPtr hq, const Taps& taps, hipStream_t st) {
    int lpr, cpl;
    if (!pick_gu(nchunks(m.kin, m.fmt), lpr, cpl)) return hipErrorInvalidConfiguration;
    GUArgs a;
    a.experts = experts;
    a.eb = m.expert_bytes;
    a.gu_scales_off = m.gu.scales_off;
    a.K = m.kin; a.F = m.F; a.k = m.k; a.T = T;
    a.ain = ain; a.b = b; a.hq = hq; a.taps = taps;
    int slots = std::min(m.E, T * m.k);
    dim3 grid(slots * (m.F / QK));
    bool tap = taps.h || taps.isum_gu;
    if (m.fmt == MOE_FMT_Q4_0)
        return tap ? gate_up_fmt<MOE_FMT_Q4_0, true>(lpr, cpl, grid, a, st)
                   : gate_up_fmt<MOE_FMT_Q4_0, false>(lpr, cpl, grid, a, st);
    return tap ? gate_up_fmt<MOE_FMT_Q8_0, true>(lpr, cpl, grid, a, st)
               : gate_up_fmt<MOE_FMT_Q8_0, false>(lpr, cpl, grid, a, st);
}

constexpr int ROWS_NW = 8;

template <int FMT, bool TAP>
static hipError_t rows_fmt(int lpr, int cpl, int ngroups, const RowsArgs& a, hipStream_t st) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        constexpr int RT = ROWS_NW * (64 / L);
        dim3 grid(ngroups * (a.rows / RT));
        hipLaunchKernelGGL((k_rows_mv<FMT, L, C, ROWS_NW, TAP>), grid, dim3(ROWS_NW * 64), 0, st, a);
    }));
    return hipGetLastError();
}

static hipError_t rows_dispatch(int fmt, int ngroups, const RowsArgs& a, hipStream_t st) {
    int lpr, cpl;
    if (!pick(nchunks(a.K, fmt), lpr, cpl)) return hipErrorInvalidConfiguration;
    if (a.rows % (ROWS_NW * (64 / lpr))) return hipErrorInvalidConfiguration;
    bool tap = a.isum_tap != nullptr;
    if (fmt == MOE_FMT_Q4_0)
        return tap ? rows_fmt<MOE_FMT_Q4_0, true>(lpr, cpl, ngroups, a, st)
                   : rows_fmt<MOE_FMT_Q4_0, false>(lpr, cpl, ngroups, a, st);
    return tap ? rows_fmt<MOE_FMT_Q8_0, true>(lpr, cpl, ngroups, a, st)
               : rows_fmt<MOE_FMT_Q8_0, false>(lpr, cpl, ngroups, a, st);
}

hipError_t launch_down_slot_mv(const Dims& m, int T, const uint8_t* experts, ActPtr hq,
                               const Buckets& b, float* y, const Taps& taps, hipStream_t st) {
    RowsArgs a;
    a.base = experts;
    a.group_stride = m.expert_bytes;
    a.codes_off = m.dn_off + m.dn.codes_off;
    a.scales_off = m.dn_off + m.dn.scales_off;
    a.rows = m.kout; a.K = m.F; a.T = T;
    a.b = b; a.ain = hq; a.out = y;
    a.tap_div = m.k; a.isum_tap = taps.isum_dn; a.tap_tokens = taps.tap_tokens;
    return rows_dispatch(m.fmt, std::min(m.E, T * m.k), a, st);
}

hipError_t launch_dense_mv(const MatLayout& W, const uint8_t* base, int T, ActPtr ain, float* out,
                           int32_t* isum_tap, int tap_tokens, hipStream_t st) {
    RowsArgs a;
    a.base = base;
    a.group_stride = 0;
    a.codes_off = W.codes_off;
    a.scales_off = W.scales_off;
    a.rows = W.rows; a.K = W.nblk * QK; a.T = T;
    a.b = Buckets{};
    a.ain = ain; a.out = out;
    a.tap_div = 1; a.isum_tap = isum_tap; a.tap_tokens = tap_tokens;
    return rows_dispatch(W.fmt, 1, a, st);
}

constexpr int DT_NW = 8;

template <int FMT, bool TAP>
static hipError_t down_tok_fmt(int lpr, int cpl, int T, const DownTokArgs& a, hipStream_t st) {
    MOE_LPR_CPL_SWITCH(lpr, cpl, ({
        constexpr int RT = DT_NW * (64 / L);
        if (a.Kout % RT) return hipErrorInvalidConfiguration;
        dim3 grid(T * (a.Kout / RT));
        hipLaunchKernelGGL((k_down_tok_mv<FMT, L, C, DT_NW, TAP>), grid, dim3(DT_NW * 64), 0, st, a);
    }));
    return hipGetLastError();
}

hipError_t launch_down_tok_mv(const Dims& m, int T, const uint8_t* experts, ActPtr hq,
                              const Buckets& b, float* out, const Taps& taps, hipStream_t st) {
    int lpr, cpl;
    if (!pick(nchunks(m.F, m.fmt), lpr, cpl)) return hipErrorInvalidConfiguration;
    DownTokArgs a;
    a.experts = experts;
    a.eb = m.expert_bytes;
    a.dn_off = m.dn_off + m.dn.codes_off;
    a.dn_scales_off = m.dn.scales_off - m.dn.codes_off;
    a.F = m.F; a.Kout = m.kout; a.k = m.k;
    a.hq = hq; a.b = b; a.out = out; a.taps = taps;
    bool tap = taps.isum_dn || taps.y;
    if (m.fmt == MOE_FMT_Q4_0)
        return tap ? down_tok_fmt<MOE_FMT_Q4_0, true>(lpr, cpl, T, a, st)
                   : down_tok_fmt<MOE_FMT_Q4_0, false>(lpr, cpl, T, a, st);
    return tap ? down_tok_fmt<MOE_FMT_Q8_0, true>(lpr, cpl, T, a, st)
               : down_tok_fmt<MOE_FMT_Q8_0, false>(lpr, cpl, T, a, st);
}

}  // namespace moe
