// Router, activation quantiser, token-to-expert bucketing, combine and tap
// kernels of libmoe.
//
// Router (Strata PR 24, SYCL port commits: top-k over the experts per token;
// edge0-strata README: expert group labels): logits accumulate in fp64 so that
// the chosen experts do not depend on summation order except at genuine
// near-ties; top-k with ties to the lower id; softmax over the chosen logits.
// Bucketing (same PR: "per-layer grouping" of prompt tokens by expert): every
// expert gets the list of its assignments a = t*k + j in token order, and the
// experts with tokens are compacted into slots in id order.
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Q8_1 quantisation of fp32 rows [rows][K]: one 32-lane group per block.
__global__ __launch_bounds__(256) void k_quant_rows(const float* __restrict__ x, int rows, int K,
                                                    ActPtr out) {
    const int nb = K / QK;
    const long blk = (long)blockIdx.x * 8 + threadIdx.x / 32;
    if (blk >= (long)rows * nb) return;               // whole 32-lane groups exit together
    const int l = threadIdx.x % 32;
    const long r = blk / nb, b = blk % nb;
    float v = x[r * K + b * QK + l];
    quant_q8_1_32(v, l, out.q + r * K + b * QK, out.ds + r * nb + b, out.sq + r * nb + b);
}

// ---------------------------------------------------------------------------
// Router logits, partial over K slices: part[s][t][e] = sum_{i in slice s} x[t,i] W[e,i],
// plus the Q8_1 quantisation of x in the trailing workgroups of the same grid.
// A logits workgroup = 4 waves = 4 experts for TT tokens of one K slice.
// Products of two floats are exact in fp64; only the additions round.
template <int TT>
__global__ __launch_bounds__(256) void k_route_logits(const float* __restrict__ x,
                                                      const float* __restrict__ W, int T, int H,
                                                      int E, int S, double* __restrict__ part,
                                                      int n_logit_wg, ActPtr xq) {
    if ((int)blockIdx.x >= n_logit_wg) {
        // x -> Q8_1, one 32-lane group per block
        const int nb = H / QK;
        const long blk = (long)(blockIdx.x - n_logit_wg) * 8 + threadIdx.x / 32;
        if (blk >= (long)T * nb) return;
        const int l = threadIdx.x % 32;
        const long r = blk / nb, b = blk % nb;
        quant_q8_1_32(x[r * H + b * QK + l], l, xq.q + r * H + b * QK, xq.ds + r * nb + b,
                      xq.sq + r * nb + b);
        return;
    }
    const int ge = (E + 3) / 4;
    const int bx = blockIdx.x % ge, s = (blockIdx.x / ge) % S, tz = blockIdx.x / (ge * S);
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int e = bx * 4 + wave;
    const int t0 = tz * TT;
    if (e >= E) return;
    const int nt = min(TT, T - t0);
    const int slice = H / S, k0 = s * slice;
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
    const float* wrow = W + (size_t)e * H;
    for (int i = k0 + lane * 4; i < k0 + slice; i += 256) {
        const float4 w = *reinterpret_cast<const float4*>(wrow + i);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t < nt) {
                const float4 xv = *reinterpret_cast<const float4*>(x + (size_t)(t0 + t) * H + i);
                acc[t] = fma((double)xv.x, (double)w.x, acc[t]);
                acc[t] = fma((double)xv.y, (double)w.y, acc[t]);
                acc[t] = fma((double)xv.z, (double)w.z, acc[t]);
                acc[t] = fma((double)xv.w, (double)w.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (t < nt) {
            const double v = wave_sum_d(acc[t]);
            if (lane == 0) part[((size_t)s * T + t0 + t) * E + e] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Router logits on the fp64 matrix cores, partial over K slices:
// part[s][t][e] = sum_{i in slice s} x[t,i] W[e,i].  x and W_r are fp32, so
// their products are exact in fp64 and only the accumulation rounds.
// One v_mfma_f64_16x16x4f64 takes a 16-token x 4 and a 4 x 16-expert operand,
// one double per lane: lane l holds row l%16 at k-slot l/16, and the 16x16
// fp64 result sits as rows l/16 + 4*v, column l%16 (v < 4).  Each lane loads
// four consecutive floats of its row per 16-wide K chunk and feeds them to
// four MFMAs as k = 4*(l/16) + j, so a chunk is covered once.
// A workgroup is four waves on a (16*MT*WM tokens) x (16*NT*WN experts) tile;
// with WK > 1 the waves split the slice's chunks and are summed in wave order.
// Trailing workgroups quantise x to Q8_1 as in the other router kernels.
typedef double d4 __attribute__((ext_vector_type(4)));

template <int MT, int NT, int WM, int WN, int WK>
__global__ __launch_bounds__(256) void k_route_logits_mf(const float* __restrict__ x,
                                                         const float* __restrict__ W, int T,
                                                         int H, int E, int S,
                                                         double* __restrict__ part,
                                                         int n_logit_wg, ActPtr xq) {
    static_assert(WM * WN * WK == 4, "four waves per workgroup");
    if ((int)blockIdx.x >= n_logit_wg) {
        const int nb = H / QK;
        const long blk = (long)(blockIdx.x - n_logit_wg) * 8 + threadIdx.x / 32;
        if (blk >= (long)T * nb) return;
        const int l = threadIdx.x % 32;
        const long r = blk / nb, b = blk % nb;
        quant_q8_1_32(x[r * H + b * QK + l], l, xq.q + r * H + b * QK, xq.ds + r * nb + b,
                      xq.sq + r * nb + b);
        return;
    }
    constexpr int BM = 16 * MT * WM, BN = 16 * NT * WN;
    const int gm = (T + BM - 1) / BM, gn = (E + BN - 1) / BN;
    int b = blockIdx.x;
    const int tm = b % gm;
    b /= gm;
    const int tn = b % gn;
    const int s = b / gn;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wk = wave % WK, wm = (wave / WK) % WM, wn = wave / (WK * WM);
    const int r = lane & 15, q = lane >> 4;
    const int slice = H / S, nch = slice / 16;
    const int tb = tm * BM + wm * 16 * MT, eb = tn * BN + wn * 16 * NT;
    const float* xr[MT];
    const float* wr[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
        xr[i] = x + (size_t)min(tb + i * 16 + r, T - 1) * H + s * slice + 4 * q;
#pragma unroll
    for (int j = 0; j < NT; ++j)
        wr[j] = W + (size_t)min(eb + j * 16 + r, E - 1) * H + s * slice + 4 * q;
    d4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = d4{0.0, 0.0, 0.0, 0.0};
    // the wave's chunks are wk, wk + WK, ...; they are taken CG at a time into
    // two register sets used in turn (no copies between them, so a set's loads
    // stay in flight while the other set is multiplied).  A chunk past the
    // last is loaded from the last chunk and not multiplied.
    constexpr int CG = 2;
    float4 a0[CG][MT], w0[CG][NT], a1[CG][MT], w1[CG][NT];
    auto load_set = [&](float4 (&as)[CG][MT], float4 (&ws)[CG][NT], int c) {
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            const int cc = min(c + g * WK, nch - 1);
#pragma unroll
            for (int i = 0; i < MT; ++i) as[g][i] = *reinterpret_cast<const float4*>(xr[i] + cc * 16);
#pragma unroll
            for (int j = 0; j < NT; ++j) ws[g][j] = *reinterpret_cast<const float4*>(wr[j] + cc * 16);
        }
    };
    auto mul_set = [&](const float4 (&as)[CG][MT], const float4 (&ws)[CG][NT], int c) {
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            if (c + g * WK >= nch) break;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const float4 av4 = as[g][i];
                    const float av = u == 0 ? av4.x : u == 1 ? av4.y : u == 2 ? av4.z : av4.w;
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const float4 bv4 = ws[g][j];
                        const float bv = u == 0 ? bv4.x : u == 1 ? bv4.y : u == 2 ? bv4.z : bv4.w;
                        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av, (double)bv,
                                                                         acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
    };
    constexpr int STEP = CG * WK;
    load_set(a0, w0, wk);
    for (int c = wk; c < nch; c += 2 * STEP) {
        load_set(a1, w1, c + STEP);
        mul_set(a0, w0, c);
        load_set(a0, w0, c + 2 * STEP);
        mul_set(a1, w1, c + STEP);
    }
    if constexpr (WK > 1) {
        __shared__ double s_red[WK - 1][MT * NT * 4][64];
        if (wk > 0) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) s_red[wk - 1][(i * NT + j) * 4 + v][lane] = acc[i][j][v];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll
        for (int o = 0; o < WK - 1; ++o)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][v] += s_red[o][(i * NT + j) * 4 + v][lane];
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int e = eb + j * 16 + r;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = tb + i * 16 + q + 4 * v;
                if (t < T && e < E) part[((size_t)s * T + t) * E + e] = acc[i][j][v];
            }
        }
}

// ---------------------------------------------------------------------------
// Many-token router logits: a workgroup computes a 64-token x 64-expert tile of
// one K slice.  x and W_r tiles are staged in LDS as fp64 (k-major), each thread
// accumulates 4 tokens x 4 experts in fp64 (products of two floats are exact in
// fp64).  Trailing workgroups quantise x to Q8_1, as in k_route_logits.
constexpr int RT_M = 64, RT_N = 64, RT_K = 32, RT_PAD = 2;

__global__ __launch_bounds__(256) void k_route_logits_tiled(const float* __restrict__ x,
                                                            const float* __restrict__ W, int T,
                                                            int H, int E, int S,
                                                            double* __restrict__ part,
                                                            int n_logit_wg, ActPtr xq) {
    if ((int)blockIdx.x >= n_logit_wg) {
        const int nb = H / QK;
        const long blk = (long)(blockIdx.x - n_logit_wg) * 8 + threadIdx.x / 32;
        if (blk >= (long)T * nb) return;
        const int l = threadIdx.x % 32;
        const long r = blk / nb, b = blk % nb;
        quant_q8_1_32(x[r * H + b * QK + l], l, xq.q + r * H + b * QK, xq.ds + r * nb + b,
                      xq.sq + r * nb + b);
        return;
    }
    __shared__ __align__(16) double sx[RT_K][RT_M + RT_PAD];
    __shared__ __align__(16) double sw[RT_K][RT_N + RT_PAD];
    const int gm = (T + RT_M - 1) / RT_M, gn = (E + RT_N - 1) / RT_N;
    int b = blockIdx.x;
    const int tm = b % gm;
    b /= gm;
    const int tn = b % gn;
    const int s = b / gn;
    const int slice = H / S, k0 = s * slice;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int kk = k0; kk < k0 + slice; kk += RT_K) {
        // 64 rows x 32 floats of x and of W_r: two float4 per thread each
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int idx = threadIdx.x + j * 256;
            const int row = idx >> 3, c4 = idx & 7;
            const int t = min(tm * RT_M + row, T - 1), e = min(tn * RT_N + row, E - 1);
            const float4 xv = *reinterpret_cast<const float4*>(x + (size_t)t * H + kk + c4 * 4);
            const float4 wv = *reinterpret_cast<const float4*>(W + (size_t)e * H + kk + c4 * 4);
            sx[c4 * 4 + 0][row] = xv.x;
            sx[c4 * 4 + 1][row] = xv.y;
            sx[c4 * 4 + 2][row] = xv.z;
            sx[c4 * 4 + 3][row] = xv.w;
            sw[c4 * 4 + 0][row] = wv.x;
            sw[c4 * 4 + 1][row] = wv.y;
            sw[c4 * 4 + 2][row] = wv.z;
            sw[c4 * 4 + 3][row] = wv.w;
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < RT_K; ++k) {
            double xa[4], wb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xa[i] = sx[k][ty * 4 + i];
                wb[i] = sw[k][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(xa[i], wb[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tm * RT_M + ty * 4 + i;
        if (t >= T) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tn * RT_N + tx * 4 + j;
            if (e < E) part[((size_t)s * T + t) * E + e] = acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Selection for one token by one wave: sum the K-slice partials (in slice
// order), add the bias, apply the group limit, top-k with ties to the lower id,
// softmax over the chosen logits in fp64.  Lane j < k returns rank j's expert
// and weight; other lanes return id -1.
// (value, index) pair of lane `src` moved in by one cross-lane step: DPP row
// ops inside a 16-lane row, the gfx950 row swaps across rows.  The reduction
// below is a max over (value, -index), which is associative and commutative,
// so mirrored partners reduce as well as butterflies do.
template <int STEP>
__device__ __forceinline__ void xlane(double v, int i, double& ov, int& oi) {
    const long long b = __double_as_longlong(v);
    int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
    if constexpr (STEP < 4) {
        constexpr int CTRL = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
        lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xf, 0xf, false);
        hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xf, 0xf, false);
        oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
    } else if constexpr (STEP == 4) {
        auto a = __builtin_amdgcn_permlane16_swap((unsigned)lo, (unsigned)lo, false, false);
        auto c = __builtin_amdgcn_permlane16_swap((unsigned)hi, (unsigned)hi, false, false);
        auto d = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
        // the swap hands each lane its partner row's value in one of the two results
        const bool odd_row = (threadIdx.x & 16) != 0;
        lo = (int)(odd_row ? a[0] : a[1]);
        hi = (int)(odd_row ? c[0] : c[1]);
        oi = (int)(odd_row ? d[0] : d[1]);
    } else {
        auto a = __builtin_amdgcn_permlane32_swap((unsigned)lo, (unsigned)lo, false, false);
        auto c = __builtin_amdgcn_permlane32_swap((unsigned)hi, (unsigned)hi, false, false);
        auto d = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
        const bool upper = (threadIdx.x & 32) != 0;
        lo = (int)(upper ? a[0] : a[1]);
        hi = (int)(upper ? c[0] : c[1]);
        oi = (int)(upper ? d[0] : d[1]);
    }
    ov = __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

template <int STEP>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
    double ov;
    int oi;
    xlane<STEP>(v, i, ov, oi);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}

template <int STEP>
__device__ __forceinline__ void argmax_step_f(float& v, int& i) {
    float ov;
    int oi;
    if constexpr (STEP < 4) {
        constexpr int CTRL = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
        ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
        oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
    } else if constexpr (STEP == 4) {
        auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        auto d = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
        const bool odd_row = (threadIdx.x & 16) != 0;
        ov = __uint_as_float(odd_row ? a[0] : a[1]);
        oi = (int)(odd_row ? d[0] : d[1]);
    } else {
        auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        auto d = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
        const bool upper = (threadIdx.x & 32) != 0;
        ov = __uint_as_float(upper ? a[0] : a[1]);
        oi = (int)(upper ? d[0] : d[1]);
    }
    // (value desc, id asc); an empty lane (id 0x7fffffff) loses to any candidate
    if (oi != 0x7fffffff && (i == 0x7fffffff || ov > v || (ov == v && oi < i))) { v = ov; i = oi; }
}

__device__ __forceinline__ void argmax_f(float& v, int& i) {
    argmax_step_f<0>(v, i);
    argmax_step_f<1>(v, i);
    argmax_step_f<2>(v, i);
    argmax_step_f<3>(v, i);
    argmax_step_f<4>(v, i);
    argmax_step_f<5>(v, i);
}

__device__ __forceinline__ void argmax_pair(double& v, int& i) {
    argmax_step<0>(v, i);
    argmax_step<1>(v, i);
    argmax_step<2>(v, i);
    argmax_step<3>(v, i);
    argmax_step<4>(v, i);
    argmax_step<5>(v, i);
}

// order-preserving map of a double to an unsigned 64-bit key
__device__ __forceinline__ unsigned long long dkey(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double dkey_inv(unsigned long long k) {
    const unsigned long long b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)b);
}

constexpr int ROUTE_SMAX = 16; // K slices

struct SelectArgs {
    const double* part;
    int S, T, E, k;
    const float* bias;
    const int32_t* groups;
    int G, TG;
    double* logits_tap;
};

// gkey: 64 words of LDS private to the calling wave.  MAXE_LANE = experts per
// lane (E <= 64 * MAXE_LANE).
template <int MAXE_LANE>
__device__ __forceinline__ void select_token(const SelectArgs& A, int t,
                                             unsigned long long* gkey, int& my_id,
                                             float& my_w) {
    const int lane = threadIdx.x & 63;
    const double NEG = -__builtin_huge_val();
    double l[MAXE_LANE];
    bool ok[MAXE_LANE];
    bool taken[MAXE_LANE];
#pragma unroll
    for (int m = 0; m < MAXE_LANE; ++m) {
        const int e = lane + 64 * m;
        l[m] = NEG;
        ok[m] = e < A.E;
        taken[m] = e >= A.E;
        if (e < A.E) {
            double ps[ROUTE_SMAX];
#pragma unroll
            for (int s = 0; s < ROUTE_SMAX; ++s)
                ps[s] = s < A.S ? A.part[((size_t)s * A.T + t) * A.E + e] : 0.0;
            double v = 0.0;
#pragma unroll
            for (int s = 0; s < ROUTE_SMAX; ++s)
                if (s < A.S) v += ps[s];
            if (A.bias) v += (double)A.bias[e];
            l[m] = v;
            if (A.logits_tap) A.logits_tap[(size_t)t * A.E + e] = v;
        }
    }
    if (A.G > 0) {
        // group score = largest member logit, through order-preserving keys
        gkey[lane] = 0ull;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m) {
            const int e = lane + 64 * m;
            if (e < A.E) {
                const unsigned gl = (unsigned)A.groups[e];
                if (gl < (unsigned)A.G) atomicMax(&gkey[gl], dkey(l[m] + 0.0));   // -0 -> +0
            }
        }
        __builtin_amdgcn_wave_barrier();
        const double gs = lane < A.G && gkey[lane] ? dkey_inv(gkey[lane]) : NEG;
        bool gsel = false;
        for (int n = 0; n < A.TG; ++n) {
            double v = (lane < A.G && !gsel) ? gs : NEG;
            int i = (lane < A.G && !gsel) ? lane : 0x7fffffff;
            argmax_pair(v, i);
            if (lane == i) gsel = true;
        }
        const unsigned long long sel = __ballot(gsel);
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m) {
            const int e = lane + 64 * m;
            if (e < A.E) {
                const unsigned gl = (unsigned)A.groups[e];
                ok[m] = gl < (unsigned)A.G && ((sel >> gl) & 1ull);
            }
        }
    }
    // Fast path: rank by (fp32(l) desc, id asc) with 32-bit lane exchanges.
    // fp32 rounding is monotone, so when the k+1 best fp32 values are strictly
    // decreasing the chosen set and its order are those of the fp64 logits;
    // otherwise (an fp32 tie among them) rank again in fp64.
    double top_l = 0.0, mine = 0.0;
    my_id = -1;
    float f[MAXE_LANE];
#pragma unroll
    for (int m = 0; m < MAXE_LANE; ++m) f[m] = (float)l[m];
    bool ftaken[MAXE_LANE];
#pragma unroll
    for (int m = 0; m < MAXE_LANE; ++m) ftaken[m] = taken[m] || !ok[m];
    float prev = __builtin_inff();
    bool strict = true;
    int fid = -1, found = 0;
    const int need = A.k + 1;
    for (int j = 0; j < need; ++j) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m) {
            const int e = lane + 64 * m;
            if (!ftaken[m] && (bi == 0x7fffffff || f[m] > bv)) { bv = f[m]; bi = e; }
        }
        argmax_f(bv, bi);
        if (bi == 0x7fffffff) break;                 // fewer than k+1 candidates
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m)
            if (lane + 64 * m == bi) ftaken[m] = true;
        if (!(bv < prev)) strict = false;
        prev = bv;
        if (j < A.k && lane == j) fid = bi;
        ++found;
    }
    if (found < A.k) strict = false;    // too few allowed experts: the fp64 path falls back
    if (strict) {
        // fp64 logit of each chosen expert, from the lane that holds it
        my_id = fid;
        const int src = fid < 0 ? 0 : fid & 63, slot = fid < 0 ? 0 : fid >> 6;
        double got = 0.0;
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m) {
            const double lm = __shfl(l[m], src, 64);
            if (m == slot) got = lm;
        }
        mine = got;
        top_l = __shfl(mine, 0, 64);
    } else {
        for (int j = 0; j < A.k; ++j) {
            double bv = NEG;
            int bi = 0x7fffffff;
#pragma unroll
            for (int m = 0; m < MAXE_LANE; ++m) {
                const int e = lane + 64 * m;
                if (ok[m] && !taken[m] && (l[m] > bv || (l[m] == bv && e < bi))) { bv = l[m]; bi = e; }
            }
            argmax_pair(bv, bi);
            if (bi == 0x7fffffff) {
                // labels that break the equal-size-groups contract left fewer than k
                // candidates: fall back to every expert not yet chosen (k <= E)
                bv = NEG;
#pragma unroll
                for (int m = 0; m < MAXE_LANE; ++m) {
                    const int e = lane + 64 * m;
                    if (!taken[m] && (bi == 0x7fffffff || l[m] > bv || (l[m] == bv && e < bi))) { bv = l[m]; bi = e; }
                }
                argmax_pair(bv, bi);
            }
#pragma unroll
            for (int m = 0; m < MAXE_LANE; ++m)
                if (lane + 64 * m == bi) taken[m] = true;
            if (j == 0) top_l = bv;
            if (lane == j) { my_id = bi; mine = bv; }
        }
    }
    const double ex = lane < A.k ? exp(mine - top_l) : 0.0;
    double den = 0.0;
    for (int j = 0; j < A.k; ++j) den += __shfl(ex, j, 64);        // rank order
    my_w = lane < A.k ? (float)(ex / den) : 0.0f;
}

// One wave per token (any T).
template <int MAXE_LANE>
__global__ __launch_bounds__(64) void k_router_topk(SelectArgs A, int32_t* __restrict__ ids,
                                                    float* __restrict__ wts) {
    __shared__ unsigned long long gkey[64];
    const int t = blockIdx.x, lane = threadIdx.x;
    int id;
    float wt;
    select_token<MAXE_LANE>(A, t, gkey, id, wt);
    if (lane < A.k) {
        ids[(size_t)t * A.k + lane] = id;
        wts[(size_t)t * A.k + lane] = wt;
    }
}

// Decode sizes (T <= 32, T*k <= 1024): one workgroup routes every token (one wave
// per token) and buckets the assignments.  Per expert: count, token bitmask;
// slots = experts with tokens in id order; an assignment's place in its
// expert's list = its token's rank among that expert's tokens.
constexpr int SMALL_TMAX = 32;
constexpr int SMALL_NW = 16;

template <int MAXE_LANE>
__global__ __launch_bounds__(SMALL_NW * 64) void k_route_small(SelectArgs A, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ lists,
                                                               uint32_t* __restrict__ ctrl,
                                                               int32_t* __restrict__ active) {
    __shared__ unsigned long long gkey[SMALL_NW][64];
    __shared__ int s_cnt[512];
    __shared__ unsigned s_mask[512];
    __shared__ int s_wtot[SMALL_NW];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int e = threadIdx.x; e < A.E; e += blockDim.x) {
        s_cnt[e] = 0;
        s_mask[e] = 0u;
    }
    __syncthreads();
    int my_id[2] = {-1, -1};
    for (int rep = 0; rep < 2; ++rep) {
        const int t = wave + rep * SMALL_NW;
        if (t >= A.T) break;
        float wt;
        select_token<MAXE_LANE>(A, t, gkey[wave], my_id[rep], wt);
        if (lane < A.k) {
            ids[(size_t)t * A.k + lane] = my_id[rep];
            wts[(size_t)t * A.k + lane] = wt;
            atomicAdd(&s_cnt[my_id[rep]], 1);
            atomicOr(&s_mask[my_id[rep]], 1u << t);
        }
    }
    __syncthreads();
    // counts of every expert; slots of the active ones (prefix over E <= 512 = 8 waves)
    const int e = threadIdx.x;
    const int c = e < A.E ? s_cnt[e] : 0;
    const unsigned long long bal = __ballot(c > 0);
    if (lane == 0) s_wtot[wave] = __popcll(bal);
    __syncthreads();
    if (e < A.E) {
        counts[e] = c;
        if (c > 0) {
            int slot = __popcll(bal & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w) slot += s_wtot[w];
            active[slot] = e;
        }
    }
    if (threadIdx.x == 0) {
        int n = 0;
        for (int w = 0; w < SMALL_NW; ++w) n += s_wtot[w];
        ctrl[CW_N_ACTIVE] = n;
    }
    // list positions: the token's rank among the expert's tokens
    for (int rep = 0; rep < 2; ++rep) {
        const int t = wave + rep * SMALL_NW;
        if (t >= A.T) break;
        if (lane < A.k) {
            const int id = my_id[rep];
            const int pos = __popc(s_mask[id] & ((1u << t) - 1u));
            lists[(size_t)id * A.T + pos] = t * A.k + lane;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode routing (T <= DECODE_T), two launches and no cross-workgroup fences.
//
// k_route_logits_dec: workgroups [0, E): expert e = blockIdx.x, 256 threads
// over the H-wide row of W_r with every load issued at once (indices past the
// row are clamped and masked), logits l[t][e] in fp64 for every token;
// workgroups [E, E + nq): Q8_1(x).
constexpr int ROUTE_U = 8;   // float4 per thread: H <= 8192

__global__ __launch_bounds__(256) void k_route_logits_dec(const float* __restrict__ x,
                                                          const float* __restrict__ W, int T,
                                                          int H, int E, double* __restrict__ logits,
                                                          ActPtr xq) {
    __shared__ double s_part[DECODE_T][4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((int)blockIdx.x >= E) {
        const int nb = H / QK;
        const long blk = (long)(blockIdx.x - E) * 8 + threadIdx.x / 32;
        if (blk >= (long)T * nb) return;
        const int l = threadIdx.x % 32;
        const long r = blk / nb, b = blk % nb;
        quant_q8_1_32(x[r * H + b * QK + l], l, xq.q + r * H + b * QK, xq.ds + r * nb + b,
                      xq.sq + r * nb + b);
        return;
    }
    const int e = blockIdx.x;
    const int h4 = H / 4;
    const float4* wrow = reinterpret_cast<const float4*>(W + (size_t)e * H);
    float4 w[ROUTE_U];
    bool valid[ROUTE_U];
#pragma unroll
    for (int u = 0; u < ROUTE_U; ++u) {
        const int i = threadIdx.x + 256 * u;
        valid[u] = i < h4;
        w[u] = wrow[min(i, h4 - 1)];
    }
    for (int t = 0; t < T; ++t) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)t * H);
        float4 xv[ROUTE_U];
#pragma unroll
        for (int u = 0; u < ROUTE_U; ++u) xv[u] = xr[min((int)threadIdx.x + 256 * u, h4 - 1)];
        double acc = 0.0;
#pragma unroll
        for (int u = 0; u < ROUTE_U; ++u) {
            if (valid[u]) {
                acc = fma((double)xv[u].x, (double)w[u].x, acc);
                acc = fma((double)xv[u].y, (double)w[u].y, acc);
                acc = fma((double)xv[u].z, (double)w[u].z, acc);
                acc = fma((double)xv[u].w, (double)w[u].w, acc);
            }
        }
        acc = wave_sum_d(acc);
        if (lane == 0) s_part[t][wave] = acc;
    }
    __syncthreads();
    if ((int)threadIdx.x < T) {
        const int t = threadIdx.x;
        logits[(size_t)t * E + e] = ((s_part[t][0] + s_part[t][1]) + s_part[t][2]) + s_part[t][3];
    }
}

// k_route_select_dec: one workgroup.  Every (token, expert) pair computes its
// rank = the number of allowed experts that beat it ((logit desc, id asc), in
// fp64, all pairs in parallel); rank < k gives the slot.  With group labels the
// groups are ranked the same way by their largest member logit first.  Then
// softmax over the chosen logits (fp64, rank order) and the bucketing.
constexpr int SEL_NT = 1024;

__global__ __launch_bounds__(SEL_NT) void k_route_select_dec(SelectArgs A,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ wts,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ lists,
                                                             uint32_t* __restrict__ ctrl,
                                                             int32_t* __restrict__ active) {
    // logits live as ordered keys (dkey of l + 0.0: -0 and +0 compare equal as
    // doubles and get one key); dkey_inv gives the logit back for the softmax
    __shared__ unsigned long long s_key[DECODE_T * 512];
    __shared__ unsigned long long s_gkey[DECODE_T][64];
    __shared__ unsigned char s_gsel[DECODE_T][64];
    __shared__ int s_nallow[DECODE_T];
    __shared__ int s_sel[DECODE_T][32];
    __shared__ double s_ex[DECODE_T][32];
    __shared__ int s_cnt[512];
    __shared__ unsigned s_mask[512];
    __shared__ int s_wtot[SEL_NT / 64];
    const int T = A.T, E = A.E, k = A.k, G = A.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int TE = T * E;
    for (int i = tid; i < TE; i += SEL_NT) {
        const int e = i % E;
        double v = A.part[i];
        if (A.bias) v += (double)A.bias[e];
        s_key[i] = dkey(v + 0.0);
        if (A.logits_tap) A.logits_tap[i] = v;
    }
    for (int i = tid; i < E; i += SEL_NT) {
        s_cnt[i] = 0;
        s_mask[i] = 0u;
    }
    if (G > 0) {
        for (int i = tid; i < T * 64; i += SEL_NT) s_gkey[i / 64][i % 64] = 0ull;
        if (tid < T) s_nallow[tid] = 0;
    }
    __syncthreads();
    if (G > 0) {
        for (int i = tid; i < TE; i += SEL_NT) {
            const int t = i / E, e = i - t * E;
            const unsigned gl = (unsigned)A.groups[e];
            if (gl < (unsigned)G) atomicMax(&s_gkey[t][gl], s_key[i]);
        }
        __syncthreads();
        // group rank among the token's groups (key desc, group asc); keep rank < TG
        for (int i = tid; i < T * G; i += SEL_NT) {
            const int t = i / G, g = i - t * G;
            const unsigned long long kg = s_gkey[t][g];
            int r = 0;
            for (int h = 0; h < G; ++h) {
                const unsigned long long kh = s_gkey[t][h];
                r += (int)(kh > kg) | ((int)(kh == kg) & (int)(h < g));
            }
            s_gsel[t][g] = r < A.TG;
        }
        __syncthreads();
        // allowed experts per token: one LDS atomic per wave and token run
        for (int b0 = 0; b0 < TE; b0 += SEL_NT) {
            const int i = b0 + tid;
            int t = -1;
            bool al = false;
            if (i < TE) {
                t = i / E;
                const unsigned gl = (unsigned)A.groups[i - t * E];
                al = gl < (unsigned)G && s_gsel[t][gl];
            }
            if (al) atomicAdd(&s_nallow[t], 1);
        }
        __syncthreads();
        // an excluded expert gets key 0: below every logit's key, so it never
        // beats another and is never chosen; a token with fewer than k allowed
        // experts (labels that break the equal-size-groups contract) keeps all
        for (int i = tid; i < TE; i += SEL_NT) {
            const int t = i / E;
            const unsigned gl = (unsigned)A.groups[i - t * E];
            const bool al = gl < (unsigned)G && s_gsel[t][gl];
            if (!al && s_nallow[t] >= k) s_key[i] = 0ull;
        }
        __syncthreads();
    }
    // exact ranks: P lanes per (token, expert) pair each count the rivals
    // (key desc, id asc) among E/P of them, eight loads at a time, no branches
    int P = 1;
    while (P < 64 && TE * P * 2 <= SEL_NT) P *= 2;
    const int lp = 31 - __clz(P);
    for (int b0 = 0; b0 < (TE << lp); b0 += SEL_NT) {
        const int gi = b0 + tid;
        const int i = gi >> lp, part = gi & (P - 1);
        int r = 0, t = 0, e = 0;
        unsigned long long ke = 0ull;
        if (i < TE) {
            t = i / E;
            e = i - t * E;
            ke = s_key[i];
        }
        const bool cand = ke != 0ull;
        if (cand) {
            constexpr int U = 8;
            const unsigned long long* kt = s_key + t * E;
            for (int h0 = part; h0 < E; h0 += U * P) {
                unsigned long long kh[U];
#pragma unroll
                for (int u = 0; u < U; ++u) kh[u] = kt[min(h0 + u * P, E - 1)];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int h = h0 + u * P;
                    r += (int)(h < E) & ((int)(kh[u] > ke) | ((int)(kh[u] == ke) & (int)(h < e)));
                }
            }
        }
        for (int o = 1; o < P; o <<= 1) r += __shfl_xor(r, o);
        if (cand && part == 0 && r < k) s_sel[t][r] = e;
    }
    __syncthreads();
    // softmax over the chosen logits, rank order, fp64
    for (int i = tid; i < T * k; i += SEL_NT) {
        const int t = i / k, j = i - t * k;
        s_ex[t][j] = exp(dkey_inv(s_key[t * E + s_sel[t][j]]) - dkey_inv(s_key[t * E + s_sel[t][0]]));
    }
    __syncthreads();
    for (int i = tid; i < T * k; i += SEL_NT) {
        const int t = i / k, j = i - t * k;
        double den = 0.0;
        for (int jj = 0; jj < k; ++jj) den += s_ex[t][jj];
        const int id = s_sel[t][j];
        ids[i] = id;
        wts[i] = (float)(s_ex[t][j] / den);
        atomicAdd(&s_cnt[id], 1);
        atomicOr(&s_mask[id], 1u << t);
    }
    __syncthreads();
    // counts of every expert; slots of the active ones in id order (one expert per thread)
    const int c = tid < E ? s_cnt[tid] : 0;
    const unsigned long long bal = __ballot(c > 0);
    if (lane == 0) s_wtot[wave] = __popcll(bal);
    __syncthreads();
    if (tid < E) {
        counts[tid] = c;
        if (c > 0) {
            int slot = __popcll(bal & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w) slot += s_wtot[w];
            active[slot] = tid;
        }
    }
    if (tid == 0) {
        int n = 0;
        for (int w = 0; w < SEL_NT / 64; ++w) n += s_wtot[w];
        ctrl[CW_N_ACTIVE] = n;
    }
    // list positions: the token's rank among the expert's tokens
    for (int i = tid; i < T * k; i += SEL_NT) {
        const int t = i / k;
        const int id = s_sel[t][i - t * k];
        lists[(size_t)id * T + __popc(s_mask[id] & ((1u << t) - 1u))] = i;
    }
}

// ---------------------------------------------------------------------------
// Per-token selection, one workgroup per token (any T): the token's logits are
// the K-slice partials summed in slice order plus the bias, held as ordered
// keys; with group labels the groups are ranked first by their largest member
// key and the experts outside the chosen groups get key 0; every expert's rank
// is the number of experts that beat it ((key desc, id asc)); rank < k is the
// slot.  Softmax over the chosen logits in fp64, rank order.
// BUCKET (T <= 32, T*k <= 1024): the last workgroup to finish (an arrival
// counter) buckets every token's assignments, as k_route_select_dec does, and
// clears the counter for the next call.
// (NT threads: 1024 when few tokens share the chip, 256 when many do)
template <bool BUCKET, int TSEL_NT>
__global__ __launch_bounds__(TSEL_NT) void k_route_select_tok(SelectArgs A,
                                                              int32_t* __restrict__ ids,
                                                              float* __restrict__ wts,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ lists,
                                                              uint32_t* __restrict__ ctrl,
                                                              int32_t* __restrict__ active) {
    __shared__ unsigned long long s_key[512];
    __shared__ unsigned s_khi[512];
    __shared__ unsigned long long s_gkey[64];
    __shared__ unsigned char s_gsel[64];
    __shared__ int s_nallow;
    __shared__ int s_sel[32];
    __shared__ double s_ex[32];
    __shared__ int s_last;
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = A.T, E = A.E, k = A.k, G = A.G;
    for (int e = tid; e < E; e += TSEL_NT) {
        double ps[ROUTE_SMAX];
#pragma unroll
        for (int sl = 0; sl < ROUTE_SMAX; ++sl)
            ps[sl] = sl < A.S ? A.part[((size_t)sl * T + t) * E + e] : 0.0;
        double v = 0.0;
#pragma unroll
        for (int sl = 0; sl < ROUTE_SMAX; ++sl)
            if (sl < A.S) v += ps[sl];
        if (A.bias) v += (double)A.bias[e];
        if (A.logits_tap) A.logits_tap[(size_t)t * E + e] = v;
        s_key[e] = dkey(v + 0.0);
    }
    if (G > 0) {
        if (tid < 64) s_gkey[tid] = 0ull;
        if (tid == 0) s_nallow = 0;
        __syncthreads();
        for (int e = tid; e < E; e += TSEL_NT) {
            const unsigned gl = (unsigned)A.groups[e];
            if (gl < (unsigned)G) atomicMax(&s_gkey[gl], s_key[e]);
        }
        __syncthreads();
        if (tid < G) {
            const unsigned long long kg = s_gkey[tid];
            int r = 0;
            for (int h = 0; h < G; ++h) {
                const unsigned long long kh = s_gkey[h];
                r += (int)(kh > kg) | ((int)(kh == kg) & (int)(h < tid));
            }
            s_gsel[tid] = r < A.TG;
        }
        __syncthreads();
        int nal = 0;
        for (int e = tid; e < E; e += TSEL_NT) {
            const unsigned gl = (unsigned)A.groups[e];
            nal += (int)(gl < (unsigned)G && s_gsel[gl]);
        }
        for (int o = 32; o > 0; o >>= 1) nal += __shfl_xor(nal, o, 64);
        if (lane == 0 && nal) atomicAdd(&s_nallow, nal);
        __syncthreads();
        // fewer than k allowed (labels that break the equal-size-groups
        // contract): every expert stays a candidate
        if (s_nallow >= k) {
            for (int e = tid; e < E; e += TSEL_NT) {
                const unsigned gl = (unsigned)A.groups[e];
                if (!(gl < (unsigned)G && s_gsel[gl])) s_key[e] = 0ull;
            }
        }
    }
    __syncthreads();
    // ranks: P lanes per expert each count the rivals among E/P of them, first
    // on the top 32 bits of the keys (one compare each); an expert that could
    // be chosen and shares those bits with a rival is ranked again on the
    // whole keys
    for (int e = tid; e < E; e += TSEL_NT) s_khi[e] = (unsigned)(s_key[e] >> 32);
    __syncthreads();
    int P = 1;
    while (P < 64 && E * P * 2 <= TSEL_NT) P *= 2;
    const int lp = 31 - __clz(P);
    for (int b0 = 0; b0 < (E << lp); b0 += TSEL_NT) {
        const int gi = b0 + tid;
        const int e = gi >> lp, pt = gi & (P - 1);
        const unsigned long long ke = e < E ? s_key[e] : 0ull;
        const unsigned khi = (unsigned)(ke >> 32);
        int gt = 0, eq = 0;
        if (ke != 0ull) {
            constexpr int U = 8;
            for (int h0 = pt; h0 < E; h0 += U * P) {
                unsigned kh[U];
#pragma unroll
                for (int u = 0; u < U; ++u) kh[u] = s_khi[min(h0 + u * P, E - 1)];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int in = h0 + u * P < E;
                    gt += in & (int)(kh[u] > khi);
                    eq += in & (int)(kh[u] == khi);
                }
            }
        }
        for (int o = 1; o < P; o <<= 1) {
            gt += __shfl_xor(gt, o);
            eq += __shfl_xor(eq, o);
        }
        int r = gt;
        const bool exact = ke != 0ull && gt < k && eq > 1;
        if (__ballot(exact)) {
            int rx = 0;
            if (exact) {
                for (int h = pt; h < E; h += P) {
                    const unsigned long long kh = s_key[h];
                    rx += (int)(kh > ke) | ((int)(kh == ke) & (int)(h < e));
                }
            }
            for (int o = 1; o < P; o <<= 1) rx += __shfl_xor(rx, o);
            if (exact) r = rx;
        }
        if (ke != 0ull && pt == 0 && r < k) s_sel[r] = e;
    }
    __syncthreads();
    if (tid < k) {
        const double l0 = dkey_inv(s_key[s_sel[0]]);
        s_ex[tid] = exp(dkey_inv(s_key[s_sel[tid]]) - l0);
    }
    __syncthreads();
    if (tid < k) {
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += s_ex[j];
        // ids are read by another workgroup of this grid when bucketing: an
        // agent-scope store writes through to the device-coherent level
        if constexpr (BUCKET)
            __hip_atomic_store(ids + (size_t)t * k + tid, s_sel[tid], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        else
            ids[(size_t)t * k + tid] = s_sel[tid];
        wts[(size_t)t * k + tid] = (float)(s_ex[tid] / den);
    }
    if constexpr (BUCKET) {
        __shared__ int s_ids[1024];
        __shared__ int s_cnt[512];
        __shared__ unsigned s_mask[512];
        __shared__ int s_wtot[TSEL_NT / 64];
        if (T > 1) {
            // the id stores have completed (vmcnt 0) before this workgroup
            // counts itself in; the last arrival reads every token's ids with
            // agent-scope loads
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0)
                s_last = __hip_atomic_fetch_add(&ctrl[CW_ROUTE_ARRIVE], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(T - 1);
            __syncthreads();
            if (!s_last) return;
        } else {
            __syncthreads();
        }
        const int nA = T * k;
        for (int e = tid; e < E; e += TSEL_NT) {
            s_cnt[e] = 0;
            s_mask[e] = 0u;
        }
        for (int i = tid; i < nA; i += TSEL_NT)
            s_ids[i] = __hip_atomic_load(ids + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        for (int i = tid; i < nA; i += TSEL_NT) {
            const int id = s_ids[i];
            atomicAdd(&s_cnt[id], 1);
            atomicOr(&s_mask[id], 1u << (i / k));
        }
        __syncthreads();
        // counts of every expert; slots of the active ones in id order
        int c[2], nact = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = 2 * tid + h;
            c[h] = e < E ? s_cnt[e] : 0;
            nact += c[h] > 0;
        }
        // exclusive scan of nact over the workgroup
        int incl = nact;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) s_wtot[wave] = incl;
        __syncthreads();
        int slot = incl - nact;
        for (int w2 = 0; w2 < wave; ++w2) slot += s_wtot[w2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = 2 * tid + h;
            if (e < E) {
                counts[e] = c[h];
                if (c[h] > 0) active[slot++] = e;
            }
        }
        if (tid == 0) {
            int n = 0;
            for (int w2 = 0; w2 < TSEL_NT / 64; ++w2) n += s_wtot[w2];
            ctrl[CW_N_ACTIVE] = n;
            ctrl[CW_ROUTE_ARRIVE] = 0u;
        }
        // list positions: the token's rank among the expert's tokens
        for (int i = tid; i < nA; i += TSEL_NT) {
            const int id = s_ids[i], tt = i / k;
            lists[(size_t)id * T + __popc(s_mask[id] & ((1u << tt) - 1u))] = i;
        }
    }
}

// ---------------------------------------------------------------------------
// Bucketing: workgroup e lists the assignments routed to expert e in token order.
// The last workgroup to finish compacts the experts with tokens into slots and
// computes each slot's first token tile (tiles of tile_m tokens).
constexpr int BK_NT = 1024;

__global__ __launch_bounds__(BK_NT) void k_bucket(const int32_t* __restrict__ ids, int A, int T,
                                                  int E, int tile_m, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ lists,
                                                  uint32_t* __restrict__ ctrl,
                                                  int32_t* __restrict__ active,
                                                  int32_t* __restrict__ tile_start,
                                                  int32_t* __restrict__ tile_map) {
    constexpr int NWV = BK_NT / 64;
    __shared__ int wsum[NWV];
    __shared__ int s_wa[NWV], s_wt[NWV];
    __shared__ int is_last;
    const int e = blockIdx.x, tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    // wave w owns the contiguous w-th sixteenth [q0, q1) of the assignments:
    // count its matches, then (after one exchange of the wave totals) list
    // them in order
    const int Q = (A + NWV - 1) / NWV;
    const int q0 = min(wave * Q, A), q1 = min(q0 + Q, A);
    int cnt = 0;
#pragma unroll 4
    for (int a0 = q0; a0 < q1; a0 += 64) {
        const int a = a0 + lane;
        cnt += __popcll(__ballot(a < q1 && ids[a] == e));
    }
    if (lane == 0) wsum[wave] = cnt;
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wave; ++w) off += wsum[w];
#pragma unroll 4
    for (int a0 = q0; a0 < q1; a0 += 64) {
        const int a = a0 + lane;
        const bool f = a < q1 && ids[a] == e;
        const unsigned long long m = __ballot(f);
        if (f) lists[(size_t)e * T + off + __popcll(m & ((1ull << lane) - 1ull))] = a;
        off += __popcll(m);
    }
    // the count is the only value another workgroup of this grid reads: an
    // agent-scope store writes it through to the device-coherent level and has
    // completed (vmcnt 0) before the arrival is counted; the lists are for the
    // next kernels
    if (tid == 0) {
        int c = 0;
        for (int w = 0; w < NWV; ++w) c += wsum[w];
        __hip_atomic_store(counts + e, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        is_last = __hip_atomic_fetch_add(&ctrl[CW_BUCKET_ARRIVE], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(E - 1);
    }
    __syncthreads();
    if (!is_last) return;
    // compact: slot order = expert id order, one expert per thread (E <= 512);
    // exclusive scans of (active, tiles) over the threads
    const int c = tid < E ? __hip_atomic_load(counts + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0;
    const int act = c > 0, til = (c + tile_m - 1) / tile_m;
    int ia = act, it = til;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int va = __shfl_up(ia, o, 64), vt = __shfl_up(it, o, 64);
        if (lane >= o) {
            ia += va;
            it += vt;
        }
    }
    if (lane == 63) {
        s_wa[wave] = ia;
        s_wt[wave] = it;
    }
    __syncthreads();
    int slot = ia - act, tl = it - til;
    for (int w = 0; w < wave; ++w) {
        slot += s_wa[w];
        tl += s_wt[w];
    }
    // tile map entry: expert | (tile index within the expert << 16)
    if (c > 0) {
        active[slot] = tid;
        tile_start[slot] = tl;
        for (int i = 0; i < til; ++i) tile_map[tl + i] = tid | (i << 16);
    }
    if (tid == 0) {
        int na = 0, nt = 0;
        for (int w = 0; w < NWV; ++w) {
            na += s_wa[w];
            nt += s_wt[w];
        }
        ctrl[CW_N_ACTIVE] = na;
        ctrl[CW_N_TILES] = nt;
        tile_start[na] = nt;
        ctrl[CW_BUCKET_ARRIVE] = 0u;    // ready for the next call
    }
}

// ---------------------------------------------------------------------------
// out[t][r] = sum_j w[t][j] * y[t*k + j][r], rank order, fp32.  With a latent
// layer the sum is y_lat and out is the latent buffer.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ wts, int T, int k,
                                                 int R, float* __restrict__ out) {
    // one float4 of out per thread (R is a multiple of 4)
    const int R4 = R / 4;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)T * R4) return;
    const long t = i / R4, r4 = i % R4;
    float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
        const float w = wts[t * k + j];
        const float4 v = reinterpret_cast<const float4*>(y + (t * k + j) * R)[r4];
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
    }
    reinterpret_cast<float4*>(out)[i] = acc;
}

// Canonical 36-byte Q8_1 blocks from the split activation layout.
__global__ __launch_bounds__(256) void k_tap_q8_1(ActPtr a, long rows, int K,
                                                  uint8_t* __restrict__ out) {
    const int nb = K / QK;
    const long blk = (long)blockIdx.x * 8 + threadIdx.x / 32;
    if (blk >= rows * nb) return;
    const int l = threadIdx.x % 32;
    const long r = blk / nb, b = blk % nb;
    uint8_t* o = out + blk * Q8_1_CANON;
    if (l < 4) o[l] = (uint8_t)(a.ds[blk] >> (8 * l));
    o[4 + l] = (uint8_t)a.q[r * K + b * QK + l];
}

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_quant_rows(const float* x, int rows, int K, ActPtr out, hipStream_t st) {
    long blocks = (long)rows * (K / QK);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((blocks + 7) / 8)), dim3(256), 0, st, x, rows,
                       K, out);
    return hipGetLastError();
}

hipError_t launch_router(const Dims& m, const WsLayout& w, char* ws, const float* x, int T,
                         const float* Wr, const float* br, const int32_t* groups, double* logits_tap,
                         ActPtr xq, bool* bucketed, hipStream_t st) {
    double* part = (double*)(ws + w.logit_part);
    const int S = w.S;
    const long qblocks = (long)T * (m.H / QK);
    const int qwg = (int)((qblocks + 7) / 8);
    int32_t* ids = (int32_t*)(ws + w.ids);
    float* wts = (float*)(ws + w.wts);
    SelectArgs a;
    a.part = part; a.S = S; a.T = T; a.E = m.E; a.k = m.k;
    a.bias = br; a.groups = groups; a.G = m.G; a.TG = m.TG; a.logits_tap = logits_tap;
    if (T <= ROUTE_DEC_MAX_T && m.E <= 512 && m.k <= 32) {
        hipLaunchKernelGGL(k_route_logits_dec, dim3(m.E + qwg), dim3(256), 0, st, x, Wr, T, m.H,
                           m.E, part, xq);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_route_select_dec, dim3(1), dim3(SEL_NT), 0, st, a, ids, wts,
                           (int32_t*)(ws + w.counts), (int32_t*)(ws + w.lists),
                           (uint32_t*)(ws + w.ctrl), (int32_t*)(ws + w.active));
        *bucketed = true;
        return hipGetLastError();
    }
    const RouterTile rt = router_tile(T);
    const int nl = ((T + rt.bm - 1) / rt.bm) * ((m.E + rt.bn - 1) / rt.bn) * S;
    const dim3 lg(nl + qwg);
    switch (rt.kind) {
        case 0:
            hipLaunchKernelGGL((k_route_logits_mf<1, 1, 1, 1, 4>), lg, dim3(256), 0, st, x, Wr, T,
                               m.H, m.E, S, part, nl, xq);
            break;
        case 1:
            hipLaunchKernelGGL((k_route_logits_mf<2, 1, 1, 1, 4>), lg, dim3(256), 0, st, x, Wr, T,
                               m.H, m.E, S, part, nl, xq);
            break;
        default:
            hipLaunchKernelGGL((k_route_logits_mf<2, 2, 2, 2, 1>), lg, dim3(256), 0, st, x, Wr, T,
                               m.H, m.E, S, part, nl, xq);
            break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int32_t* counts = (int32_t*)(ws + w.counts);
    int32_t* lists = (int32_t*)(ws + w.lists);
    uint32_t* ctrl = (uint32_t*)(ws + w.ctrl);
    int32_t* active = (int32_t*)(ws + w.active);
    if (T <= SMALL_TMAX && T * m.k <= 1024 && m.E <= 512) {
        hipLaunchKernelGGL((k_route_select_tok<true, 1024>), dim3(T), dim3(1024), 0, st, a, ids,
                           wts, counts, lists, ctrl, active);
        *bucketed = true;
    } else {
        hipLaunchKernelGGL((k_route_select_tok<false, 256>), dim3(T), dim3(256), 0, st, a, ids,
                           wts, counts, lists, ctrl, active);
        *bucketed = false;
    }
#undef MOE_MAXE
    return hipGetLastError();
}

hipError_t launch_bucket(const Dims& m, const WsLayout& w, char* ws, int T,
                         hipStream_t st) {
    hipLaunchKernelGGL(k_bucket, dim3(m.E), dim3(BK_NT), 0, st, (const int32_t*)(ws + w.ids), T * m.k,
                       T, m.E, GEMM_TILE_M, (int32_t*)(ws + w.counts), (int32_t*)(ws + w.lists),
                       (uint32_t*)(ws + w.ctrl), (int32_t*)(ws + w.active),
                       (int32_t*)(ws + w.tile_start), (int32_t*)(ws + w.tile_map));
    return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* wts, int T, int k, int R, float* out,
                          hipStream_t st) {
    long n = (long)T * (R / 4);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y, wts, T, k,
                       R, out);
    return hipGetLastError();
}

hipError_t launch_tap_q8_1(ActPtr a, long rows, int K, uint8_t* out, hipStream_t st) {
    long blocks = rows * (K / QK);
    if (blocks == 0 || !out) return hipSuccess;
    hipLaunchKernelGGL(k_tap_q8_1, dim3((unsigned)((blocks + 7) / 8)), dim3(256), 0, st, a, rows, K,
                       out);
    return hipGetLastError();
}

}  // namespace moe
