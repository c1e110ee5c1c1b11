// Dense projections of a few tokens (latent D and U at 2..32 tokens) on the
// int8 matrix cores.
//
// Latent MoE (edge0-strata README, section "Changes from upstream Strata"):
// z = D . Q8_1(x) before the experts and out = U . Q8_1(y_lat) after them,
// with D and U Q8_0 (or Q4_0) block matrices; each block's int32 sum against
// the Q8_1 row is scaled by d_w * d_a.
//
// At a few tokens the matrix is read once and the arithmetic is small, so the
// kernel is laid out for memory-level parallelism rather than reuse:
//   * a workgroup owns 32 weight rows and one of S slices of K; its TH_NW waves
//     split the slice's blocks, and every wave issues the loads of up to TH_UB
//     blocks before its first product;
//   * one v_mfma_i32_32x32x32_i8 per block gives the exact block sums of the 32
//     rows against all tokens at once (token columns past T repeat the last
//     token and are dropped), and an f16 outer product gives the 32 x 32 scale
//     products d_w * d_a, exact in fp32, as in the many-token GEMM;
//   * the waves' 32 x 32 fp32 tiles are added in wave order through LDS; with
//     S > 1 slice s writes partial rows out[s][t][r], which the Q8_1
//     quantisation of z adds in slice order, so the result does not depend on
//     timing.
// Each workgroup row-slice is read by exactly one wave: no re-reads to save, so
// the activations (at most 32 x 7168 bytes, cache-resident) are the only data
// shared between workgroups.
#include "kernels.h"
#include "mfma_ops.h"
#include "select.h"

namespace moe {

constexpr int TH_NW = 8;    // waves per workgroup
constexpr int TH_UB = 8;    // blocks per load batch of a wave

struct ThinArgs {
    const uint8_t* codes;       // [rows][nb] blocks of codes (32 bytes Q8_0, 16 Q4_0)
    const uint16_t* scl;        // [rows][nb] binary16 d
    int rows, nb, T, S;         // weight rows, blocks per row, tokens (<= 32), K slices
    ActPtr ain;                 // [T][nb * 32] Q8_1 activation rows
    float* out;                 // [S][T][rows]
    int32_t* tap_isum;          // [T][rows][nb] block sums of tokens < tap_tokens, or null
    int tap_tokens;
    // SEL: workgroups 0..T-1 select token t's experts from its whole router
    // logits (route.part + t * E) and write ids / wts [T][k] in rank order; the
    // tiles are the workgroups after them
    SelectArgs route;
    int32_t* ids;
    float* wts;
};

// (SEL: an instance of its own, so that the tiles of the plain instance keep
// their registers)
template <int FMT, bool TAP, bool SEL = false>
__global__ __launch_bounds__(TH_NW * 64) void k_dense_thin(ThinArgs A) {
    constexpr bool Q4 = FMT == MOE_FMT_Q4_0;
    constexpr int CB = Q4 ? 16 : 32;        // code bytes per block
    // [wave][lane][result i], padded so that both the writes (lane-major) and
    // the reads (32 rows of one token) spread over the banks
    __shared__ __align__(16) float red[TH_NW][64][17];
    static_assert(sizeof(red) >= sizeof(RouteLds), "the selection's LDS lives in red");

    int bid = blockIdx.x;
    if constexpr (SEL) {
        if (bid < A.T) {
            // one token's selection, in parallel with the tiles
            const int t = bid;
            SelectArgs sa = A.route;
            sa.part += (size_t)t * sa.E;
            if (sa.logits_tap) sa.logits_tap += (size_t)t * sa.E;
            RouteLds& S = *reinterpret_cast<RouteLds*>(&red[0][0][0]);
            float w = 0.0f;
            select_wg<TH_NW * 64>(sa, S, true, &w);
            if ((int)threadIdx.x < sa.k) {
                A.ids[t * sa.k + threadIdx.x] = S.sel[threadIdx.x];
                A.wts[t * sa.k + threadIdx.x] = w;
            }
            return;
        }
        bid -= A.T;
    }

    const int ntile = A.rows / 32;
    const int tile = bid % ntile, s = bid / ntile;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int nb = A.nb, bps = nb / A.S;
    const int bpw = (bps + TH_NW - 1) / TH_NW;
    const int b0 = s * bps + min(wave * bpw, bps);
    const int b1 = s * bps + min(wave * bpw + bpw, bps);

    // lane operands: weight row tile*32 + l32, K half `half` of each block;
    // token column l32 (clamped to the last token)
    const int row = tile * 32 + l32;
    const int tok = min(l32, A.T - 1);
    const uint8_t* wrow = A.codes + (size_t)row * nb * CB + (Q4 ? 0 : half * 16);
    const uint16_t* wsc = A.scl + (size_t)row * nb;
    const int8_t* arow = A.ain.q + (size_t)tok * nb * QK + half * 16;
    const uint32_t* ads = A.ain.ds + (size_t)tok * nb;

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    for (int bb = b0; bb < b1; bb += TH_UB) {
        v4i wq[TH_UB], aq[TH_UB];
        uint32_t dw[TH_UB], da[TH_UB];
#pragma unroll
        for (int u = 0; u < TH_UB; ++u) {
            const int b = min(bb + u, b1 - 1);   // past the wave's blocks: re-read the last (unused)
            wq[u] = ld16(wrow + (size_t)b * CB);
            aq[u] = ld16(arow + (size_t)b * QK);
            dw[u] = wsc[b];
            da[u] = ads[b];
        }
#pragma unroll
        for (int u = 0; u < TH_UB; ++u) {
            if (bb + u >= b1) break;
            v4i a = wq[u];
            if constexpr (Q4) {
                // elements 0..15 are the low nibbles, 16..31 the high ones
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = (uint32_t)a[d];
                    a[d] = (int)q4_widen(half ? (x >> 4) & 0x0F0F0F0Fu : x & 0x0F0F0F0Fu);
                }
            }
            const v16i is = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, aq[u], v16i{}, 0, 0, 0);
            const v16f sc = scale_mfma(scale_op(half ? 0u : dw[u]), scale_op(half ? 0u : (da[u] & 0xFFFFu)));
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf((float)is[i], sc[i], acc[i]);
            if constexpr (TAP) {
                if (A.tap_isum && l32 < A.T && l32 < A.tap_tokens) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = tile * 32 + mf_row_of(i, half);
                        A.tap_isum[((size_t)l32 * A.rows + r) * nb + bb + u] = is[i];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][lane][i] = acc[i];
    __syncthreads();
    // thread -> (token c, row r of the tile); consecutive threads store
    // consecutive rows of one token
    for (int e = threadIdx.x; e < 32 * 32; e += TH_NW * 64) {
        const int c = e >> 5, r = e & 31;
        if (c >= A.T) break;
        const int ln = c + 32 * ((r >> 2) & 1), i = (r >> 3) * 4 + (r & 3);
        float v = red[0][ln][i];
#pragma unroll
        for (int w = 1; w < TH_NW; ++w) v += red[w][ln][i];
        A.out[((size_t)s * A.T + c) * A.rows + tile * 32 + r] = v;
    }
}

bool dense_thin_ok(const MatLayout& W, int T) {
    return T >= 1 && T <= 32 && W.rows % 32 == 0 && (W.fmt == MOE_FMT_Q8_0 || W.fmt == MOE_FMT_Q4_0);
}

hipError_t launch_dense_thin(const MatLayout& W, const uint8_t* base, int T, ActPtr ain, float* out,
                             int S, int32_t* isum_tap, int tap_tokens, hipStream_t st,
                             const SelectArgs* route, int32_t* ids, float* wts) {
    if (!dense_thin_ok(W, T) || S < 1 || W.nblk % S) return hipErrorInvalidValue;
    ThinArgs a{};
    if (route) {
        // whole logits of T tokens, within the selection's limits
        if (!ids || !wts || route->S != 1 || route->T != T || route->E > 512 || route->k > 32 ||
            route->G > 64)
            return hipErrorInvalidValue;
        a.route = *route;
        a.ids = ids;
        a.wts = wts;
    }
    a.codes = base + W.codes_off;
    a.scl = reinterpret_cast<const uint16_t*>(base + W.scales_off);
    a.rows = W.rows; a.nb = W.nblk; a.T = T; a.S = S;
    a.ain = ain;
    a.out = out;
    a.tap_isum = isum_tap;
    a.tap_tokens = tap_tokens;
    const dim3 grid((unsigned)((W.rows / 32) * S + (route ? T : 0))), block(TH_NW * 64);
    const bool tap = isum_tap != nullptr;
    if (route) {
        if (W.fmt == MOE_FMT_Q4_0) {
            if (tap)
                hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q4_0, true, true>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q4_0, false, true>), grid, block, 0, st, a);
        } else {
            if (tap)
                hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q8_0, true, true>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q8_0, false, true>), grid, block, 0, st, a);
        }
        return hipGetLastError();
    }
    if (W.fmt == MOE_FMT_Q4_0) {
        if (tap)
            hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q4_0, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q4_0, false>), grid, block, 0, st, a);
    } else {
        if (tap)
            hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q8_0, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((k_dense_thin<MOE_FMT_Q8_0, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace moe
