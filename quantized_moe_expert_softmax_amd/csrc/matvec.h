// Matrix-vector path of libmoe: the arguments of its kernels and the per-format
// launch functions that the launchers (matvec.hip) call.  The kernels themselves
// (matvec_kern.h) are instantiated one format per translation unit (mv_*.hip).
#pragma once
#include "kernels.h"
#include "select.h"

namespace moe {

// LDS bytes of n staged rows of K elements (codes, d, sums), 16-byte aligned.
__host__ __device__ constexpr size_t stage_bytes(int n, int K) {
    return (size_t)n * K + 2 * (size_t)n * (K / QK) * 4;
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU + Q8_1.  Workgroup = (slot, fb): the 64-row slab of gate
// rows fb*32.. and up rows fb*32.. of the slot's expert, for every token routed
// to it.  Output: hq rows a = t*k + j, block fb.
struct GUArgs {
    const uint8_t* experts;
    const uint8_t* const* etab;   // expert pack addresses, or null (experts + e * eb)
    size_t eb, gu_scales_off;
    int K, F, k, T, tch;
    ActPtr ain;           // quantised expert input rows [T][K], or
    const float* ain_f32; // fp32 rows [T][K] quantised in the prologue (latent z)
    ActPtr keep;          // where the prologue also stores Q8_1(z) (taps), q == nullptr: off
    Buckets b;
    ActPtr hq;
    Taps taps;
    SelectArgs route;     // route.part != null: one token, routed in the prologue
    RouteOut rout;
    int ids_slots;        // 1: the slots come from b.ids (T * k <= DECODE_T * 32), not buckets
    int ids_direct;       // 1: one token routed by an earlier launch: slot j serves b.ids[j]
    size_t ts_off;        // NVFP4: the tensor scales (gate, up fp32) in an expert pack; else 0
};


// ---------------------------------------------------------------------------
// Rows kernel: out[s][r] = W_g[r] . act[s] for a tile of rows of a block matrix.
// Expert mode (b.ctrl != nullptr): group = slot, W_g = the down matrix of expert
// active[slot], act/out rows = the expert's assignments (hq rows).  Dense mode:
// one matrix, act/out rows = tokens 0..T-1 (D on Q8_1(x), U on Q8_1(y_lat)).
struct RowsArgs {
    const uint8_t* base;
    size_t group_stride, codes_off, scales_off;
    const uint8_t* const* etab;   // expert mode: pack addresses, or null (base + e * stride)
    int rows, K, T, rt, tch;
    Buckets b;                 // b.ctrl == nullptr: dense mode
    ActPtr ain;                // quantised act rows, or
    const float* ain_f32;      // fp32 act rows quantised in the prologue
    ActPtr keep;               // Q8_1 of the fp32 rows, stored for taps (q == nullptr: off)
    float* out;                // [act row][rows]
    int tap_div;               // token of act row s = s / tap_div
    int32_t* isum_tap;         // [act row][rows][K/32]
    int tap_tokens;
    size_t ts_off;             // expert mode, NVFP4: the down tensor scale in a pack; else 0
    // dense mode, one token, route.part != null: workgroup 0 selects the token's
    // k experts from the router logits and publishes the routing to rout (as
    // the gate/up prologue does); the row tiles are workgroups 1..
    SelectArgs route;
    RouteOut rout;
    int k;
};

// ---------------------------------------------------------------------------
// Down projection with the combine fused, one workgroup per (token, 16-row
// tile); wave j computes rank j's expert rows, then the tile is combined in
// rank order: out[t][r] = sum_j w[t][j] * (W_down[e_j][r] . hq[t*k+j]).  With
// outq, 32-row tiles, and each tile's Q8_1 block of out is written as well (the
// latent layer's y_lat, quantised once for the U projection).
struct DownTokArgs {
    const uint8_t* experts;
    size_t eb, dn_off, dn_scales_off;
    int F, Kout, k;
    ActPtr hq;
    Buckets b;
    float* out;              // [T][Kout]: the layer output, or y_lat for a latent layer
    Taps taps;
    const uint8_t* const* etab;   // expert pack addresses, or null (experts + e * eb)
    ActPtr outq;                  // q != null: also Q8_1 of out (not with etab)
    uint32_t* arrive;             // with outq: [T][Kout/32] block arrival counters (16-row
                                  // tiles, zero on entry and on exit); null: 32-row tiles
    size_t ts_off;                // NVFP4: the down tensor scale in an expert pack; else 0
};

constexpr int DT_RT = 16;    // output rows per workgroup
// output rows per workgroup of a latent layer's one-token down projection (the
// Q8_1(y_lat) blocks handed over by arrival counters): 1280 or 1792 latent rows
// give 320 or 448 workgroups instead of 80 or 112 with 16-row tiles
constexpr int DT_RT_ONE = 4;
constexpr int DT_NW = 8;     // waves per workgroup (ranks in parallel)
constexpr int DT_KMAX = 32;  // largest top_k

constexpr int ROWS_NW = 4;   // waves per rows workgroup (8 spill the K-quant down rows)

// waves per gate/up workgroup: 8 lanes per row cover the 64-row slab in one
// pass with 8 waves; Q8_0's wider rows use 4 waves and several passes.  The
// other formats use 8 waves on every row width: their unpack needs the extra
// waves to hide its latency, and the 8-wave bound (two waves per SIMD) leaves
// 256 registers where the 4-wave bound (three) leaves 170 and Q4_0 / Q5_1
// spilled (measured: Q5_K decode gate/up 44.6 -> 30.9 us, Q4_K 28.3 -> 26.0)
__host__ __device__ constexpr int gu_waves_c(int lpr, int fmt) {
    return lpr == 8 || fmt != MOE_FMT_Q8_0 ? 8 : 4;
}
inline int gu_waves(int lpr, int fmt) { return gu_waves_c(lpr, fmt); }

// Launch one instance by (lanes per row, 16-byte chunks per lane); defined and
// instantiated for every format in mv_*.hip (down_tok_fmt for Q8_0, Q4_0, Q5_1,
// down_tok_kq_fmt for the K-quants).
template <int FMT, bool TAP>
hipError_t gate_up_fmt(int lpr, int cpl, dim3 grid, size_t lds, const GUArgs& a, hipStream_t st,
                       const KEvents& ev);
template <int FMT, bool TAP>
hipError_t rows_fmt(int lpr, int cpl, dim3 grid, size_t lds, const RowsArgs& a, hipStream_t st);
template <int FMT, bool TAP>
hipError_t down_tok_fmt(int lpr, int cpl, int T, const DownTokArgs& a, hipStream_t st);
template <int FMT, bool TAP>
hipError_t down_tok_kq_fmt(int lpr, int cpl, int T, size_t lds, const DownTokArgs& a, hipStream_t st);

}  // namespace moe
