// Internal layout and launch interface of libmoe (host and device code of the
// library only; the public ABI is include/moe.h).
//
// Packed block matrix [rows][nblk] (any format): the codes of all rows first,
// row-major (32 bytes per Q8_0 block, 16 per Q4_0 or Q5_1 block, in element
// order for Q8_0 and in the canonical nibble-byte order otherwise; 128 per
// Q4_K / Q5_K super-block; 108 per Q3_K super-block), then each unit's side
// data, row-major [row][unit]: the binary16 d (2 bytes), for Q5_1 d, m and qh
// (8 bytes), for Q4_K / Q5_K the super-block header and scales (16, 48 bytes
// with Q5_K's qh), for Q3_K the binary16 d.  The canonical unit is [side
// data][codes] in every format except Q3_K, and the byte count is the same.
//
// Packed Q3_K super-block: eight 12-byte blocks, then the 12 canonical scale
// bytes.  Block b of 32: two little-endian words of 2-bit codes, word h holding
// element 16h + 4m + p at bits 8p + 2m (so (word >> 2m) & 0x03030303 gives
// elements 16h + 4m .. + 3 in its bytes), then one word of high bits, element
// 4m + p at bit 8p + m.
//
// Packed expert: gate/up matrix of 2F rows then the down matrix [Kout][F/32].
// The gate/up rows come in pairs of 32-row tiles: packed row fb*64 + r holds
// gate row fb*32 + r for r < 32 and up row fb*32 + r - 32 otherwise, so one
// 64-row slab carries everything SwiGLU needs for 32 outputs.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int QK = 32;              // elements per block
constexpr int Q8_1_CANON = 36;      // canonical Q8_1 block bytes

// Canonical units: unit_blocks(fmt) blocks of 32 (a K-quant super-block is one
// unit of 8).  Packed bytes per unit: codes, and side data.
inline bool kquant(int fmt) { return fmt == MOE_FMT_Q4_K || fmt == MOE_FMT_Q5_K || fmt == MOE_FMT_Q3_K; }
inline int unit_blocks(int fmt) { return kquant(fmt) ? 8 : 1; }
inline int unit_code_bytes(int fmt) {
    return fmt == MOE_FMT_Q8_0 ? 32 : fmt == MOE_FMT_Q3_K ? 108 : 16 * unit_blocks(fmt);
}
inline int unit_side_bytes(int fmt) {
    return fmt == MOE_FMT_Q5_1 ? 8 : fmt == MOE_FMT_Q4_K ? 16 : fmt == MOE_FMT_Q5_K ? 48 : 2;
}
inline int unit_bytes(int fmt) { return unit_code_bytes(fmt) + unit_side_bytes(fmt); }
struct MatLayout {                  // one packed block matrix
    int rows = 0, nblk = 0, fmt = MOE_FMT_Q8_0;
    size_t codes_off = 0;           // from the matrix base
    size_t scales_off = 0;
    size_t units() const { return (size_t)nblk / unit_blocks(fmt); }
    size_t row_code_bytes() const { return units() * unit_code_bytes(fmt); }
    size_t bytes() const { return (size_t)rows * units() * unit_bytes(fmt); }
};

inline MatLayout mat_layout(int rows, int nblk, int fmt) {
    MatLayout m;
    m.rows = rows;
    m.nblk = nblk;
    m.fmt = fmt;
    m.codes_off = 0;
    m.scales_off = (size_t)rows * m.row_code_bytes();
    return m;
}

struct Dims {
    int H, E, k, F, L, kin, kout, fmt, dfmt, G, TG, max_tokens;
    MatLayout gu, dn;               // offsets within one expert
    size_t dn_off;                  // byte offset of the down matrix in an expert
    size_t ts_off;                  // NVFP4: of the tensor scales (gate, up, down fp32), the
                                    // start of a 256-byte tail (packs stay 256-byte multiples); else 0
    size_t expert_bytes;
    MatLayout D, U;                 // latent dense projections
};

inline Dims make_dims(const moe_desc& d) {
    Dims m;
    m.H = d.hidden; m.E = d.n_experts; m.k = d.top_k; m.F = d.n_ff; m.L = d.latent;
    m.kin = d.latent ? d.latent : d.hidden;
    m.kout = m.kin;
    m.fmt = d.expert_fmt; m.dfmt = d.latent ? d.dense_fmt : MOE_FMT_Q8_0;
    m.G = d.n_groups; m.TG = d.topk_groups; m.max_tokens = d.max_tokens;
    m.gu = mat_layout(2 * m.F, m.kin / QK, m.fmt);
    m.dn = mat_layout(m.kout, m.F / QK, m.fmt);
    m.dn_off = m.gu.bytes();
    m.expert_bytes = m.gu.bytes() + m.dn.bytes();
    m.ts_off = 0;
    if (m.fmt == MOE_FMT_NVFP4) {
        m.ts_off = m.expert_bytes;
        m.expert_bytes += 256;
    }
    if (m.L) {
        m.D = mat_layout(m.L, m.H / QK, m.dfmt);
        m.U = mat_layout(m.H, m.L / QK, m.dfmt);
    }
    return m;
}

// Quantised activations in the workspace (Q8_1 content, split layout):
//   q  int8   [rows][K]
//   ds uint32 [rows][K/32]   binary16 d in the low half, binary16 s in the high half
//   sq int32  [rows][K/32]   sum of the block's q (exact)
struct ActPtr {
    int8_t* q;
    uint32_t* ds;
    int32_t* sq;
};

constexpr int ROUTER_SPLIT_MAX = 16;

// Control words at the start of the workspace.
enum CtrlWord {
    CW_BUCKET_ARRIVE = 0,   // arrivals of the per-expert bucketing workgroups
    CW_N_ACTIVE = 1,        // experts with at least one token
    CW_N_TILES = 2,         // token tiles over all active experts (grouped GEMM)
    CW_ROUTE_ARRIVE = 3,    // arrivals of the decode routing logits workgroups
    CW_COUNT = 64
};

struct WsLayout {
    size_t ctrl, logit_part, ids, wts, counts, active, tile_start, tile_map, lists;
    size_t xq_q, xq_ds, xq_sq;
    size_t z, zq_q, zq_ds, zq_sq;
    size_t hq_q, hq_ds, hq_sq;
    size_t y;
    size_t ylat, ylq_q, ylq_ds, ylq_sq;
    size_t dpart;                   // latent D partial rows of the few-token kernel
    size_t yarrive;                 // latent, per-token down: Q8_1(y_lat) block arrival
                                    // counters [T][L/32] (T <= DECODE_T), fixed offset and size
    size_t total;
    int T, S;                       // tokens, router K-splits
};

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr int DECODE_T = 8;  // largest T the few-token router logits kernel is sized for
// (and up to which the gate/up kernel can take its expert and tokens straight
// from the routing ids: T * k <= DECODE_T * 32 assignments)
// T up to this takes that kernel and leaves top-k, softmax and bucketing to the
// gate/up kernel's prologue, which routes a single token
constexpr int ROUTE_DEC_MAX_T = 1;
constexpr int MV_MAX_T = 32; // T up to this runs the matrix-vector expert kernels
constexpr int LAT_FUSED_Q_MAX_T = 1;  // latent: consumers quantise z / y_lat up to this T
// latent D and U at THIN_MIN_T..MV_MAX_T tokens: the few-token matrix-core kernel
constexpr int THIN_MIN_T = 2;

// K slices of the few-token dense kernel for a rows x (nb blocks) matrix:
// doubled while fewer than 256 workgroups (32-row tiles x slices) would run and
// a slice keeps at least 16 blocks (two per wave).
inline int thin_splits(int rows, int nb) {
    int S = 1;
    while ((rows / 32) * S < 256 && nb % (2 * S) == 0 && nb / (2 * S) >= 16) S *= 2;
    return S;
}
constexpr int GEMM_TILE_M = 64;  // token tile of the grouped matrix-core GEMM

// Upper bound of the token tiles over all active experts: every expert adds at
// most one partial tile.
inline int gemm_max_tiles(int T, int k, int E) {
    const long A = (long)T * k;
    return (int)((A + GEMM_TILE_M - 1) / GEMM_TILE_M + (A < E ? A : E));
}

// Router logits tile (tokens x experts per workgroup, K chunks split over its
// waves) by token count; `kind` selects the kernel instance.
struct RouterTile {
    int bm, bn, wk, kind;
};
inline RouterTile router_tile(int T) {
    if (T <= 16) return {16, 16, 4, 0};
    if (T <= 32) return {32, 16, 4, 1};
    return {64, 64, 1, 2};
}

inline int router_splits(const Dims& m, int T) {
    // K slices of the router logits: enough workgroups to spread the router
    // matrix (few tokens) or the token x expert tiles (many); the single-token
    // router computes whole logits
    if (T <= DECODE_T) return 1;
    const RouterTile rt = router_tile(T);
    const long tiles = (long)((T + rt.bm - 1) / rt.bm) * ((m.E + rt.bn - 1) / rt.bn);
    const int chunks = m.H / 16;
    int s = 1;
    while (s < ROUTER_SPLIT_MAX && tiles * s * 2 <= 512 && chunks % (s * 2 * rt.wk) == 0) s *= 2;
    return s;
}

inline WsLayout ws_layout(const Dims& m, int T) {
    WsLayout w;
    w.T = T;
    w.S = router_splits(m, T);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = al256(o + bytes); return r; };
    size_t A = (size_t)T * m.k;
    w.ctrl = take(sizeof(uint32_t) * CW_COUNT);
    // counters that must read zero at every call sit at the same offsets, with
    // the same sizes, for every layer and every T (a call with another layer or
    // T sharing the workspace may leave data anywhere else): the control words,
    // then the per-token down kernel's Q8_1(y_lat) block arrivals for DECODE_T
    // tokens of the widest latent row (8192)
    w.yarrive = take(sizeof(uint32_t) * DECODE_T * (8192 / QK));
    w.logit_part = take(sizeof(double) * w.S * T * m.E);
    w.ids = take(sizeof(int32_t) * A);
    w.wts = take(sizeof(float) * A);
    w.counts = take(sizeof(int32_t) * m.E);
    w.active = take(sizeof(int32_t) * m.E);
    w.tile_start = take(sizeof(int32_t) * (m.E + 1));
    w.tile_map = take(sizeof(int32_t) * gemm_max_tiles(T, m.k, m.E));
    w.lists = take(sizeof(int32_t) * (size_t)m.E * T);
    w.xq_q = take((size_t)T * m.H);
    w.xq_ds = take(sizeof(uint32_t) * T * (m.H / QK));
    w.xq_sq = take(sizeof(int32_t) * T * (m.H / QK));
    const size_t L = m.L ? m.L : QK;
    w.z = take(sizeof(float) * (size_t)T * L);
    w.zq_q = take((size_t)T * L);
    w.zq_ds = take(sizeof(uint32_t) * T * (L / QK));
    w.zq_sq = take(sizeof(int32_t) * T * (L / QK));
    w.hq_q = take(A * m.F);
    w.hq_ds = take(sizeof(uint32_t) * A * (m.F / QK));
    w.hq_sq = take(sizeof(int32_t) * A * (m.F / QK));
    w.y = take(sizeof(float) * A * m.kout);
    w.ylat = take(sizeof(float) * (size_t)T * L);
    w.ylq_q = take((size_t)T * L);
    w.ylq_ds = take(sizeof(uint32_t) * T * (L / QK));
    w.ylq_sq = take(sizeof(int32_t) * T * (L / QK));
    const bool thin = m.L && T >= THIN_MIN_T && T <= MV_MAX_T;
    w.dpart = take(thin ? sizeof(float) * thin_splits(m.L, m.H / QK) * (size_t)T * m.L : 0);
    w.total = o;
    return w;
}

}  // namespace moe
