// Kernel launchers of libmoe (host side of the HIP translation units).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "device.h"
#include "moe_internal.h"

namespace moe {

// Where the expert FFN kernels find routing and buckets.
struct Buckets {
    const uint32_t* ctrl;     // CW_N_ACTIVE, CW_N_TILES
    const int32_t* active;    // slot -> expert
    const int32_t* counts;    // [E] tokens per expert
    const int32_t* lists;     // [E][T] assignments a = t*k + j, token order
    const int32_t* tile_start;// [E+1] first token tile of each slot
    const int32_t* ids;       // [T][k]
    const float* wts;         // [T][k]
};

// Where the expert FFN kernels find expert e's pack: at base + e * stride (one
// array of E packs), or at table[e] when a table is given.  A table entry may
// point into device memory or into pinned host memory that is mapped into the
// device's address space (the kernels then read that expert over the bus).
struct ExpertSrc {
    const uint8_t* base = nullptr;
    const uint8_t* const* table = nullptr;
    ExpertSrc() = default;
    ExpertSrc(const uint8_t* b, const uint8_t* const* t = nullptr) : base(b), table(t) {}
};

// The entries are read as global-address-space pointers: a pointer loaded from
// memory is otherwise generic, and the loads through it (and through the other
// arm of the select) would become flat loads.
__device__ __forceinline__ const uint8_t* expert_pack(const uint8_t* base,
                                                      const uint8_t* const* table, int e,
                                                      size_t stride) {
    typedef __attribute__((address_space(1))) const uint8_t* gptr;
    if (!table) return base + (size_t)e * stride;
    return (const uint8_t*)static_cast<const gptr*>(static_cast<const void*>(table))[e];
}

// Events recorded by one kernel's own dispatch (its start and end), for timing
// that kernel alone; both null = a plain launch.
struct KEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                     const KEvents& ev, Args... args) {
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

// Router logits and selection parameters: part[s][t][e] are the logits'
// K-slice partials (S slices, summed in slice order), bias [E] or null, group
// labels [E] when G > 0, TG groups kept; logits_tap [T][E] or null.
constexpr int ROUTE_SMAX = 16;
struct SelectArgs {
    const double* part;
    int S, T, E, k;
    const float* bias;
    const int32_t* groups;
    int G, TG;
    double* logits_tap;
};

// Where a kernel that routes a single token itself publishes the result (the
// same content as the router and bucketing kernels write).
struct RouteOut {
    int32_t* ids;
    float* wts;
    int32_t* counts;
    int32_t* lists;
    uint32_t* ctrl;
    int32_t* active;
};

struct Taps {                 // device pointers, NULL = off
    float* h = nullptr;       // [A][F]
    float* y = nullptr;       // [A][Kout]
    int32_t* isum_gu = nullptr;
    int32_t* isum_dn = nullptr;
    int32_t* isum_d = nullptr;
    int32_t* isum_u = nullptr;
    int tap_tokens = 0;
};

hipError_t launch_quant_rows(const float* x, int rows, int K, ActPtr out, hipStream_t st);
// the same of x = sum_{s < S} part[s] (added in slice order; part[s] is
// [rows][K]), also stored to x when x is not null
hipError_t launch_quant_rows_sum(const float* part, int S, float* x, int rows, int K, ActPtr out,
                                 hipStream_t st);
// Q8_1(x) and the router logits; then, from two tokens on, top-k and softmax
// per token, and up to 32 tokens the bucketing too, unless `ids_only` (2 to
// DECODE_T tokens whose consumers read the ids: no buckets).  *done tells how
// far the launched kernels go; *sel receives the selection parameters (for a
// single token the gate/up kernel selects in its prologue from them).
// (ROUTE_DEFERRED: 2..DECODE_T tokens with defer_select, the logits only; the
// launch after the router selects, writing the ids as ROUTE_IDS does)
enum RouteDone { ROUTE_LOGITS, ROUTE_SELECTED, ROUTE_BUCKETED, ROUTE_IDS, ROUTE_DEFERRED };
hipError_t launch_router(const Dims& m, const WsLayout& w, char* ws, const float* x, int T,
                         const float* Wr, const float* br, const int32_t* groups, double* logits_tap,
                         ActPtr xq, bool ids_only, bool defer_select, RouteDone* done, SelectArgs* sel,
                         hipStream_t st);
// Per-expert assignment lists in token order, the active experts, and the
// token tiles (GEMM_TILE_M assignments) of each, numbered in tile_map.
hipError_t launch_bucket(const Dims& m, const WsLayout& w, char* ws, int T, hipStream_t st);
hipError_t launch_combine(const float* y, const float* wts, int T, int k, int R, float* out,
                          hipStream_t st);
// the same, and Q8_1 of out into outq (R a multiple of 32)
hipError_t launch_combine_q(const float* y, const float* wts, int T, int k, int R, float* out,
                            ActPtr outq, hipStream_t st);
hipError_t launch_tap_q8_1(ActPtr a, long rows, int K, uint8_t* out, hipStream_t st);

// True when the matrix-vector kernels have a configuration for rows of K
// elements of format fmt.
bool mv_config_ok(int K, int fmt, bool gate_up);

// Decode-path expert and dense kernels (matrix-vector, one pass over the weights).
// The expert input is either quantised rows (ain) or fp32 rows quantised inside
// the kernel (ain_f32, with `keep` receiving the Q8_1 blocks when non-null).
// route != null (T == 1 only): every workgroup selects the token's experts
// from the router logits in its prologue and workgroup 0 publishes ids,
// weights and buckets to *rout; b is then not read.  ids_direct (T == 1): an
// earlier launch routed the token, and slot j serves expert b.ids[j].
hipError_t launch_gate_up_mv(const Dims& m, int T, ExpertSrc experts, ActPtr ain,
                             const float* ain_f32, ActPtr keep, const Buckets& b, ActPtr hq,
                             const Taps& taps, hipStream_t st, const KEvents& ev = KEvents{},
                             const SelectArgs* route = nullptr, const RouteOut* rout = nullptr,
                             bool ids_slots = false, bool ids_direct = false);
// outq.q != null (array form): Q8_1 of out is written too, by 16-row tiles that
// hand each block to its second finisher through the counters `arrive` ([T][Kout/32],
// zero on entry and left zero), or by 32-row tiles when arrive is null
hipError_t launch_down_tok_mv(const Dims& m, int T, ExpertSrc experts, ActPtr hq,
                              const Buckets& b, float* out, const Taps& taps, hipStream_t st,
                              ActPtr outq = ActPtr{nullptr, nullptr, nullptr},
                              uint32_t* arrive = nullptr);
hipError_t launch_down_slot_mv(const Dims& m, int T, ExpertSrc experts, ActPtr hq,
                               const Buckets& b, float* y, const Taps& taps, hipStream_t st);
// route != null (T == 1, dense): one more workgroup selects the token's k
// experts from the router logits and publishes ids, weights and buckets to
// *rout, in parallel with the row tiles.
hipError_t launch_dense_mv(const MatLayout& W, const uint8_t* base, int T, ActPtr ain,
                           const float* ain_f32, ActPtr keep, float* out, int32_t* isum_tap,
                           int tap_tokens, hipStream_t st, const SelectArgs* route = nullptr,
                           const RouteOut* rout = nullptr, int k = 0);

// Many-token path: grouped int8 matrix-core GEMM over the token tiles that the
// bucketing kernel numbered in tile_map (tiles of GEMM_TILE_M assignments).
bool mfma_config_ok(int rows, int K);
hipError_t launch_gate_up_mfma(const Dims& m, int T, ExpertSrc experts, ActPtr ain,
                               const Buckets& b, const int32_t* tile_map, ActPtr hq,
                               const Taps& taps, hipStream_t st, const KEvents& ev = KEvents{});
hipError_t launch_down_mfma(const Dims& m, int T, ExpertSrc experts, ActPtr hq,
                            const Buckets& b, const int32_t* tile_map, float* y, const Taps& taps,
                            hipStream_t st);
hipError_t launch_dense_mfma(const MatLayout& W, const uint8_t* base, int T, ActPtr ain, float* out,
                             int32_t* isum_tap, int tap_tokens, hipStream_t st);

// Few-token dense projection (T <= 32, Q8_0 or Q4_0, rows a multiple of 32):
// out[s][t][r] over S K-slices (S divides the blocks per row; thin_splits).
bool dense_thin_ok(const MatLayout& W, int T);
// route != null: T more workgroups select each token's k experts from its
// router logits (S = 1) and write ids / wts [T][k], in parallel with the tiles.
hipError_t launch_dense_thin(const MatLayout& W, const uint8_t* base, int T, ActPtr ain, float* out,
                             int S, int32_t* isum_tap, int tap_tokens, hipStream_t st,
                             const SelectArgs* route = nullptr, int32_t* ids = nullptr,
                             float* wts = nullptr);

// Expert-address table: fill entries 0..E-1 with base + e * stride, or set
// u.n (at most TABLE_UPDATE_MAX) entries, stream-ordered.
constexpr int TABLE_UPDATE_MAX = 64;
struct TableUpdate {
    int n;
    int expert[TABLE_UPDATE_MAX];
    const uint8_t* addr[TABLE_UPDATE_MAX];
};
hipError_t launch_table_fill(const uint8_t** table, int E, const uint8_t* base, size_t stride,
                             hipStream_t st);
hipError_t launch_table_set(const uint8_t** table, const TableUpdate& u, hipStream_t st);

}  // namespace moe
