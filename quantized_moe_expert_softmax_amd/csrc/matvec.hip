// Launchers of the matrix-vector path: configuration (lanes per row, chunks per
// lane, staged tokens, rows per workgroup) from the row length and format, and
// the dispatch to the per-format instances.
#include <algorithm>

#include "matvec.h"

namespace moe {

static bool pick(int nch, int& lpr, int& cpl) {
    for (int c = 8; c >= 1; --c)
        for (int l = 8; l <= 64; l *= 2)
            if (l * c == nch) { lpr = l; cpl = c; return true; }
    if (nch <= 512) { lpr = 64; cpl = (nch + 63) / 64; return true; }
    return false;
}

static int nchunks(int K, int fmt) { return fmt == MOE_FMT_Q8_0 ? K / 16 : K / 32; }

// gate/up: two passes of weights live at once, so at most 5 chunks per lane
// (4 preferred: whole 4 KB rows per wave at K = 4096)
static bool pick_gu(int nch, int& lpr, int& cpl) {
    for (int c = 4; c >= 1; --c)
        for (int l = 64; l >= 8; l /= 2)
            if (l * c == nch) { lpr = l; cpl = c; return true; }
    for (int c = 5; c <= 8; ++c)             // one pass of 8-lane rows: one buffer
        if (8 * c == nch) { lpr = 8; cpl = c; return true; }
    for (int l = 64; l >= 16; l /= 2)
        for (int c = 5; c <= 8; ++c)
            if (l * c == nch) { lpr = l; cpl = c; return true; }
    return pick(nch, lpr, cpl);
}

// gate/up of the nibble and K-quant formats: two chunks per lane over the
// narrowest lane group that covers the row (64 lanes at most).  Their unpack
// chains are long, and few chunks per lane put more rows in flight per wave.
// Measured at T = 1, us per layer against pick_gu's choice: Q5_1 38.4 -> 32.7,
// Q3_K 36.0 -> 29.9, Q5_K 44.6 -> 42.6, Q4_K 38.2 -> 37.5; latent Q3_K (56
// chunks) 51.9 -> 46.7 with 32 x 2, 47.3 with 64 x 1; Q3_K T = 6 133.7 ->
// 110.7.  Q8_0 rows keep pick_gu (32 x 8 instead of 64 x 4: 40.3 -> 64.3).
static bool pick_gu_fmt(int nch, int fmt, int& lpr, int& cpl) {
    if (fmt == MOE_FMT_Q8_0) return pick_gu(nch, lpr, cpl);
    int l = 8;
    while (l < 64 && l * 2 < nch) l *= 2;
    const int c = (nch + l - 1) / l;
    if (c > 8) return false;
    lpr = l;
    cpl = c;
    return true;
}

// staged tokens per chunk: about 32 KB of codes
static int pick_tch(int K) { return std::max(4, std::min(16, 32768 / K)); }

// rows kernels: the gate/up choice of at most four chunks per lane.  More
// chunks per lane spilled for the nibble formats (unpacked codes and side data
// in registers: K-quant down at F = 1536, Q4_0 D at H = 4096), and for Q8_0
// fewer rows per workgroup give the short latent D more workgroups (1280 rows
// at K = 4096: 320 workgroups instead of 160; latent_q8 T = 1 41.1 -> 40.6 us)
static bool pick_rows(int nch, int& lpr, int& cpl) { return pick_gu(nch, lpr, cpl); }

bool mv_config_ok(int K, int fmt, bool gate_up) {
    int l, c;
    if (gate_up ? !pick_gu_fmt(nchunks(K, fmt), fmt, l, c) : !pick_rows(nchunks(K, fmt), l, c))
        return false;
    return c >= 1 && c <= 8 && (l == 8 || l == 16 || l == 32 || l == 64);
}

hipError_t launch_gate_up_mv(const Dims& m, int T, ExpertSrc experts, ActPtr ain,
                             const float* ain_f32, ActPtr keep, const Buckets& b, ActPtr hq,
                             const Taps& taps, hipStream_t st, const KEvents& ev,
                             const SelectArgs* route, const RouteOut* rout, bool ids_slots,
                             bool ids_direct) {
    int lpr, cpl;
    if (!pick_gu_fmt(nchunks(m.kin, m.fmt), m.fmt, lpr, cpl)) return hipErrorInvalidConfiguration;
    if (64 % (gu_waves(lpr, m.fmt) * (64 / lpr))) return hipErrorInvalidConfiguration;
    GUArgs a;
    a.experts = experts.base;
    a.etab = experts.table;
    a.eb = m.expert_bytes;
    a.gu_scales_off = m.gu.scales_off;
    a.K = m.kin; a.F = m.F; a.k = m.k; a.T = T;
    // (no expert holds more than T tokens: staging room for min(T, chunk))
    a.tch = std::min(pick_tch(m.kin), std::max(T, 1));
    a.ain = ain; a.ain_f32 = ain_f32; a.keep = keep;
    a.b = b; a.hq = hq; a.taps = taps;
    a.ts_off = m.ts_off;
    size_t lds = stage_bytes(a.tch, a.K) + (size_t)a.tch * 64 * 4 + (size_t)a.tch * 8;
    a.route = SelectArgs{};
    a.rout = RouteOut{};
    a.ids_slots = 0;
    a.ids_direct = 0;
    if (ids_direct) {
        // one token whose k ids an earlier launch wrote to b.ids
        if (route || ids_slots || T != 1 || !b.ids) return hipErrorInvalidValue;
        a.ids_direct = 1;
    }
    if (ids_slots) {
        // every assignment id is held by one thread of the (at least 256-thread) workgroup
        // (and the expert ids fit the prologue's two per thread)
        if (route || T * m.k > DECODE_T * 32 || !b.ids || m.E > 2 * 64 * gu_waves(lpr, m.fmt))
            return hipErrorInvalidValue;
        a.ids_slots = 1;
    }
    if (route) {
        // the prologue's selection: one token, its whole logits (S = 1), and
        // its LDS after the staging area
        if (T != 1 || !rout || route->S != 1 || route->T != 1 || route->E > 512 || route->k > 32 ||
            route->G > 64)
            return hipErrorInvalidValue;
        a.route = *route;
        a.rout = *rout;
        lds = ((lds + 15) & ~(size_t)15) + sizeof(RouteLds);
    }
    int slots = std::min(m.E, T * m.k);
    dim3 grid(slots * (m.F / QK));
    bool tap = taps.h || taps.isum_gu;
    if (m.fmt == MOE_FMT_Q4_0)
        return tap ? gate_up_fmt<MOE_FMT_Q4_0, true>(lpr, cpl, grid, lds, a, st, ev)
                   : gate_up_fmt<MOE_FMT_Q4_0, false>(lpr, cpl, grid, lds, a, st, ev);
    if (m.fmt == MOE_FMT_Q5_1)
        return tap ? gate_up_fmt<MOE_FMT_Q5_1, true>(lpr, cpl, grid, lds, a, st, ev)
                   : gate_up_fmt<MOE_FMT_Q5_1, false>(lpr, cpl, grid, lds, a, st, ev);
    if (m.fmt == MOE_FMT_Q4_K)
        return tap ? gate_up_fmt<MOE_FMT_Q4_K, true>(lpr, cpl, grid, lds, a, st, ev)
                   : gate_up_fmt<MOE_FMT_Q4_K, false>(lpr, cpl, grid, lds, a, st, ev);
    if (m.fmt == MOE_FMT_Q5_K)
        return tap ? gate_up_fmt<MOE_FMT_Q5_K, true>(lpr, cpl, grid, lds, a, st, ev)
                   : gate_up_fmt<MOE_FMT_Q5_K, false>(lpr, cpl, grid, lds, a, st, ev);
    if (m.fmt == MOE_FMT_Q3_K)
        return tap ? gate_up_fmt<MOE_FMT_Q3_K, true>(lpr, cpl, grid, lds, a, st, ev)
                   : gate_up_fmt<MOE_FMT_Q3_K, false>(lpr, cpl, grid, lds, a, st, ev);
    if (m.fmt == MOE_FMT_NVFP4)
        return tap ? gate_up_fmt<MOE_FMT_NVFP4, true>(lpr, cpl, grid, lds, a, st, ev)
                   : gate_up_fmt<MOE_FMT_NVFP4, false>(lpr, cpl, grid, lds, a, st, ev);
    return tap ? gate_up_fmt<MOE_FMT_Q8_0, true>(lpr, cpl, grid, lds, a, st, ev)
               : gate_up_fmt<MOE_FMT_Q8_0, false>(lpr, cpl, grid, lds, a, st, ev);
}

// rows per workgroup: a multiple of the rows one pass covers, dividing `rows`,
// small enough to give about 512 workgroups
static int pick_rt(int rows, int groups, int rpp) {
    int rt = rpp;
    while (rt * 2 <= 64 && rows % (rt * 2) == 0 && (long)groups * (rows / (rt * 2)) >= 512) rt *= 2;
    return rt;
}

static hipError_t rows_dispatch(int fmt, int groups, RowsArgs& a, hipStream_t st) {
    int lpr, cpl;
    if (!pick_rows(nchunks(a.K, fmt), lpr, cpl)) return hipErrorInvalidConfiguration;
    const int rpp = ROWS_NW * (64 / lpr);
    if (a.rows % rpp) return hipErrorInvalidConfiguration;
    a.rt = pick_rt(a.rows, groups, rpp);
    a.tch = std::min(pick_tch(a.K), std::max(a.T, 1));
    size_t lds = stage_bytes(a.tch, a.K) + (size_t)a.tch * 4;
    dim3 grid(groups * (a.rows / a.rt));
    if (a.route.part) {
        // one more workgroup, the selection (its LDS is the selection's only)
        grid.x += 1;
        lds = std::max(lds, sizeof(RouteLds));
    }
    bool tap = a.isum_tap != nullptr;
    if (fmt == MOE_FMT_Q4_0)
        return tap ? rows_fmt<MOE_FMT_Q4_0, true>(lpr, cpl, grid, lds, a, st)
                   : rows_fmt<MOE_FMT_Q4_0, false>(lpr, cpl, grid, lds, a, st);
    if (fmt == MOE_FMT_Q5_1)
        return tap ? rows_fmt<MOE_FMT_Q5_1, true>(lpr, cpl, grid, lds, a, st)
                   : rows_fmt<MOE_FMT_Q5_1, false>(lpr, cpl, grid, lds, a, st);
    if (fmt == MOE_FMT_Q4_K)
        return tap ? rows_fmt<MOE_FMT_Q4_K, true>(lpr, cpl, grid, lds, a, st)
                   : rows_fmt<MOE_FMT_Q4_K, false>(lpr, cpl, grid, lds, a, st);
    if (fmt == MOE_FMT_Q5_K)
        return tap ? rows_fmt<MOE_FMT_Q5_K, true>(lpr, cpl, grid, lds, a, st)
                   : rows_fmt<MOE_FMT_Q5_K, false>(lpr, cpl, grid, lds, a, st);
    if (fmt == MOE_FMT_Q3_K)
        return tap ? rows_fmt<MOE_FMT_Q3_K, true>(lpr, cpl, grid, lds, a, st)
                   : rows_fmt<MOE_FMT_Q3_K, false>(lpr, cpl, grid, lds, a, st);
    if (fmt == MOE_FMT_NVFP4)
        return tap ? rows_fmt<MOE_FMT_NVFP4, true>(lpr, cpl, grid, lds, a, st)
                   : rows_fmt<MOE_FMT_NVFP4, false>(lpr, cpl, grid, lds, a, st);
    return tap ? rows_fmt<MOE_FMT_Q8_0, true>(lpr, cpl, grid, lds, a, st)
               : rows_fmt<MOE_FMT_Q8_0, false>(lpr, cpl, grid, lds, a, st);
}

hipError_t launch_down_slot_mv(const Dims& m, int T, ExpertSrc experts, ActPtr hq,
                               const Buckets& b, float* y, const Taps& taps, hipStream_t st) {
    RowsArgs a{};
    a.base = experts.base;
    a.etab = experts.table;
    a.group_stride = m.expert_bytes;
    a.codes_off = m.dn_off + m.dn.codes_off;
    a.scales_off = m.dn_off + m.dn.scales_off;
    a.rows = m.kout; a.K = m.F; a.T = T;
    a.b = b; a.ain = hq; a.ain_f32 = nullptr; a.keep = ActPtr{}; a.out = y;
    a.tap_div = m.k; a.isum_tap = taps.isum_dn; a.tap_tokens = taps.tap_tokens;
    a.ts_off = m.ts_off ? m.ts_off + 8 : 0;     // NVFP4: the down tensor scale
    return rows_dispatch(m.fmt, std::min(m.E, T * m.k), a, st);
}

hipError_t launch_dense_mv(const MatLayout& W, const uint8_t* base, int T, ActPtr ain,
                           const float* ain_f32, ActPtr keep, float* out, int32_t* isum_tap,
                           int tap_tokens, hipStream_t st, const SelectArgs* route,
                           const RouteOut* rout, int k) {
    RowsArgs a{};
    if (route) {
        // one token, its whole logits (S = 1), within the selection's limits
        if (T != 1 || !rout || route->S != 1 || route->T != 1 || route->E > 512 || route->k > 32 ||
            route->G > 64 || route->k != k)
            return hipErrorInvalidValue;
        a.route = *route;
        a.rout = *rout;
        a.k = k;
    }
    a.base = base;
    a.group_stride = 0;
    a.codes_off = W.codes_off;
    a.scales_off = W.scales_off;
    a.rows = W.rows; a.K = W.nblk * QK; a.T = T;
    a.b = Buckets{};
    a.ain = ain; a.ain_f32 = ain_f32; a.keep = keep; a.out = out;
    a.tap_div = 1; a.isum_tap = isum_tap; a.tap_tokens = tap_tokens;
    return rows_dispatch(W.fmt, 1, a, st);
}

hipError_t launch_down_tok_mv(const Dims& m, int T, ExpertSrc experts, ActPtr hq,
                              const Buckets& b, float* out, const Taps& taps, hipStream_t st,
                              ActPtr outq, uint32_t* arrive) {
    const bool kq = kquant(m.fmt);
    if (outq.q && (experts.table || m.kout % QK)) return hipErrorInvalidValue;
    int lpr, cpl;
    // (the K-quant dots keep a whole super-block's side data per chunk: at most
    // four chunks per lane, as in the rows kernel).  The others take three
    // chunks per lane where that splits the row exactly (measured, us per
    // layer: Q8_0 at F = 1536, 32 x 3 against 16 x 6: T = 6 163.0 -> 159.4, T = 1
    // unchanged; Q5_1, 16 x 3 against 8 x 6: T = 1 32.9 -> 32.2)
    const int nch = nchunks(m.F, m.fmt);
    // one token of a latent layer (Q8_1(y_lat) through arrival counters): rows of
    // at least 16 lanes, so that DT_RT_ONE-row tiles hold whole passes
    bool one = false;
    if (outq.q && arrive) {
        for (int l = 16; l <= 64 && !one; l *= 2)
            if (nch % l == 0 && nch / l <= (kq ? 4 : 8)) { lpr = l; cpl = nch / l; one = true; }
    }
    if (!one) {
        if (kq) {
            if (!pick_rows(nch, lpr, cpl)) return hipErrorInvalidConfiguration;
        } else if (nch % 3 == 0 && (nch / 3 == 8 || nch / 3 == 16 || nch / 3 == 32 || nch / 3 == 64)) {
            lpr = nch / 3;
            cpl = 3;
        } else if (!pick(nch, lpr, cpl)) {
            return hipErrorInvalidConfiguration;
        }
    }
    if (m.k > DT_KMAX || m.kout % DT_RT) return hipErrorInvalidConfiguration;
    DownTokArgs a;
    a.experts = experts.base;
    a.etab = experts.table;
    a.eb = m.expert_bytes;
    a.dn_off = m.dn_off + m.dn.codes_off;
    a.dn_scales_off = m.dn.scales_off - m.dn.codes_off;
    a.F = m.F; a.Kout = m.kout; a.k = m.k;
    a.hq = hq; a.b = b; a.out = out; a.taps = taps;
    a.outq = outq;
    a.arrive = outq.q ? arrive : nullptr;
    a.ts_off = m.ts_off ? m.ts_off + 8 : 0;     // NVFP4: the down tensor scale
    bool tap = taps.isum_dn || taps.y;
    if (kq) {
        const size_t lds = (size_t)m.k * (m.F + 8 * (m.F / QK));
        if (m.fmt == MOE_FMT_Q4_K)
            return tap ? down_tok_kq_fmt<MOE_FMT_Q4_K, true>(lpr, cpl, T, lds, a, st)
                       : down_tok_kq_fmt<MOE_FMT_Q4_K, false>(lpr, cpl, T, lds, a, st);
        if (m.fmt == MOE_FMT_Q5_K)
            return tap ? down_tok_kq_fmt<MOE_FMT_Q5_K, true>(lpr, cpl, T, lds, a, st)
                       : down_tok_kq_fmt<MOE_FMT_Q5_K, false>(lpr, cpl, T, lds, a, st);
        return tap ? down_tok_kq_fmt<MOE_FMT_Q3_K, true>(lpr, cpl, T, lds, a, st)
                   : down_tok_kq_fmt<MOE_FMT_Q3_K, false>(lpr, cpl, T, lds, a, st);
    }
    if (m.fmt == MOE_FMT_Q4_0)
        return tap ? down_tok_fmt<MOE_FMT_Q4_0, true>(lpr, cpl, T, a, st)
                   : down_tok_fmt<MOE_FMT_Q4_0, false>(lpr, cpl, T, a, st);
    if (m.fmt == MOE_FMT_Q5_1)
        return tap ? down_tok_fmt<MOE_FMT_Q5_1, true>(lpr, cpl, T, a, st)
                   : down_tok_fmt<MOE_FMT_Q5_1, false>(lpr, cpl, T, a, st);
    if (m.fmt == MOE_FMT_NVFP4)
        return tap ? down_tok_fmt<MOE_FMT_NVFP4, true>(lpr, cpl, T, a, st)
                   : down_tok_fmt<MOE_FMT_NVFP4, false>(lpr, cpl, T, a, st);
    return tap ? down_tok_fmt<MOE_FMT_Q8_0, true>(lpr, cpl, T, a, st)
               : down_tok_fmt<MOE_FMT_Q8_0, false>(lpr, cpl, T, a, st);
}

}  // namespace moe
