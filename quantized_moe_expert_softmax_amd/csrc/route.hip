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
#include "select.h"

namespace moe {

// ---------------------------------------------------------------------------
// Q8_1 quantisation of fp32 rows [rows][K]: one 32-lane group per block.
// With S > 1, x holds S partial arrays that are added in slice order first
// (and the sums stored to xsum when it is not null).
__global__ __launch_bounds__(256) void k_quant_rows(const float* __restrict__ x, int S, float* xsum,
                                                    int rows, int K, ActPtr out) {
    const int nb = K / QK;
    const long blk = (long)blockIdx.x * 8 + threadIdx.x / 32;
    if (blk >= (long)rows * nb) return;               // whole 32-lane groups exit together
    const int l = threadIdx.x % 32;
    const long r = blk / nb, b = blk % nb;
    const long i = r * K + b * QK + l;
    float v = x[i];
    for (int s = 1; s < S; ++s) v += x[(long)s * rows * K + i];
    if (xsum) xsum[i] = v;
    quant_q8_1_32(v, l, out.q + r * K + b * QK, out.ds + r * nb + b, out.sq + r * nb + b);
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
// Router logits of a few tokens (T <= DECODE_T): whole logits, no K slices.  A
// single token's top-k, softmax and bucketing then run in the prologue of the
// gate/up kernel; two to DECODE_T tokens are selected by k_route_select_tok.
//
// k_route_logits_dec: workgroups [0, E): expert e = blockIdx.x, 256 threads
// over the H-wide row of W_r with every load issued at once (ROUTE_U float4 per
// thread, the fewest that cover the row; indices past the row are clamped and
// masked), logits l[t][e] in fp64 for every token; workgroups [E, E + nq):
// Q8_1(x).
constexpr int ROUTE_U_MAX = 8;   // float4 per thread: H <= 8192

template <int ROUTE_U>
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
    // token rows through two register buffers: the next token's row is in
    // flight while one is multiplied (a load past the last token re-reads it)
    auto load_x = [&](int t, float4 (&xv)[ROUTE_U]) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)min(t, T - 1) * H);
#pragma unroll
        for (int u = 0; u < ROUTE_U; ++u) xv[u] = xr[min((int)threadIdx.x + 256 * u, h4 - 1)];
    };
    auto dot = [&](int t, const float4 (&xv)[ROUTE_U]) {
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
    };
    float4 xa[ROUTE_U], xb[ROUTE_U];
    load_x(0, xa);
    for (int t = 0; t < T; t += 2) {
        load_x(t + 1, xb);
        dot(t, xa);
        load_x(t + 2, xa);
        if (t + 1 < T) dot(t + 1, xb);
    }
    __syncthreads();
    if ((int)threadIdx.x < T) {
        const int t = threadIdx.x;
        logits[(size_t)t * E + e] = ((s_part[t][0] + s_part[t][1]) + s_part[t][2]) + s_part[t][3];
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
// counter) buckets every token's assignments and clears the counter for the
// next call: per expert the count and a token bitmask; the slots are the
// experts with tokens in id order; an assignment's place in its expert's list
// is its token's rank among that expert's tokens.
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
    __shared__ int s_gcnt[64];
    __shared__ unsigned char s_gsel[64];
    __shared__ int s_nallow;
    __shared__ int s_sel[32];
    __shared__ double s_ex[32];
    __shared__ int s_last;
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = A.T, E = A.E, k = A.k, G = A.G;
    // each thread's experts tid + m * TSEL_NT: partial logits, bias and group
    // label, every load issued before the first is used
    constexpr int EPT = (512 + TSEL_NT - 1) / TSEL_NT;
    unsigned gl[EPT];
    unsigned long long key[EPT];
    if (G > 0 && tid < 64) {
        s_gkey[tid] = 0ull;
        s_gcnt[tid] = 0;
    }
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + m * TSEL_NT;
        gl[m] = ~0u;
        key[m] = 0ull;
        if (e < E) {
            double ps[ROUTE_SMAX];
#pragma unroll
            for (int sl = 0; sl < ROUTE_SMAX; ++sl)
                ps[sl] = sl < A.S ? A.part[((size_t)sl * T + t) * E + e] : 0.0;
            const float b = A.bias ? A.bias[e] : 0.0f;
            if (G > 0) gl[m] = (unsigned)A.groups[e];
            double v = 0.0;
#pragma unroll
            for (int sl = 0; sl < ROUTE_SMAX; ++sl)
                if (sl < A.S) v += ps[sl];
            if (A.bias) v += (double)b;
            if (A.logits_tap) A.logits_tap[(size_t)t * E + e] = v;
            key[m] = dkey(v + 0.0);
        }
    }
    if (G > 0) {
        // groups ranked by their largest member key (ties to the lower group);
        // the experts outside the TG best get key 0, unless fewer than k would
        // stay (labels that break the equal-size-groups contract)
        __syncthreads();
#pragma unroll
        for (int m = 0; m < EPT; ++m)
            if (gl[m] < (unsigned)G) {
                atomicMax(&s_gkey[gl[m]], key[m]);
                atomicAdd(&s_gcnt[gl[m]], 1);
            }
        __syncthreads();
        if (tid < 64) {
            const unsigned long long kg = tid < G ? s_gkey[tid] : 0ull;
            int r = 0;
            for (int h = 0; h < G; ++h) {
                const unsigned long long kh = s_gkey[h];
                r += (int)(kh > kg) | ((int)(kh == kg) & (int)(h < tid));
            }
            const bool kept = tid < G && r < A.TG;
            if (tid < G) s_gsel[tid] = kept;
            int n = kept ? s_gcnt[tid] : 0;
            for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
            if (tid == 0) s_nallow = n;
        }
        __syncthreads();
        if (s_nallow >= k) {
#pragma unroll
            for (int m = 0; m < EPT; ++m)
                if (!(gl[m] < (unsigned)G && s_gsel[gl[m]])) key[m] = 0ull;
        }
    }
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + m * TSEL_NT;
        if (e < E) {
            s_key[e] = key[m];
            s_khi[e] = (unsigned)(key[m] >> 32);
        }
    }
    __syncthreads();
    // ranks: P lanes per expert each count the rivals among E/P of them, first
    // on the top 32 bits of the keys (one compare each); an expert that could
    // be chosen and shares those bits with a rival is ranked again on the
    // whole keys
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

// The same sums, one 32-lane group per Q8_1 block of out, which also writes
// Q8_1(out) (a latent layer's y_lat, for the U projection): each element is
// added in the same order as above, so out is the same.
__global__ __launch_bounds__(256) void k_combine_q(const float* __restrict__ y,
                                                   const float* __restrict__ wts, int T, int k,
                                                   int R, float* __restrict__ out, ActPtr outq) {
    const int nb = R / QK;
    const long blk = (long)blockIdx.x * 8 + threadIdx.x / 32;
    if (blk >= (long)T * nb) return;                  // whole 32-lane groups exit together
    const int l = threadIdx.x % 32;
    const long t = blk / nb, b = blk % nb;
    const long r = b * QK + l;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc = fmaf(wts[t * k + j], y[(t * k + j) * R + r], acc);
    out[t * R + r] = acc;
    quant_q8_1_32(acc, l, outq.q + t * R + b * QK, outq.ds + t * nb + b, outq.sq + t * nb + b);
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
    hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((blocks + 7) / 8)), dim3(256), 0, st, x, 1,
                       (float*)nullptr, rows, K, out);
    return hipGetLastError();
}

hipError_t launch_quant_rows_sum(const float* part, int S, float* x, int rows, int K, ActPtr out,
                                 hipStream_t st) {
    long blocks = (long)rows * (K / QK);
    if (blocks == 0) return hipSuccess;
    if (S < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((blocks + 7) / 8)), dim3(256), 0, st, part, S,
                       x, rows, K, out);
    return hipGetLastError();
}

hipError_t launch_router(const Dims& m, const WsLayout& w, char* ws, const float* x, int T,
                         const float* Wr, const float* br, const int32_t* groups, double* logits_tap,
                         ActPtr xq, bool ids_only, bool defer_select, RouteDone* done,
                         SelectArgs* sel, hipStream_t st) {
    double* part = (double*)(ws + w.logit_part);
    const int S = w.S;
    const long qblocks = (long)T * (m.H / QK);
    const int qwg = (int)((qblocks + 7) / 8);
    int32_t* ids = (int32_t*)(ws + w.ids);
    float* wts = (float*)(ws + w.wts);
    SelectArgs a;
    a.part = part; a.S = S; a.T = T; a.E = m.E; a.k = m.k;
    a.bias = br; a.groups = groups; a.G = m.G; a.TG = m.TG; a.logits_tap = logits_tap;
    *sel = a;
    int32_t* counts = (int32_t*)(ws + w.counts);
    int32_t* lists = (int32_t*)(ws + w.lists);
    uint32_t* ctrl = (uint32_t*)(ws + w.ctrl);
    int32_t* active = (int32_t*)(ws + w.active);
    if (T <= DECODE_T) {
        if (S != 1) return hipErrorInvalidValue;
        const int h4 = m.H / 4;
        const dim3 grid(m.E + qwg), block(256);
        if (h4 <= 256)
            hipLaunchKernelGGL(k_route_logits_dec<1>, grid, block, 0, st, x, Wr, T, m.H, m.E, part, xq);
        else if (h4 <= 512)
            hipLaunchKernelGGL(k_route_logits_dec<2>, grid, block, 0, st, x, Wr, T, m.H, m.E, part, xq);
        else if (h4 <= 1024)
            hipLaunchKernelGGL(k_route_logits_dec<4>, grid, block, 0, st, x, Wr, T, m.H, m.E, part, xq);
        else if (h4 <= 256 * ROUTE_U_MAX)
            hipLaunchKernelGGL(k_route_logits_dec<8>, grid, block, 0, st, x, Wr, T, m.H, m.E, part, xq);
        else
            return hipErrorInvalidValue;
        if (T <= ROUTE_DEC_MAX_T) {
            *done = ROUTE_LOGITS;
        } else if (ids_only && defer_select) {
            *done = ROUTE_DEFERRED;
        } else if (ids_only) {
            hipLaunchKernelGGL((k_route_select_tok<false, 1024>), dim3(T), dim3(1024), 0, st, a, ids,
                               wts, counts, lists, ctrl, active);
            *done = ROUTE_IDS;
        } else {
            hipLaunchKernelGGL((k_route_select_tok<true, 1024>), dim3(T), dim3(1024), 0, st, a, ids,
                               wts, counts, lists, ctrl, active);
            *done = ROUTE_BUCKETED;
        }
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
    if (T <= MV_MAX_T && T * m.k <= 1024 && m.E <= 512) {
        hipLaunchKernelGGL((k_route_select_tok<true, 1024>), dim3(T), dim3(1024), 0, st, a, ids,
                           wts, counts, lists, ctrl, active);
        *done = ROUTE_BUCKETED;
    } else {
        hipLaunchKernelGGL((k_route_select_tok<false, 256>), dim3(T), dim3(256), 0, st, a, ids,
                           wts, counts, lists, ctrl, active);
        *done = ROUTE_SELECTED;
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

hipError_t launch_combine_q(const float* y, const float* wts, int T, int k, int R, float* out,
                            ActPtr outq, hipStream_t st) {
    long blocks = (long)T * (R / QK);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_combine_q, dim3((unsigned)((blocks + 7) / 8)), dim3(256), 0, st, y, wts, T,
                       k, R, out, outq);
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
