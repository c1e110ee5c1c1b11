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
// Router logits, partial over K slices: part[s][t][e] = sum_{i in slice s} x[t,i] W[e,i].
// A workgroup = 4 waves = 4 experts; blockIdx.y = slice; blockIdx.z = token tile.
// Products of two floats are exact in fp64; only the additions round.
template <int TT>
__global__ __launch_bounds__(256) void k_router_logits(const float* __restrict__ x,
                                                       const float* __restrict__ W, int T, int H,
                                                       int E, int S, double* __restrict__ part) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int e = blockIdx.x * 4 + wave;
    const int s = blockIdx.y;
    const int t0 = blockIdx.z * TT;
    if (e >= E) return;
    const int nt = min(TT, T - t0);
    const int slice = H / S, k0 = s * slice;
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
    const float* wrow = W + (size_t)e * H;
    for (int i = k0 + lane * 4; i < k0 + slice; i += 256) {
        float4 w = *reinterpret_cast<const float4*>(wrow + i);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t < nt) {
                float4 xv = *reinterpret_cast<const float4*>(x + (size_t)(t0 + t) * H + i);
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
            double v = wave_sum_d(acc[t]);
            if (lane == 0) part[((size_t)s * T + t0 + t) * E + e] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// One wave per token: sum the slices, add the bias, group limit, top-k, softmax.
__device__ __forceinline__ void argmax_pair(double& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        double ov = __shfl_xor(v, o, 64);
        int oi = __shfl_xor(i, o, 64);
        if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
    }
}

constexpr int MAXE_LANE = 8;   // experts per lane: E <= 512

__global__ __launch_bounds__(64) void k_router_topk(const double* __restrict__ part, int S, int T,
                                                    int E, int k, const float* __restrict__ bias,
                                                    const int32_t* __restrict__ groups, int G,
                                                    int TG, int32_t* __restrict__ ids,
                                                    float* __restrict__ wts,
                                                    double* __restrict__ logits_tap) {
    __shared__ double sl[512];
    const int t = blockIdx.x, lane = threadIdx.x;
    const double NEG = -__builtin_huge_val();
    double l[MAXE_LANE];
    bool ok[MAXE_LANE];      // allowed by the group limit
    bool taken[MAXE_LANE];
#pragma unroll
    for (int m = 0; m < MAXE_LANE; ++m) {
        int e = lane + 64 * m;
        l[m] = NEG;
        ok[m] = false;
        taken[m] = e >= E;
        if (e < E) {
            double v = 0.0;
            for (int s = 0; s < S; ++s) v += part[((size_t)s * T + t) * E + e];
            if (bias) v += (double)bias[e];
            l[m] = v;
            ok[m] = true;
            sl[e] = v;
            if (logits_tap) logits_tap[(size_t)t * E + e] = v;
        }
    }
    if (G > 0) {
        __syncthreads();
        // score of group `lane` = its largest member logit
        double gs = NEG;
        if (lane < G)
            for (int e = 0; e < E; ++e)
                if (groups[e] == lane && sl[e] > gs) gs = sl[e];
        bool gsel = false;
        for (int n = 0; n < TG; ++n) {
            double v = (lane < G && !gsel) ? gs : NEG;
            int i = (lane < G && !gsel) ? lane : 0x7fffffff;
            argmax_pair(v, i);
            if (lane == i) gsel = true;
        }
        __syncthreads();
        // publish the chosen groups through LDS (reuse the first 64 doubles as flags)
        sl[lane] = gsel ? 1.0 : 0.0;
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m) {
            int e = lane + 64 * m;
            if (e < E) {
                unsigned gl = (unsigned)groups[e];
                ok[m] = gl < (unsigned)G && sl[gl] != 0.0;
            }
        }
    }
    double top_l = 0.0;
    int my_id = -1;
    double my_l = 0.0;
    for (int j = 0; j < k; ++j) {
        double bv = NEG;
        int bi = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m) {
            int e = lane + 64 * m;
            if (ok[m] && !taken[m] && (l[m] > bv || (l[m] == bv && e < bi))) { bv = l[m]; bi = e; }
        }
        argmax_pair(bv, bi);
        if (bi == 0x7fffffff) {
            // labels that break the one-size-groups contract left fewer than k
            // candidates: fall back to every expert not yet chosen (k <= E)
            bv = NEG;
#pragma unroll
            for (int m = 0; m < MAXE_LANE; ++m) {
                int e = lane + 64 * m;
                if (!taken[m] && (bi == 0x7fffffff || l[m] > bv || (l[m] == bv && e < bi))) { bv = l[m]; bi = e; }
            }
            argmax_pair(bv, bi);
        }
#pragma unroll
        for (int m = 0; m < MAXE_LANE; ++m)
            if (lane + 64 * m == bi) taken[m] = true;
        if (j == 0) top_l = bv;
        if (lane == j) { my_id = bi; my_l = bv; }
    }
    double ex = lane < k ? exp(my_l - top_l) : 0.0;
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += __shfl(ex, j, 64);        // rank order
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        wts[(size_t)t * k + lane] = (float)(ex / den);
    }
}

// ---------------------------------------------------------------------------
// Bucketing: workgroup e lists the assignments routed to expert e in token order.
// The last workgroup to finish compacts the experts with tokens into slots and
// computes each slot's first token tile (tiles of tile_m tokens).
__global__ __launch_bounds__(256) void k_bucket(const int32_t* __restrict__ ids, int A, int T,
                                                int E, int tile_m, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ lists,
                                                uint32_t* __restrict__ ctrl,
                                                int32_t* __restrict__ active,
                                                int32_t* __restrict__ tile_start) {
    __shared__ int wsum[4];
    __shared__ int base;
    __shared__ int is_last;
    const int e = blockIdx.x, tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    if (tid == 0) base = 0;
    __syncthreads();
    for (int a0 = 0; a0 < A; a0 += 256) {
        int a = a0 + tid;
        bool f = a < A && ids[a] == e;
        uint64_t m = __ballot(f);
        int pre = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[wave] = __popcll(m);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wsum[w];
        if (f) lists[(size_t)e * T + off + pre] = a;
        __syncthreads();
        if (tid == 0) base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (tid == 0) counts[e] = base;
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = atomicAdd(&ctrl[CW_BUCKET_ARRIVE], 1u) == (unsigned)(E - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    // compact: slot order = expert id order.  Two experts per thread (E <= 512).
    __shared__ int sc[512];
    __shared__ int tiles[512];
    int c0 = 0, c1 = 0;
    int e0 = 2 * tid, e1 = 2 * tid + 1;
    if (e0 < E) c0 = __atomic_load_n(&counts[e0], __ATOMIC_RELAXED);
    if (e1 < E) c1 = __atomic_load_n(&counts[e1], __ATOMIC_RELAXED);
    // inclusive scan of (active count, tile count) over threads
    int act = (c0 > 0) + (c1 > 0);
    int til = (c0 + tile_m - 1) / tile_m + (c1 + tile_m - 1) / tile_m;
    sc[tid] = act;
    tiles[tid] = til;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int va = tid >= o ? sc[tid - o] : 0;
        int vt = tid >= o ? tiles[tid - o] : 0;
        __syncthreads();
        sc[tid] += va;
        tiles[tid] += vt;
        __syncthreads();
    }
    int slot = sc[tid] - act;           // exclusive
    int tl = tiles[tid] - til;
    if (c0 > 0) { active[slot] = e0; tile_start[slot] = tl; ++slot; tl += (c0 + tile_m - 1) / tile_m; }
    if (c1 > 0) { active[slot] = e1; tile_start[slot] = tl; }
    if (tid == 255) {
        ctrl[CW_N_ACTIVE] = sc[255];
        ctrl[CW_N_TILES] = tiles[255];
        tile_start[sc[255]] = tiles[255];
        ctrl[CW_BUCKET_ARRIVE] = 0u;    // ready for the next call
    }
}

// ---------------------------------------------------------------------------
// out[t][r] = sum_j w[t][j] * y[t*k + j][r], rank order, fp32.  With a latent
// layer the sum is y_lat and out is the latent buffer.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ wts, int T, int k,
                                                 int R, float* __restrict__ out) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)T * R) return;
    const long t = i / R, r = i % R;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc = fmaf(wts[t * k + j], y[(t * k + j) * R + r], acc);
    out[i] = acc;
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
                         hipStream_t st) {
    double* part = (double*)(ws + w.logit_part);
    int S = w.S;
    if (T <= 8) {
        dim3 g((m.E + 3) / 4, S, (T + 7) / 8);
        hipLaunchKernelGGL(k_router_logits<8>, g, dim3(256), 0, st, x, Wr, T, m.H, m.E, S, part);
    } else {
        dim3 g((m.E + 3) / 4, S, (T + 31) / 32);
        hipLaunchKernelGGL(k_router_logits<32>, g, dim3(256), 0, st, x, Wr, T, m.H, m.E, S, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_router_topk, dim3(T), dim3(64), 0, st, part, S, T, m.E, m.k, br, groups,
                       m.G, m.TG, (int32_t*)(ws + w.ids), (float*)(ws + w.wts), logits_tap);
    return hipGetLastError();
}

hipError_t launch_bucket(const Dims& m, const WsLayout& w, char* ws, int T, int tile_m,
                         hipStream_t st) {
    hipLaunchKernelGGL(k_bucket, dim3(m.E), dim3(256), 0, st, (const int32_t*)(ws + w.ids), T * m.k,
                       T, m.E, tile_m, (int32_t*)(ws + w.counts), (int32_t*)(ws + w.lists),
                       (uint32_t*)(ws + w.ctrl), (int32_t*)(ws + w.active),
                       (int32_t*)(ws + w.tile_start));
    return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* wts, int T, int k, int R, float* out,
                          hipStream_t st) {
    long n = (long)T * R;
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
