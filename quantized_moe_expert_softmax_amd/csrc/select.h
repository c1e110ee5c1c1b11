// Per-token expert selection: the ordered keys that the router kernels rank
// logits by, and the workgroup-wide selection of a single token that the
// gate/up kernel runs in its prologue.
//
// Router (Strata PR 24, SYCL port commits: top-k over the experts per token;
// edge0-strata README: expert group labels).
#pragma once
#include "kernels.h"

namespace moe {

// order-preserving map of a double to an unsigned 64-bit key
__device__ __forceinline__ unsigned long long dkey(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double dkey_inv(unsigned long long k) {
    const unsigned long long b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)b);
}

// LDS of the single-token selection (E <= 512, k <= 32, n_groups <= 64).
struct RouteLds {
    unsigned long long key[512];    // ordered key of each logit; 0 = excluded
    unsigned long long gkey[64];    // group score: largest member key
    double ex[32];                  // exp(l_j - l_0), rank order
    int sel[32];                    // rank -> expert
    int nallow;                     // experts in the kept groups
    unsigned char gsel[64];         // group kept
};

// Selection for one token by a whole workgroup of NT threads (every thread
// calls; `weights` uniform over the workgroup), from its logits part[e]
// (+ bias[e]).  Group limit: the groups are ranked by their largest member
// key (ties to the lower group) and the experts outside the TG best get key 0,
// unless that leaves fewer than k (labels that break the equal-size-groups
// contract).  Every candidate's rank is the number of candidates that beat it
// ((key desc, id asc)), P threads per expert each counting over E/P rivals;
// rank < k gives S.sel[rank].  With `weights`, S.ex[j] = exp(l_j - l_0) in fp64
// and *w (threads j < k) = ex_j / sum of ex in rank order.
template <int NT>
__device__ __forceinline__ void select_wg(const SelectArgs& A, RouteLds& S, bool weights, float* w) {
    const int tid = threadIdx.x, E = A.E, k = A.k, G = A.G;
    for (int i = tid; i < E; i += NT) {
        double v = 0.0 + A.part[i];
        if (A.bias) v += (double)A.bias[i];
        S.key[i] = dkey(v + 0.0);      // -0 and +0 get one key
        if (A.logits_tap) A.logits_tap[i] = v;
    }
    if (G > 0) {
        if (tid < 64) S.gkey[tid] = 0ull;
        if (tid == 0) S.nallow = 0;
    }
    __syncthreads();
    if (G > 0) {
        for (int i = tid; i < E; i += NT) {
            const unsigned gl = (unsigned)A.groups[i];
            if (gl < (unsigned)G) atomicMax(&S.gkey[gl], S.key[i]);
        }
        __syncthreads();
        for (int g = tid; g < G; g += NT) {
            const unsigned long long kg = S.gkey[g];
            int r = 0;
            for (int h = 0; h < G; ++h) {
                const unsigned long long kh = S.gkey[h];
                r += (int)(kh > kg) | ((int)(kh == kg) & (int)(h < g));
            }
            S.gsel[g] = r < A.TG;
        }
        __syncthreads();
        for (int i = tid; i < E; i += NT) {
            const unsigned gl = (unsigned)A.groups[i];
            if (gl < (unsigned)G && S.gsel[gl]) atomicAdd(&S.nallow, 1);
        }
        __syncthreads();
        for (int i = tid; i < E; i += NT) {
            const unsigned gl = (unsigned)A.groups[i];
            const bool al = gl < (unsigned)G && S.gsel[gl];
            if (!al && S.nallow >= k) S.key[i] = 0ull;
        }
        __syncthreads();
    }
    int P = 1;
    while (P < 64 && E * P * 2 <= NT) P *= 2;
    const int lp = 31 - __clz(P);
    for (int b0 = 0; b0 < (E << lp); b0 += NT) {
        const int gi = b0 + tid;
        const int i = gi >> lp, part = gi & (P - 1);
        int r = 0;
        const unsigned long long ke = i < E ? S.key[i] : 0ull;
        const bool cand = ke != 0ull;
        if (cand) {
            constexpr int U = 8;
            for (int h0 = part; h0 < E; h0 += U * P) {
                unsigned long long kh[U];
#pragma unroll
                for (int u = 0; u < U; ++u) kh[u] = S.key[min(h0 + u * P, E - 1)];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int h = h0 + u * P;
                    r += (int)(h < E) & ((int)(kh[u] > ke) | ((int)(kh[u] == ke) & (int)(h < i)));
                }
            }
        }
        for (int o = 1; o < P; o <<= 1) r += __shfl_xor(r, o);
        if (cand && part == 0 && r < k) S.sel[r] = i;
    }
    __syncthreads();
    if (weights) {
        if (tid < k) S.ex[tid] = exp(dkey_inv(S.key[S.sel[tid]]) - dkey_inv(S.key[S.sel[0]]));
        __syncthreads();
        if (tid < k) {
            double den = 0.0;
            for (int j = 0; j < k; ++j) den += S.ex[j];
            *w = (float)(S.ex[tid] / den);
        }
    }
}

}  // namespace moe
