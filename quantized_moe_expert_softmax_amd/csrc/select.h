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
// the same for a float: rounding a double to float is monotone, so the fp32
// key of a logit never reverses the order of two fp64 keys (it may merge them)
__device__ __forceinline__ unsigned fkey(float f) {
    const unsigned b = __float_as_uint(f);
    return (b >> 31) ? ~b : (b | 0x80000000u);
}

// LDS of the single-token selection (E <= 512, k <= 32, n_groups <= 64, at
// most 8 waves), 16-byte aligned.
struct alignas(16) RouteLds {
    unsigned long long key[512];    // ordered key of each logit; 0 = excluded
    unsigned long long ckey[256];   // candidates: wave w's local rank r at w*k + r
    unsigned long long gkey[64];    // group score: largest member key
    double ex[32];                  // exp(l_j - l_0), rank order
    int cid[256];                   // candidate expert ids
    int gcnt[64];                   // experts per group label
    int sel[32];                    // rank -> expert
    int rp[512];                    // fast ranking: one thread's share of an expert's count
    unsigned k32[520];              // fast ranking: fp32 key of each logit (0 = excluded; 8 spare)
    unsigned ck32[264];             // fast ranking: fp32 keys of the candidates (8 spare)
    unsigned cbits[8];              // fast ranking: local ranks claimed in each wave
    unsigned rmask;                 // fast ranking: ranks claimed
    int tie;                        // fast ranking: a rank was claimed twice
    int nallow;                     // experts in the kept groups
    unsigned char gsel[64];         // group kept
};

__device__ __forceinline__ void claim_rank(RouteLds& S, int r, int id) {
    const unsigned bit = 1u << r;
    if (atomicOr(&S.rmask, bit) & bit) S.tie = 1;
    S.sel[r] = id;
}

// Ranking by strict count over the fp32 keys: an expert's rank is taken as
// the number of keys above its own, the rivals' keys read eight at a time
// (two 16-byte LDS loads at a wave-uniform address) with no range masks:
// every range is a whole number of eights and S.k32 holds zeros past E (a
// zero key never counts), as does S.ck32 past the candidates.  Each rank
// below k is claimed with an atomic bit (S.rmask, S.tie, S.cbits zero on
// entry, S.k32 and S.ck32 written, after a barrier).  The claims are the
// exact top k whenever they are k distinct ranks: two experts with equal keys
// get equal counts, so a tie inside the top k or across its boundary (in
// fp32, also two fp64 logits that round to one float) makes two experts claim
// one rank, or one local rank in the two-level form, where the candidates of
// a wave are those with fewer than k of the wave's keys above them, and a
// candidate outside the global top k always has the k members above it.
// Returns false on such a tie, when the fp64 keys in (key desc, id asc) order
// have to decide.
__device__ __forceinline__ int count_above(const unsigned* kp, int n8, unsigned ke) {
    int r = 0;
    for (int hb = 0; hb < n8; hb += 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(kp + hb);
        const uint4 b = *reinterpret_cast<const uint4*>(kp + hb + 4);
        // one add with carry per rival
        r += (int)(a.x > ke);
        r += (int)(a.y > ke);
        r += (int)(a.z > ke);
        r += (int)(a.w > ke);
        r += (int)(b.x > ke);
        r += (int)(b.y > ke);
        r += (int)(b.z > ke);
        r += (int)(b.w > ke);
    }
    return r;
}

template <int NT, int MPT>
__device__ __forceinline__ bool rank_gt(RouteLds& S, const unsigned (&k32)[MPT], int E, int k) {
    constexpr int NWV = NT / 64;
    const int tid = threadIdx.x;
    if (E * 2 <= NT) {
        // P threads per expert: expert i = tid % EPP, its part tid / EPP of the
        // rivals, CH8 of them (the part is the same across a wave when EPP >= 64)
        int P = 2;
        while (P < 64 && E * P * 2 <= NT) P *= 2;
        const int EPP = NT / P, le = 31 - __clz(EPP);
        const int i = tid & (EPP - 1);
        int part = tid >> le;
        if (EPP >= 64) part = __builtin_amdgcn_readfirstlane(part);
        const int CH8 = (((E + P - 1) / P) + 7) & ~7;   // P * CH8 <= E + 8P <= 520
        const unsigned ke = i < E ? S.k32[i] : 0u;
        S.rp[tid] = count_above(S.k32 + part * CH8, CH8, ke);
        __syncthreads();
        if (tid < EPP && i < E && ke != 0u) {
            int rr = 0;
            for (int q = 0; q < P; ++q) rr += S.rp[q * EPP + i];
            if (rr < k) claim_rank(S, rr, i);
        }
    } else {
        // level 1 over the wave's experts 64*wave + j and NT + 64*wave + j
        const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int nb = min(MPT, (E + NT - 1) / NT);
#pragma unroll
        for (int m = 0; m < MPT; ++m) {
            const unsigned ke = k32[m];
            if (ke != 0u) {
                int r = 0;
                for (int b = 0; b < nb; ++b) r += count_above(S.k32 + b * NT + 64 * wv, 64, ke);
                if (r < k) {
                    const unsigned bit = 1u << r;
                    if (atomicOr(&S.cbits[wv], bit) & bit) S.tie = 1;
                    S.ck32[wv * k + r] = ke;
                    S.cid[wv * k + r] = tid + m * NT;
                }
            }
        }
        __syncthreads();
        const int NC = NWV * k, NC8 = (NC + 7) & ~7;
        for (int c = tid; c < NC; c += NT) {
            const unsigned kc = S.ck32[c];
            if (kc != 0u) {
                const int r = count_above(S.ck32, NC8, kc);
                if (r < k) claim_rank(S, r, S.cid[c]);
            }
        }
    }
    __syncthreads();
    return S.tie == 0 && __popc(S.rmask) == (unsigned)k;
}

// Selection for one token by a whole workgroup of NT threads (every thread
// calls; `weights` uniform over the workgroup), from its logits part[e]
// (+ bias[e]).  Thread t holds experts t and t + NT.
//  * Group limit: the groups are ranked by their largest member key (ties to
//    the lower group) and the experts outside the TG best get key 0, unless
//    that leaves fewer than k (labels that break the equal-size-groups
//    contract).
//  * Top-k with ties to the lower id: an expert's rank is the number of
//    experts whose (key desc, id asc) order beats it; S.sel[rank] for rank < k.
//    With at least two threads per expert, P threads count one expert's rivals
//    directly.  Otherwise in two levels: the rank among the experts the wave
//    holds; those of local rank < k are the candidates, and a candidate's rank
//    among all candidates is its global rank (every expert that beats a global
//    top-k member is itself a candidate).  The strict counts of rank_gt over
//    the fp32 keys come first and decide whenever no tie touches the top k;
//    otherwise these (key desc, id asc) counts over the fp64 keys run.
//  * With `weights`: S.ex[j] = exp(l_j - l_0) in fp64 and *w (threads j < k) =
//    ex_j / the sum of ex in rank order.
template <int NT>
__device__ __forceinline__ void select_wg(const SelectArgs& A, RouteLds& S, bool weights, float* w) {
    constexpr int MPT = (512 + NT - 1) / NT;      // experts per thread
    constexpr int NWV = NT / 64;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int E = A.E, k = A.k, G = A.G;
    unsigned long long key[MPT];
    unsigned gl[MPT];
#pragma unroll
    for (int m = 0; m < MPT; ++m) {
        const int i = tid + m * NT;
        key[m] = 0ull;
        gl[m] = ~0u;
        if (i < E) {
            double v = 0.0 + A.part[i];
            const float b = A.bias ? A.bias[i] : 0.0f;
            if (G > 0) gl[m] = (unsigned)A.groups[i];
            if (A.bias) v += (double)b;
            key[m] = dkey(v + 0.0);     // -0 and +0 get one key
            if (A.logits_tap) A.logits_tap[i] = v;
        }
    }
    for (int c = tid; c < NWV * k; c += NT) S.ckey[c] = 0ull;
    for (int c = tid; c < NWV * k + 8; c += NT) S.ck32[c] = 0u;
    for (int c = E + tid; c < 520; c += NT) S.k32[c] = 0u;
    if (G > 0) {
        if (tid < 64) {
            S.gkey[tid] = 0ull;
            S.gcnt[tid] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MPT; ++m)
            if (gl[m] < (unsigned)G) {
                atomicMax(&S.gkey[gl[m]], key[m]);
                atomicAdd(&S.gcnt[gl[m]], 1);
            }
        __syncthreads();
        if (tid < 64) {
            // wave 0, lane g: the group's rank, and the experts the kept groups hold
            const int g = tid;
            const unsigned long long kg = g < G ? S.gkey[g] : 0ull;
            int r = 0;
#pragma unroll 8
            for (int h = 0; h < G; ++h) {
                const unsigned long long kh = S.gkey[h];
                r += (int)(kh > kg) | ((int)(kh == kg) & (int)(h < g));
            }
            const bool kept = g < G && r < A.TG;
            if (g < G) S.gsel[g] = kept;
            int n = kept ? S.gcnt[g] : 0;
            for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
            if (g == 0) S.nallow = n;
        }
        __syncthreads();
        if (S.nallow >= k) {
#pragma unroll
            for (int m = 0; m < MPT; ++m)
                if (!(gl[m] < (unsigned)G && S.gsel[gl[m]])) key[m] = 0ull;
        }
    }
    unsigned k32[MPT];
#pragma unroll
    for (int m = 0; m < MPT; ++m) {
        // (a logit whose float key would be the excluded mark is raised to 1)
        k32[m] = key[m] != 0ull ? max(fkey((float)dkey_inv(key[m])), 1u) : 0u;
        if (tid + m * NT < E) {
            S.key[tid + m * NT] = key[m];
            S.k32[tid + m * NT] = k32[m];
        }
    }
    if (tid < NWV) S.cbits[tid] = 0u;
    if (tid == 0) {
        S.rmask = 0u;
        S.tie = 0;
    }
    __syncthreads();
    if (rank_gt<NT>(S, k32, E, k)) {
        // the strict counts gave the top k
    } else if (E * 2 <= NT) {
        // at least two threads per expert: P of them count the rivals of one
        // expert over E/P of them each, which gives the global rank directly
        int P = 2;
        while (P < 64 && E * P * 2 <= NT) P *= 2;
        const int lp = 31 - __clz(P);
        const int i = tid >> lp, part = tid & (P - 1);
        int r = 0;
        const unsigned long long ke = i < E ? S.key[i] : 0ull;
        if (ke != 0ull) {
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
        if (ke != 0ull && part == 0 && r < k) S.sel[r] = i;
        __syncthreads();
    } else {
        // level 1: rank among the wave's experts 64*wave + j and NT + 64*wave + j
        // (the candidate slots cleared again after the strict counts)
        for (int c = tid; c < NWV * k; c += NT) S.ckey[c] = 0ull;
        __syncthreads();
        const int nw = 64 * min(MPT, (E + NT - 1) / NT);   // rivals held by the wave
#pragma unroll
        for (int m = 0; m < MPT; ++m) {
            const int i = tid + m * NT;
            const unsigned long long ke = key[m];
            int r = 0;
            if (ke != 0ull) {
                constexpr int U = 8;
                for (int h0 = 0; h0 < nw; h0 += U) {
                    unsigned long long kh[U];
                    int hi[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int h = h0 + u;
                        hi[u] = (h >> 6) * NT + 64 * wave + (h & 63);
                        kh[u] = S.key[min(hi[u], E - 1)];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        r += (int)(hi[u] < E) & ((int)(kh[u] > ke) | ((int)(kh[u] == ke) & (int)(hi[u] < i)));
                }
                if (r < k) {
                    S.ckey[wave * k + r] = ke;
                    S.cid[wave * k + r] = i;
                }
            }
        }
        __syncthreads();
        // level 2: rank among the candidates
        for (int c = tid; c < NWV * k; c += NT) {
            const unsigned long long kc = S.ckey[c];
            if (kc != 0ull) {
                const int ic = S.cid[c];
                int r = 0;
#pragma unroll 8
                for (int h = 0; h < NWV * k; ++h) {
                    const unsigned long long kh = S.ckey[h];
                    const int ih = S.cid[h];
                    r += (int)(kh != 0ull) & ((int)(kh > kc) | ((int)(kh == kc) & (int)(ih < ic)));
                }
                if (r < k) S.sel[r] = ic;
            }
        }
        __syncthreads();
    }
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
