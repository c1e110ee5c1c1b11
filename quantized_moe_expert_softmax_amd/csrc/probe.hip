// HBM read probe of libmoe: the rate at which one kernel launch streams a
// buffer with 16-byte loads, as the measured ceiling that the expert kernels'
// bandwidth is compared with.
//
// Prior art ("Sync upstream Strata v0.1.39 into Lanes", the SYCL port commits):
// a bandwidth probe there read incompressible data with 4-byte and 16-byte
// loads and found the wide loads faster.  Here: each thread keeps UNROLL
// independent 16-byte loads in flight per step of a grid-stride loop over the
// buffer, folds them with xor and writes one word per thread, so no load can be
// dropped by the compiler.  The launch's own dispatch records the events, so
// their difference is the kernel's duration.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__device__ __forceinline__ v4i ld(const v4i* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void k_read16(const v4i* __restrict__ src, size_t n16,
                                                uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    v4i acc = {0, 0, 0, 0};
    // whole steps: UNROLL loads per thread, all issued before any is used
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        v4i v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = ld<UNROLL, NT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= ld<UNROLL, NT>(src + i);
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

}  // namespace

template <int U>
static void launch(bool nt, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                   const v4i* src, size_t n16, uint32_t* sink) {
    if (nt)
        hipExtLaunchKernelGGL(k_read16<U, true>, grid, dim3(256), 0, st, e0, e1, 0u, src, n16, sink);
    else
        hipExtLaunchKernelGGL(k_read16<U, false>, grid, dim3(256), 0, st, e0, e1, 0u, src, n16, sink);
}

extern "C" int moe_probe_read(const void* buf, size_t bytes, int blocks, int unroll, int flags,
                              uint32_t* sink, void* stream, void* ev_start, void* ev_stop) {
    if (!buf || !sink || bytes == 0 || bytes % 16 || blocks < 1 || blocks > (1 << 20) ||
        ((uintptr_t)buf & 15) || (flags & ~MOE_PROBE_NONTEMPORAL))
        return -1;
    const v4i* src = static_cast<const v4i*>(buf);
    const size_t n16 = bytes / 16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
    const dim3 grid((unsigned)blocks);
    const bool nt = (flags & MOE_PROBE_NONTEMPORAL) != 0;
    switch (unroll) {
    case 1: launch<1>(nt, grid, st, e0, e1, src, n16, sink); break;
    case 2: launch<2>(nt, grid, st, e0, e1, src, n16, sink); break;
    case 4: launch<4>(nt, grid, st, e0, e1, src, n16, sink); break;
    case 8: launch<8>(nt, grid, st, e0, e1, src, n16, sink); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
