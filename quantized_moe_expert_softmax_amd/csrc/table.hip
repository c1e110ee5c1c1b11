// Expert-address table of libmoe: the device array of E pack addresses that
// the table form of the layer call reads (expert e's pack at table[e]).  The
// expert cache rewrites entries with these kernels, in stream order after the
// copies that fill a slot, so that no call sees an entry before its pack.
#include "kernels.h"

namespace moe {

__global__ void k_table_fill(const uint8_t** table, int E, const uint8_t* base, size_t stride) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) table[e] = base + (size_t)e * stride;
}

// the updates travel as kernel arguments: nothing on the host has to outlive
// the launch
__global__ void k_table_set(const uint8_t** table, TableUpdate u) {
    const int i = threadIdx.x;
    if (i < u.n) table[u.expert[i]] = u.addr[i];
}

hipError_t launch_table_fill(const uint8_t** table, int E, const uint8_t* base, size_t stride,
                             hipStream_t st) {
    if (E <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_table_fill, dim3((E + 255) / 256), dim3(256), 0, st, table, E, base, stride);
    return hipGetLastError();
}

hipError_t launch_table_set(const uint8_t** table, const TableUpdate& u, hipStream_t st) {
    if (u.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_table_set, dim3(1), dim3(TABLE_UPDATE_MAX), 0, st, table, u);
    return hipGetLastError();
}

}  // namespace moe
