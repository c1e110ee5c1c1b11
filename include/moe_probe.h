/*
 * moe_probe.h - HBM read probe of libmoe (measurement only; not part of the
 * layer).
 *
 * Source: "Sync upstream Strata v0.1.39 into Lanes" (Strata-Lanes pull request
 * 24), the SYCL port commits: a bandwidth probe over incompressible data with
 * 4-byte and 16-byte loads; the wide loads streamed faster, and the expert
 * matrix-vector kernels were judged against that probe.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_PROBE_NONTEMPORAL = 1 };   /* flags: streaming (non-temporal) loads */

/*
 * One kernel launch on `stream` (a hipStream_t as void*, NULL = the null
 * stream) that reads `bytes` of device memory at `buf` with 16-byte loads:
 * `blocks` workgroups of 256 threads walk the buffer in a grid-stride loop,
 * each thread keeping `unroll` (1, 2, 4 or 8) loads in flight; `flags` 0 or
 * MOE_PROBE_NONTEMPORAL (loads marked streaming, the form the expert kernels
 * do not use, to compare with).  Each thread
 * writes one uint32 (the xor of what it read) to `sink`, a device buffer of
 * blocks * 256 words that the caller owns.  buf must be 16-byte aligned and
 * bytes a multiple of 16.  ev_start / ev_stop (hipEvent_t as void*, or NULL)
 * are recorded by the launch's own dispatch, so their elapsed time is the
 * kernel's duration.  Asynchronous.  Returns 0, -1 for a bad argument, -4 when
 * the launch fails.
 */
int moe_probe_read(const void* buf, size_t bytes, int blocks, int unroll, int flags,
                   uint32_t* sink, void* stream, void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H */
