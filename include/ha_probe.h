/*
 * ha_probe.h -- achievable-peak probes of libhybrid_attn.so.
 *
 * Not part of the attention path: three measurement kernels that report what
 * the device sustains on the two resources the attention kernels are bound by,
 * so that a kernel's rate can be read against the published peak and against
 * what this part delivers under its own clock and power limit.  The caller
 * times them (e.g. with HIP events on `stream`) and divides the work by the
 * time.  Same conventions as hybrid_attn.h: the caller owns every buffer, work
 * is enqueued asynchronously on `stream` of the current device, arguments are
 * checked on the host before anything is enqueued, and the status codes are
 * those of ha_status.
 */
#ifndef HA_PROBE_H
#define HA_PROBE_H

#include "hybrid_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Limits of the MFMA probe's arguments (HA_EINVAL beyond them). */
#define HA_PROBE_MAX_BLOCKS (1 << 20)
#define HA_PROBE_MAX_ITERS (1 << 24)

/* Floating-point operations one hybrid_attn_probe_mfma call performs:
 * blocks x 4 waves x 4 chains x iters x (2 x 32 x 32 x 16).  0 for arguments
 * outside [1, HA_PROBE_MAX_BLOCKS] x [1, HA_PROBE_MAX_ITERS]. */
HA_API double hybrid_attn_probe_mfma_flops(int blocks, int iters);

/* MFMA throughput: `blocks` blocks of 256 threads, each wave running `iters`
 * rounds of 4 independent v_mfma_f32_32x32x16_bf16 (bf16 products, fp32
 * accumulation) on register operands, with no memory traffic.  sink: one float
 * of device memory, written only in a case that does not occur (it keeps the
 * work from being optimised away); its value is meaningless.
 * HA_EINVAL: sink null, blocks or iters outside their limits. */
HA_API int hybrid_attn_probe_mfma(int blocks, int iters, float* sink, hipStream_t stream);

/* HBM read bandwidth: reads `bytes` bytes of device memory at src once, as
 * 16-byte words, four in flight per thread; sink as above.  bytes = 0 enqueues
 * nothing.  HA_EINVAL: src or sink null.  HA_EALIGN: src not 16-byte aligned
 * or bytes not a multiple of 16. */
HA_API int hybrid_attn_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream);

/* HBM copy bandwidth: copies `bytes` bytes from src to dst (device memory,
 * non-overlapping) as 16-byte words, four in flight per thread, with ordinary
 * accesses (nontemporal = 0) or non-temporal loads and stores (nontemporal != 0);
 * dst then equals src bitwise.  The HBM traffic is 2 x bytes.  bytes = 0
 * enqueues nothing.  HA_EINVAL: src or dst null, or the ranges overlap.
 * HA_EALIGN: src or dst not 16-byte aligned, or bytes not a multiple of 16. */
HA_API int hybrid_attn_probe_copy(const void* src, void* dst, size_t bytes, int nontemporal,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HA_PROBE_H */
