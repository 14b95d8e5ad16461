/*
 * ha_probe.h -- achievable-peak probes of libhybrid_attn.so.
 *
 * Not part of the attention path: measurement kernels that report what the
 * device sustains on the two resources the attention kernels are bound by (and
 * how the softmax's vector work shares a SIMD with the matrix cores),
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

/* The same MFMA chains (same grid, the same work: hybrid_attn_probe_mfma_flops)
 * on operands that change with every instruction: each lane cycles through 8
 * operand pairs of pseudo-random bf16 (random sign and mantissa, magnitudes in
 * [0.5, 4)), so the matrix cores' inputs toggle as on real data.  Their power
 * draw depends on that toggling: the rate this sustains under the part's power
 * limit is what a kernel streaming real data through the MFMAs can approach.
 * sink as for hybrid_attn_probe_mfma.  HA_EINVAL: as hybrid_attn_probe_mfma. */
HA_API int hybrid_attn_probe_mfma_data(int blocks, int iters, float* sink, hipStream_t stream);

/* Issue overlap of one SIMD: does the softmax's VALU work of the anchor run
 * while MFMAs execute, within one wave and between the waves of a SIMD?
 * `blocks` blocks (the CU count fills the part once) of 256 * waves_per_simd
 * threads; each block reserves 96 KB of LDS, so no CU holds two and every SIMD
 * runs waves_per_simd waves.  Each wave runs `iters` rounds; per round
 *   the MFMA part is 4 independent v_mfma_f32_32x32x16_bf16 on accumulators in
 *     VGPRs (4 x 32768 flop), as the anchor's;
 *   the VALU part is the anchor's work for 8 probabilities: 8 fused
 *     multiply-adds, 8 exp2, 4 bf16 pair packs and 4 dot2 row-sum steps, plus
 *     one add that moves the maximum they are taken against (25 instructions).
 * Modes: HA_PROBE_OVERLAP_MFMA, every wave the MFMA part only;
 * HA_PROBE_OVERLAP_VALU, the VALU part only; HA_PROBE_OVERLAP_BOTH, both in
 * every wave, one MFMA then a quarter of the VALU part; HA_PROBE_OVERLAP_SPLIT
 * (waves_per_simd = 2), per SIMD one wave the VALU part and the other the MFMA
 * part (roles taken from the SIMD id in the HW_ID register, not from the wave
 * index).  With the MFMA-only time t_m and the VALU-only time t_v of the same
 * grid, a mixed run takes t_m + t_v without overlap and max(t_m, t_v) with full
 * overlap (SPLIT does half the work of each: compare with the one-wave runs).
 * sink as for the MFMA probe.  HA_EINVAL: sink null, unknown mode,
 * waves_per_simd not 1 or 2 (SPLIT: not 2), blocks or iters outside the MFMA
 * probe's limits. */
#define HA_PROBE_OVERLAP_MFMA 0
#define HA_PROBE_OVERLAP_VALU 1
#define HA_PROBE_OVERLAP_BOTH 2
#define HA_PROBE_OVERLAP_SPLIT 3
HA_API int hybrid_attn_probe_overlap(int mode, int waves_per_simd, int blocks, int iters, float* sink,
                                     hipStream_t stream);

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
