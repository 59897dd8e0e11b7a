/*
 * m3_ssm_ceilings.h -- on-chip ceilings the mixer's kernels are measured
 * against: an MFMA-only loop and a streaming copy / read-modify-write.
 *
 * The roofline of the mixer (the arithmetic intensity of its chunked prefill
 * and of its decode step, Mamba-3 review, section 3.3) places each kernel
 * under the matrix-core peak or the HBM bandwidth.  Next to the spec-sheet
 * peaks, these kernels give what this GPU reaches with plain code: the MFMA
 * instructions the mixer's kernels issue, back to back with no memory
 * traffic, and a float4 stream with no arithmetic to speak of.
 *
 * Conventions as in m3_ssm.h: device pointers, caller-owned buffers, work
 * enqueued on the given stream, no allocation and no synchronisation, an
 * m3_status_t return (M3_ERR_INVALID_ARGUMENT for a null or misaligned
 * pointer or a size out of range, M3_ERR_HIP for a failed launch).
 */
#ifndef M3_SSM_CEILINGS_H
#define M3_SSM_CEILINGS_H

#include "m3_ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA-only loop.  kind 0: v_mfma_f32_16x16x32_bf16 (16384 flops per wave
 * instruction), kind 1: v_mfma_f32_16x16x4_f32 (2048 flops).  nblocks
 * workgroups of 256 threads; every wave issues iters x 8 MFMAs on 8
 * independent accumulators and writes one float per thread to sink
 * (nblocks * 256 floats).  Flops of the launch:
 * nblocks * 4 * iters * 8 * (flops per instruction). */
m3_status_t m3_ceiling_mfma(int32_t kind, int32_t nblocks, int32_t iters, float *sink,
                            hipStream_t stream);

/* Stream of n float4 (16-byte) elements.  mode 0: dst = src (reads and
 * writes 16 n bytes each); mode 1: dst = dst * 1.0001f + 1e-7f in place
 * (reads and writes dst; src unused, may be NULL); modes 2 and 3: the same
 * as 0 and 1 with non-temporal loads and stores (global_load/store ... nt),
 * the streaming cache hints some of the mixer's kernels use.  Grid-stride
 * over nblocks workgroups of 256 threads, 8 float4 per thread per trip. */
m3_status_t m3_ceiling_stream(int32_t mode, const void *src, void *dst, int64_t n,
                              int32_t nblocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_CEILINGS_H */
