/*
 * m3_ssm_noalloc.h -- a prefill entry point that needs no caller-provided
 * workspace and allocates nothing.
 *
 * For callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * m3_ssm_prefill_noalloc is m3_ssm_prefill (m3_ssm.h: same shapes, layouts,
 * status codes, kernels and results) with its workspace -- the per-segment
 * aggregates of a sequence cut into segments, and the carried state at the
 * sequence start -- taken from a static device array of M3_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.  The
 * caller still passes every input and output.  The array's device address is
 * looked up once per device, on the first call with that device current.
 *
 * The workspace a shape needs (m3_ssm_prefill_workspace_bytes) is below about
 * 27 MB for every supported shape (segment aggregates below 16 MiB, the
 * carried state of fewer than 256 sequences), so every shape fits; a larger
 * need would return M3_ERR_WORKSPACE.
 *
 * Every call on one GPU shares that GPU's array: calls that can overlap on
 * one GPU (on different streams, or from different threads) race and must
 * not be issued.  Consecutive calls on one stream are safe.  Nothing in the
 * array needs to start at zero: every byte a call reads is written earlier in
 * the same call.  Errors: as m3_ssm_prefill, plus M3_ERR_HIP when the array's
 * address cannot be found on the current device.
 */
#ifndef M3_SSM_NOALLOC_H
#define M3_SSM_NOALLOC_H

#include "m3_ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define M3_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB per GPU */

m3_status_t m3_ssm_prefill_noalloc(const m3_shape_t *shape, const void *x, const void *dt,
                                   const float *A, const void *lam, const void *theta,
                                   const void *B, const void *C, const m3_state_t *init,
                                   m3_state_t *final_state, void *y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_NOALLOC_H */
