/*
 * m3_ssm_stages.h -- one stage of the chunked prefill at a time, for
 * measuring each kernel on its own (per-kernel time and bandwidth).
 *
 * m3_ssm_prefill (m3_ssm.h) enqueues four kernels in this order; together
 * they evaluate the chunkwise form of the SSD / masked-attention view of the
 * recurrence (Mamba-3 review, junhanzang.github.io, section 2.3 and section
 * 3.1.3, eq. (7); chunkwise algorithm on the "20.2 Mamba and S6" page,
 * sungeuns.github.io, section 2):
 *   M3_STAGE_CHUNK_COEF    per-chunk cumulative sum of log alpha = dt A, the
 *                          weights gamma_t and gamma_t + delta_{t+1}; folds the
 *                          carried state into the state entering chunk 0
 *   M3_STAGE_CHUNK_STATE   each chunk's own contribution to its end state and
 *                          its summed rotary angle (MFMA)
 *   M3_STAGE_STATE_SCAN    passes states from chunk to chunk; writes the
 *                          final carried state
 *   M3_STAGE_CHUNK_OUTPUT  intra-chunk masked contraction plus the incoming
 *                          state's contribution: y (MFMA)
 * Stage k reads what stages < k wrote into the workspace, so a full prefill is
 * the four stages in order with the same arguments.  Any single stage may be
 * enqueued again afterwards with the same arguments: CHUNK_COEF,
 * CHUNK_STATE and CHUNK_OUTPUT rewrite the same outputs; STATE_SCAN is not
 * repeatable on its own (it turns the chunk contributions into incoming
 * states in place) and must follow a CHUNK_STATE.
 *
 * Arguments, ownership and errors are those of m3_ssm_prefill; an unknown
 * stage gives M3_ERR_INVALID_ARGUMENT.
 */
#ifndef M3_SSM_STAGES_H
#define M3_SSM_STAGES_H

#include "m3_ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    M3_STAGE_CHUNK_COEF = 0,
    M3_STAGE_CHUNK_STATE = 1,
    M3_STAGE_STATE_SCAN = 2,
    M3_STAGE_CHUNK_OUTPUT = 3
} m3_stage_t;

m3_status_t m3_ssm_prefill_stage(int32_t stage, const m3_shape_t *shape, const void *x,
                                 const void *dt, const float *A, const void *lam,
                                 const void *theta, const void *B, const void *C,
                                 const m3_state_t *init, m3_state_t *final_state, void *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_STAGES_H */
