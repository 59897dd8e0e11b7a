/*
 * m3_ssm_stages.h -- one stage of the chunked prefill at a time, for
 * measuring each kernel on its own (per-kernel time and bandwidth).
 *
 * m3_ssm_prefill (m3_ssm.h) evaluates the chunkwise form of the SSD /
 * masked-attention view of the recurrence (Mamba-3 review,
 * junhanzang.github.io, section 2.3 and section 3.1.3, eq. (7); chunkwise
 * algorithm on the "20.2 Mamba and S6" page, sungeuns.github.io, section 2)
 * with one persistent workgroup per (batch, head, segment of chunks) that
 * passes the state from chunk to chunk on chip.  It enqueues, in order:
 *   M3_STAGE_SEGMENT_STATE  when batch * heads is too small to fill the chip,
 *                           every sequence is cut into segments and this
 *                           pre-pass computes each segment's (or each piece
 *                           of a segment's) aggregate (its
 *                           state from a zero start, summed log decay and
 *                           rotary angle) and the carried state in its own
 *                           frame; it enqueues nothing when there is one
 *                           segment per sequence
 *   M3_STAGE_OUTPUT         per segment: folds the aggregates before it into
 *                           its starting state, then per chunk the decay and
 *                           angle prefixes, the rotation of B and C, the
 *                           intra-chunk masked contraction and the incoming-
 *                           state term (MFMA), writing y; the last segment
 *                           writes the final carried state
 * The segmentation depends on the shape only (m3_ssm_prefill_plan reports
 * it, with each stage's chunk length).  Running the stages in order
 * with the same arguments is a full prefill; either stage may be enqueued
 * again afterwards with the same arguments and rewrites the same outputs.
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
    M3_STAGE_SEGMENT_STATE = 0,
    M3_STAGE_OUTPUT = 1
} m3_stage_t;

/* How m3_ssm_prefill runs a shape with the plain kernels (with_block = 0)
 * or with the block kernels (with_block != 0: a call of m3_ssm_prefill_block
 * whose block has at least one piece): tokens per chunk of the pre-pass and
 * of the output pass (64 or m3_ssm.h's qs(R)), segments per sequence (1: no
 * pre-pass is enqueued), tokens per segment (the last segment may be
 * shorter) and the pieces the pre-pass cuts each of the first segments - 1
 * segments into (one workgroup and one aggregate per piece; more pieces than
 * one when that fills the compute units in whole rounds).  Any output pointer
 * may be NULL.  Errors: those of the shape check of m3_ssm_prefill. */
m3_status_t m3_ssm_prefill_plan(const m3_shape_t *shape, int32_t with_block, int32_t *chunk_pre,
                                int32_t *chunk_out, int32_t *segments, int64_t *segment_tokens,
                                int32_t *prepass_pieces);

m3_status_t m3_ssm_prefill_stage(int32_t stage, const m3_shape_t *shape, const void *x,
                                 const void *dt, const float *A, const void *lam,
                                 const void *theta, const void *B, const void *C,
                                 const m3_state_t *init, m3_state_t *final_state, void *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_STAGES_H */
