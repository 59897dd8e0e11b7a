/*
 * m3_ssm_block.h -- the mixer with the Mamba-3 block's prologue and epilogue
 * fused into it (C ABI, AMD MI355X / gfx950).
 *
 * Mamba-3 review page (junhanzang.github.io, "Mamba-3: expressive SSM with
 * MIMO"), section 3.4 (Mamba-3 architecture): inside the Mamba-3 block the B
 * and C projections are followed by an RMS normalisation ("BC/QK
 * normalisation") and a learnable per-head, per-channel bias ("B, C biases")
 * before the data-dependent rotation; the mixer's output then passes the
 * block's output gate.  The pages give no formulas; this library takes:
 *
 *   B'_t[h][r][:] = B_t[h][r][:] / sqrt(mean_n B_t[h][r][n]^2 + eps)
 *                   * B_weight[h][r][:] + B_bias[h][r][:]        (same for C)
 *   y'_t          = y_t * silu(z_t),  silu(z) = z / (1 + exp(-z))
 *
 * with the normalisation over the N state channels of each (token, head,
 * rank) row, computed in fp32 from the I/O values; B', C' then enter the
 * mixer exactly as B, C do in m3_ssm.h (rotation, recurrence, outputs).
 * The carried state's prev_B holds the previous token's rotated B'.
 *
 * Every piece is optional: bc_norm = 0 skips the normalisation, a NULL
 * weight means 1, a NULL bias 0, a NULL z no gate.  Shapes, layouts,
 * ownership, threading and errors are those of m3_ssm.h; in addition
 *   B_weight, B_bias, C_weight, C_bias   [H][R][N] float32, 16-byte aligned
 *   z                                    like y: [b][T][H][R][P] (prefill),
 *                                        [b][H][R][P] (decode), I/O dtype
 * must stay valid until the stream reaches the call.  A NULL block pointer,
 * or a block with no piece present, gives exactly m3_ssm_prefill /
 * m3_ssm_decode_step.  M3_ERR_INVALID_ARGUMENT: a misaligned block pointer,
 * or eps < 0 or not finite with bc_norm set.  The block kernels also keep
 * the head's weight/bias table in LDS: with chunk = 64, a shape whose
 * 64-token chunk then no longer fits (bf16 I/O with N = 128, P = 64, R = 4,
 * and the fp32 shapes m3_ssm.h lists) takes chunks of qs(R) tokens, as
 * m3_ssm_prefill does; the workspace m3_ssm_prefill_workspace_bytes reports
 * serves both.  Every shape of m3_ssm.h is supported.
 */
#ifndef M3_SSM_BLOCK_H
#define M3_SSM_BLOCK_H

#include "m3_ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t bc_norm;        /* nonzero: RMS-normalise the B and C rows over N */
    float norm_eps;         /* eps inside the square root (e.g. 1e-6)          */
    const float *B_weight;  /* [H][R][N] or NULL (1) */
    const float *B_bias;    /* [H][R][N] or NULL (0) */
    const float *C_weight;  /* [H][R][N] or NULL (1) */
    const float *C_bias;    /* [H][R][N] or NULL (0) */
    const void *z;          /* output gate input, shaped like y, or NULL */
} m3_block_t;

/* m3_ssm_prefill with the block prologue on B, C and the gate on y. */
m3_status_t m3_ssm_prefill_block(const m3_shape_t *shape, const void *x, const void *dt,
                                 const float *A, const void *lam, const void *theta,
                                 const void *B, const void *C, const m3_block_t *block,
                                 const m3_state_t *init, m3_state_t *final_state, void *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* m3_ssm_decode_step with the block prologue on B, C and the gate on y. */
m3_status_t m3_ssm_decode_step_block(const m3_shape_t *shape, const void *x, const void *dt,
                                     const float *A, const void *lam, const void *theta,
                                     const void *B, const void *C, const m3_block_t *block,
                                     m3_state_t *state, void *y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_BLOCK_H */
