/*
 * m3_ssm_backward.h -- gradients of the Mamba-3 SSM sequence mixer (C ABI,
 * AMD MI355X / gfx950).
 *
 * For the prefill map of m3_ssm.h (the exponential-trapezoidal recurrence of
 * the Mamba-3 review, section 3.1.1, eqs. (5)-(6), with the complex state as
 * the rotation of B and C of section 3.2.2, Prop. 3.2.3, and the rank-R
 * products of section 3.3) and a given upstream gradient gy of y, this
 * computes the gradients of L = sum(gy * y) with respect to every input and
 * to the carried state the call starts from (the training half of the
 * prefill, as in the chunked algorithm of the "20.2 Mamba and S6" page,
 * section 2, whose prefill kernels are trained through).
 *
 * The gradients of the final state's outputs are not inputs (L depends on y
 * only).  Supported: the shapes m3_ssm_prefill supports, ngroups = 0 or H,
 * state_dtype F32; otherwise M3_ERR_UNSUPPORTED.  Arithmetic is fp32 with
 * fp64 angles; every gradient is written in fp32.
 */
#ifndef M3_SSM_BACKWARD_H
#define M3_SSM_BACKWARD_H

#include "m3_ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Gradient outputs, fp32, caller-owned, 16-byte aligned; shapes as the
 * matching inputs.  A is summed over batch and tokens.  The four carried-
 * state gradients may be NULL (not written); the others are required. */
typedef struct {
    float *x;      /* [b][T][H][R][P] */
    float *dt;     /* [b][T][H]       */
    float *A;      /* [H]             */
    float *lam;    /* [b][T][H]       */
    float *theta;  /* [b][T][H][K]    */
    float *B;      /* [b][T][H][R][N] */
    float *C;      /* [b][T][H][R][N] */
    float *h;      /* [b][H][N][P]  of the initial state's h~ (rotated frame) */
    float *phi;    /* [b][H][K]     of its Phi                                */
    float *prev_B; /* [b][H][R][N]  of its rotated previous B                 */
    float *prev_x; /* [b][H][R][P]  of its previous x                         */
} m3_grads_t;

/* Bytes of device workspace m3_ssm_prefill_backward needs (0: unsupported).
 * The pass stores the state entering every chunk of 32 / R tokens in fp32
 * and the angle there in fp64, so the size grows with the sequence:
 * batch * H * ceil(T / (32 / R)) * (N * P * 4 + N / 2 * 8) bytes, plus
 * alignment and 4 bytes per (batch, head).  The workspace is caller-owned
 * and needs no initialisation. */
size_t m3_ssm_prefill_backward_workspace_bytes(const m3_shape_t *shape);

/*
 * Gradients of L = sum(gy * y) for y = m3_ssm_prefill(shape, x, ..., init).
 *   init   NULL: a fresh sequence; otherwise the carried state (read only).
 *   gy     [b][T][H][R][P], I/O dtype.
 *   grads  outputs (see m3_grads_t); the carried-state entries are written
 *          only when init is given and the pointer is not NULL.
 * Returns M3_OK once the kernels are enqueued on stream.  Errors as in
 * m3_ssm.h; M3_ERR_WORKSPACE for a workspace below the size above.
 */
m3_status_t m3_ssm_prefill_backward(const m3_shape_t *shape, const void *x, const void *dt,
                                    const float *A, const void *lam, const void *theta,
                                    const void *B, const void *C, const m3_state_t *init,
                                    const void *gy, const m3_grads_t *grads, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_BACKWARD_H */
