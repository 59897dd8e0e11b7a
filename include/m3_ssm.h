/*
 * m3_ssm.h -- C ABI of the Mamba-3 SSM sequence mixer for AMD MI355X (gfx950).
 *
 * The mixer is the Mamba-3 selective state-space recurrence as defined on the
 * Mamba-3 review page (junhanzang.github.io, "Mamba-3: expressive SSM with
 * MIMO"):
 *   - section 3.1.1, Proposition 3.1.1, eqs. (5)-(6): the exponential-
 *     trapezoidal recurrence
 *         h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t,
 *         alpha_t = exp(dt_t A), beta_t = (1 - lam_t) dt_t alpha_t,
 *         gamma_t = lam_t dt_t,          y_t = C_t^T h_t;
 *   - section 3.2, Propositions 3.2.1-3.2.3: the complex-valued state, realised
 *     as a data-dependent rotary rotation of B_t and C_t by the cumulative
 *     angle Phi_t = Phi_{-1} + sum_{s<=t} theta_s of each adjacent row pair
 *     (2k, 2k+1) of the N state rows (rotation by +theta is counter-clockwise);
 *   - section 3.3: MIMO -- B_t, C_t are N x R, x_t is R x P, the state update
 *     is the rank-R product sum_r B[:, r] x[r, :], and y_t has R rows
 *     y_t[i, :] = C_t[:, i]^T h_t.  SISO is R = 1.
 * The chunked prefill is the SSD (masked attention) form of section 2.3 with
 * the mask of section 3.1.3, eq. (7) (decay matrix times 2-band matrix),
 * evaluated chunk by chunk; see also the chunked algorithm on the
 * "20.2 Mamba and S6" page (sungeuns.github.io), section 2.
 *
 * Conventions used by every entry point
 * -------------------------------------
 * Tensors are device pointers (HBM), row-major and contiguous, 16-byte
 * aligned.  Sizes: b = batch, T = seqlen, H = nheads, P = headdim,
 * N = dstate (even), R = rank, K = N / 2 rotation pairs.
 *     x, y          [b][T][H][R][P]    I/O dtype
 *     B, C          [b][T][G][R][N]    I/O dtype   (B[..][r][n] is B_t[n, r])
 *     dt, lam       [b][T][H]          I/O dtype
 *     theta         [b][T][H][K]       I/O dtype   (angle of pair k, radians)
 *     A             [H]                float32     (one decay rate per head)
 * G = ngroups divides H (0 means G = H): head h reads the B and C of group
 * h / (H / G), as the shared B, C projection of the MIMO instantiation in the
 * Mamba-3 review (section 3.3) suggests; every head keeps its own dt, lam,
 * theta, A, x and state, so a group's B and C still rotate per head.
 * The per-step rotation angle is theta_t itself; a caller that wants
 * dt_t * theta_t passes the product.  Decode calls drop the T axis.
 *
 * Preconditions that are not checked (values are computed as given):
 * dt > 0, 0 <= lam <= 1, A <= 0.  With A > 0 the decay factors can overflow.
 *
 * Carried state (m3_state_t) is kept in the rotated (RoPE) frame
 *     h~ = R(-Phi) h,   Phi wrapped to [-pi, pi),
 * together with the previous token's rotated B~ and its x, which the beta
 * term of the next token needs (eq. (6)).  A zero state with zero prev_B is a
 * fresh sequence.
 *
 * Ownership and threading: the caller owns every buffer, including the
 * workspace.  The library never allocates, frees or synchronises; it enqueues
 * kernels on the given stream and returns.  Buffers must stay valid until the
 * stream reaches that point.  Inputs must not alias outputs, except that the
 * final state of a prefill may alias its initial state (in-place update).
 * The library keeps no global state and is thread-safe.
 *
 * Errors: every entry point returns an m3_status_t and never aborts.  Kernel
 * faults are asynchronous and surface at the caller's next synchronisation.
 */
#ifndef M3_SSM_H
#define M3_SSM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* I/O element type of x, y, B, C, dt, lam, theta and prev_x. */
typedef enum {
    M3_DTYPE_F32 = 0,
    M3_DTYPE_BF16 = 1
} m3_dtype_t;

typedef enum {
    M3_OK = 0,
    M3_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, odd N, size < 1, bad dtype */
    M3_ERR_UNSUPPORTED = 2,      /* shape outside the compiled set (see below)          */
    M3_ERR_WORKSPACE = 3,        /* workspace pointer null or too small                 */
    M3_ERR_HIP = 4               /* a kernel launch failed                              */
} m3_status_t;

/* Problem size.  Supported: headdim P in {16, 32, 64}; dstate N in
 * {16, 32, 64, 128}; rank R in 1..4, in both I/O types; any batch >= 1,
 * nheads >= 1 and seqlen >= 1 (a ragged last chunk is masked).  io_dtype is
 * an m3_dtype_t value.
 * chunk is the chunk length Q in tokens of the chunked (SSD) form, 64 or the
 * rank's small chunk qs(R) = 64 / R tokens (R = 3: 32), i.e. 64 virtual
 * (token, rank) rows, the chunk that the Mamba-3 review's FLOP count for MIMO
 * (section 3.3, R times the SISO cost) describes.  A prefill workgroup keeps
 * one chunk's operands in the 160 KB of LDS of a gfx950 compute unit; with
 * chunk = 64, shapes whose 64-token chunk does not fit (with fp32 I/O: N = 64
 * with R = 4, N = 128 with R >= 2) take chunks of qs(R) tokens.  qs(R)
 * divides 64, so either chunking gives the same result up to rounding.
 * Another chunk value is M3_ERR_UNSUPPORTED.
 * Element offsets within one token are 32-bit: 64 * nheads * R * max(N, P)
 * (and 64 * ngroups * R * N) must stay below 2^31, else M3_ERR_UNSUPPORTED.
 * ngroups < 0 or not dividing nheads is M3_ERR_INVALID_ARGUMENT.
 * state_dtype BF16 keeps h~ in bf16 (round to nearest even at every store;
 * all arithmetic stays fp32): half the state traffic of a decode step, at a
 * rounding error of about 2^-9 of the state per store.  Phi and prev_B stay
 * fp32.  Another value is M3_ERR_INVALID_ARGUMENT. */
typedef struct {
    int64_t batch;
    int64_t seqlen;   /* T; ignored by m3_ssm_decode_step */
    int32_t nheads;   /* H */
    int32_t headdim;  /* P */
    int32_t dstate;   /* N, even */
    int32_t rank;     /* R, 1 = SISO */
    int32_t chunk;    /* Q: 64, or qs(R) = 64 / R tokens (R = 3: 32) */
    int32_t io_dtype; /* m3_dtype_t */
    int32_t ngroups;  /* G: B and C shared by groups of H/G consecutive heads; 0 = H */
    int32_t state_dtype; /* m3_dtype_t of the carried state h~: F32 (0, default) or BF16 */
} m3_shape_t;

/* Carried state of one batch of sequences (caller-owned device buffers). */
typedef struct {
    void  *h;       /* [b][H][N][P]  rotated-frame state h~ = R(-Phi) h, state_dtype  */
    float *phi;     /* [b][H][K]     cumulative angle Phi, wrapped to [-pi, pi)       */
    float *prev_B;  /* [b][H][R][N]  rotated B~ = R(-Phi) B of the last consumed token */
    void  *prev_x;  /* [b][H][R][P]  x of the last consumed token (I/O dtype)          */
} m3_state_t;

/* Bytes of device workspace m3_ssm_prefill needs for this shape (0 if the
 * shape is invalid or unsupported).  When batch * nheads is too small to fill
 * the GPU (below 256), each sequence is cut into S segments of whole chunks;
 * the workspace holds each segment's aggregate (an N x P fp32 state, its
 * summed log decay and rotation angle) and the carried state at the sequence
 * start.  The pre-pass may cut each segment into pieces with an aggregate
 * each, when that fills the GPU in whole rounds (m3_ssm_stages.h).  It is
 * sized for both the plain and the block kernels' plans, so it serves
 * m3_ssm_prefill_block too; the aggregates stay below 16 MiB and the whole
 * workspace below about 27 MB.  With S = 1 it is 256 bytes, unused. */
size_t m3_ssm_prefill_workspace_bytes(const m3_shape_t *shape);

/*
 * Chunked (SSD-form) prefill over T tokens of every (batch, head).
 *   init        NULL: fresh sequence (zero state, Phi = 0, no previous token).
 *               Otherwise the carried state to start from (read only).
 *   final_state NULL: not written.  Otherwise receives the state after the
 *               last token (h~, Phi, prev_B, prev_x); may alias init.
 *   y           output [b][T][H][R][P], I/O dtype.
 *   workspace   device buffer of at least m3_ssm_prefill_workspace_bytes().
 *   stream      HIP stream the kernels are enqueued on (0 = default stream).
 * Returns M3_OK once every kernel has been enqueued.
 */
m3_status_t m3_ssm_prefill(const m3_shape_t *shape, const void *x, const void *dt,
                           const float *A, const void *lam, const void *theta,
                           const void *B, const void *C, const m3_state_t *init,
                           m3_state_t *final_state, void *y, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step: consumes token t for every (batch, head), updating the
 * carried state in place, and writes y_t.  Inputs drop the T axis:
 * x [b][H][R][P], dt/lam [b][H], theta [b][H][K], B/C [b][G][R][N].
 * Equivalent to m3_ssm_prefill with seqlen = 1, init = final_state = state.
 * shape->seqlen is ignored; state must not be NULL.
 */
m3_status_t m3_ssm_decode_step(const m3_shape_t *shape, const void *x, const void *dt,
                               const float *A, const void *lam, const void *theta,
                               const void *B, const void *C, m3_state_t *state,
                               void *y, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char *m3_status_string(m3_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* M3_SSM_H */
