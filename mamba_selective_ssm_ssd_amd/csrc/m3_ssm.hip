// m3_ssm.hip -- C ABI of the mixer: argument validation, workspace layout and
// the launch sequence.  See include/m3_ssm.h for the contract.
//
// Prefill enqueues, on the caller's stream:
//   1. k_chunk_coef    per-chunk cumsum of log alpha, gamma, trapezoid weights;
//                      folds the carried state into the state entering chunk 0
//   2. k_chunk_state   per-chunk state contribution U_c (MFMA), chunk angles
//   3. k_state_scan    inter-chunk state passing; final carried state
//   4. k_chunk_output  intra-chunk masked contraction + incoming state (MFMA)
// Decode enqueues one k_decode_step.  m3_ssm_prefill_stage enqueues one of
// the four prefill kernels alone (include/m3_ssm_stages.h).
#include "../../include/m3_ssm.h"
#include "../../include/m3_ssm_stages.h"
#include "m3_internal.hpp"

#include <limits>

namespace {

using m3::PrefillParams;
using m3::WorkspaceLayout;

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the shape.  Returns M3_OK or the error to report.
m3_status_t check_shape(const m3_shape_t *s, bool decode) {
    if (!s) return M3_ERR_INVALID_ARGUMENT;
    if (s->io_dtype != M3_DTYPE_F32 && s->io_dtype != M3_DTYPE_BF16) return M3_ERR_INVALID_ARGUMENT;
    if (s->batch < 1 || s->nheads < 1 || s->headdim < 1 || s->dstate < 2 || s->rank < 1)
        return M3_ERR_INVALID_ARGUMENT;
    if (!decode && s->seqlen < 1) return M3_ERR_INVALID_ARGUMENT;
    if (s->dstate % 2 != 0) return M3_ERR_INVALID_ARGUMENT;
    if (s->chunk < 1) return M3_ERR_INVALID_ARGUMENT;
    if (s->chunk != 64) return M3_ERR_UNSUPPORTED;
    if (!m3::supported_N(s->dstate) || !m3::supported_P(s->headdim) || s->rank > 4)
        return M3_ERR_UNSUPPORTED;
    // every grid dimension and element offset must stay in range
    const double bh = double(s->batch) * double(s->nheads);
    const double T = decode ? 1.0 : double(s->seqlen);
    const double elems = bh * T * double(s->rank) * double(s->dstate > s->headdim ? s->dstate : s->headdim);
    if (elems > 4.0e18) return M3_ERR_UNSUPPORTED;
    if (!decode) {
        // the chunk kernels stage a whole chunk in LDS
        const bool bf = s->io_dtype == M3_DTYPE_BF16;
        const size_t a = m3::chunk_state_lds_bytes(bf, s->dstate, s->headdim, s->rank);
        const size_t b = m3::chunk_output_lds_bytes(bf, s->dstate, s->headdim, s->rank);
        if (a == 0 || b == 0 || a > m3::kMaxLdsBytes || b > m3::kMaxLdsBytes) return M3_ERR_UNSUPPORTED;
    }
    if (bh * ((T + 63.0) / 64.0) > double(std::numeric_limits<unsigned>::max()) / 2) return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

WorkspaceLayout layout(const m3_shape_t *s) {
    const size_t bh = size_t(s->batch) * size_t(s->nheads);
    const size_t T = size_t(s->seqlen);
    const size_t nC = (T + 63) / 64;
    const size_t N = size_t(s->dstate), P = size_t(s->headdim), K = N / 2;
    WorkspaceLayout w;
    size_t off = 0;
    w.ell = off; off += round_up(bh * T * sizeof(float));
    w.gam = off; off += round_up(bh * T * sizeof(float));
    w.wgt = off; off += round_up(bh * T * sizeof(float));
    w.ubuf = off; off += round_up(bh * nC * N * P * sizeof(float));
    w.thetaC = off; off += round_up(bh * nC * K * sizeof(double));
    w.thetaCS = off; off += round_up(bh * nC * K * sizeof(float) * 2);
    w.hinit = off; off += round_up(bh * N * P * sizeof(float));
    w.phi0 = off; off += round_up(bh * K * sizeof(double));
    w.total = off;
    return w;
}

bool state_ok(const m3_state_t *st) {
    return st->h && st->phi && st->prev_B && st->prev_x && aligned16(st->h) && aligned16(st->phi) &&
           aligned16(st->prev_B) && aligned16(st->prev_x);
}

} // namespace

extern "C" {

const char *m3_status_string(m3_status_t status) {
    switch (status) {
    case M3_OK: return "M3_OK";
    case M3_ERR_INVALID_ARGUMENT: return "M3_ERR_INVALID_ARGUMENT";
    case M3_ERR_UNSUPPORTED: return "M3_ERR_UNSUPPORTED";
    case M3_ERR_WORKSPACE: return "M3_ERR_WORKSPACE";
    case M3_ERR_HIP: return "M3_ERR_HIP";
    }
    return "M3_ERR_UNKNOWN";
}

size_t m3_ssm_prefill_workspace_bytes(const m3_shape_t *shape) {
    if (check_shape(shape, false) != M3_OK) return 0;
    return layout(shape).total;
}

// Validates a prefill call and resolves its parameters.
static m3_status_t prepare_prefill(const m3_shape_t *shape, const void *x, const void *dt,
                                   const float *A, const void *lam, const void *theta,
                                   const void *B, const void *C, const m3_state_t *init,
                                   m3_state_t *final_state, void *y, void *workspace,
                                   size_t workspace_bytes, PrefillParams &p) {
    const m3_status_t sc = check_shape(shape, false);
    if (sc != M3_OK) return sc;
    const void *ptrs[] = {x, dt, A, lam, theta, B, C, y};
    for (const void *q : ptrs)
        if (!q || !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    if (init && !state_ok(init)) return M3_ERR_INVALID_ARGUMENT;
    if (final_state && !state_ok(final_state)) return M3_ERR_INVALID_ARGUMENT;
    const WorkspaceLayout w = layout(shape);
    if (!workspace || !aligned16(workspace) || workspace_bytes < w.total) return M3_ERR_WORKSPACE;

    p = PrefillParams{};
    p.batch = shape->batch;
    p.T = shape->seqlen;
    p.H = shape->nheads;
    p.P = shape->headdim;
    p.N = shape->dstate;
    p.R = shape->rank;
    p.K = p.N / 2;
    p.nC = int32_t((p.T + 63) / 64);
    p.x = x; p.dt = dt; p.lam = lam; p.theta = theta; p.B = B; p.C = C; p.A = A; p.y = y;
    p.has_init = init != nullptr;
    if (init) {
        p.h0 = init->h; p.phi0 = init->phi; p.prevB0 = init->prev_B; p.prevx0 = init->prev_x;
    }
    p.has_final = final_state != nullptr;
    if (final_state) {
        p.hT = final_state->h; p.phiT = final_state->phi; p.prevBT = final_state->prev_B;
        p.prevxT = final_state->prev_x;
    }
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.ell = reinterpret_cast<float *>(ws + w.ell);
    p.gam = reinterpret_cast<float *>(ws + w.gam);
    p.wgt = reinterpret_cast<float *>(ws + w.wgt);
    p.ubuf = reinterpret_cast<float *>(ws + w.ubuf);
    p.thetaC = reinterpret_cast<double *>(ws + w.thetaC);
    p.thetaCS = reinterpret_cast<float2 *>(ws + w.thetaCS);
    p.hinit = reinterpret_cast<float *>(ws + w.hinit);
    p.phi0ws = reinterpret_cast<double *>(ws + w.phi0);
    return M3_OK;
}

static hipError_t launch_stage(int32_t stage, const PrefillParams &p, bool bf, hipStream_t stream) {
    switch (stage) {
    case M3_STAGE_CHUNK_COEF: return m3::launch_chunk_coef(p, bf, stream);
    case M3_STAGE_CHUNK_STATE: return m3::launch_chunk_state(p, bf, stream);
    case M3_STAGE_STATE_SCAN: return m3::launch_state_scan(p, bf, stream);
    case M3_STAGE_CHUNK_OUTPUT: return m3::launch_chunk_output(p, bf, stream);
    }
    return hipErrorInvalidValue;
}

m3_status_t m3_ssm_prefill(const m3_shape_t *shape, const void *x, const void *dt, const float *A,
                           const void *lam, const void *theta, const void *B, const void *C,
                           const m3_state_t *init, m3_state_t *final_state, void *y,
                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    PrefillParams p;
    const m3_status_t sc = prepare_prefill(shape, x, dt, A, lam, theta, B, C, init, final_state, y,
                                           workspace, workspace_bytes, p);
    if (sc != M3_OK) return sc;
    const bool bf = shape->io_dtype == M3_DTYPE_BF16;
    for (int32_t stage = M3_STAGE_CHUNK_COEF; stage <= M3_STAGE_CHUNK_OUTPUT; ++stage)
        if (launch_stage(stage, p, bf, stream) != hipSuccess) return M3_ERR_HIP;
    return M3_OK;
}

m3_status_t m3_ssm_prefill_stage(int32_t stage, const m3_shape_t *shape, const void *x,
                                 const void *dt, const float *A, const void *lam,
                                 const void *theta, const void *B, const void *C,
                                 const m3_state_t *init, m3_state_t *final_state, void *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (stage < M3_STAGE_CHUNK_COEF || stage > M3_STAGE_CHUNK_OUTPUT) return M3_ERR_INVALID_ARGUMENT;
    PrefillParams p;
    const m3_status_t sc = prepare_prefill(shape, x, dt, A, lam, theta, B, C, init, final_state, y,
                                           workspace, workspace_bytes, p);
    if (sc != M3_OK) return sc;
    if (launch_stage(stage, p, shape->io_dtype == M3_DTYPE_BF16, stream) != hipSuccess) return M3_ERR_HIP;
    return M3_OK;
}

m3_status_t m3_ssm_decode_step(const m3_shape_t *shape, const void *x, const void *dt, const float *A,
                               const void *lam, const void *theta, const void *B, const void *C,
                               m3_state_t *state, void *y, hipStream_t stream) {
    const m3_status_t sc = check_shape(shape, true);
    if (sc != M3_OK) return sc;
    const void *ptrs[] = {x, dt, A, lam, theta, B, C, y};
    for (const void *q : ptrs)
        if (!q || !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    if (!state || !state_ok(state)) return M3_ERR_INVALID_ARGUMENT;
    m3::DecodeParams p{};
    p.batch = shape->batch;
    p.H = shape->nheads;
    p.P = shape->headdim;
    p.N = shape->dstate;
    p.R = shape->rank;
    p.K = p.N / 2;
    p.x = x; p.dt = dt; p.lam = lam; p.theta = theta; p.B = B; p.C = C; p.A = A; p.y = y;
    p.h = state->h; p.phi = state->phi; p.prevB = state->prev_B; p.prevx = state->prev_x;
    if (m3::launch_decode_step(p, shape->io_dtype == M3_DTYPE_BF16, stream) != hipSuccess) return M3_ERR_HIP;
    return M3_OK;
}

} // extern "C"
