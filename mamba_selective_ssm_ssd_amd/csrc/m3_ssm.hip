// m3_ssm.hip -- C ABI of the mixer: argument validation, workspace layout and
// the launch sequence.  See include/m3_ssm.h for the contract.
//
// Prefill enqueues, on the caller's stream, the fused chunked kernel
// k_prefill (k_prefill.hpp): one persistent workgroup per (batch, head,
// segment of chunks) that carries the state across its chunks on chip.  When
// batch * heads is too small to fill the chip, each sequence is cut into S
// segments and a pre-pass of the same kernel first computes every segment's
// aggregate.  Decode enqueues one k_decode_step.  m3_ssm_prefill_stage
// enqueues one of the two prefill kernels alone (include/m3_ssm_stages.h).
#include "m3_ssm.h"
#include "m3_ssm_block.h"
#include "m3_ssm_backward.h"
#include "m3_ssm_stages.h"
#include "k_prefill.hpp"
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
    if (s->ngroups < 0 || (s->ngroups > 0 && s->nheads % s->ngroups != 0)) return M3_ERR_INVALID_ARGUMENT;
    if (s->state_dtype != M3_DTYPE_F32 && s->state_dtype != M3_DTYPE_BF16) return M3_ERR_INVALID_ARGUMENT;
    if (s->chunk != 64) return M3_ERR_UNSUPPORTED;
    if (!m3::supported_N(s->dstate) || !m3::supported_P(s->headdim) || s->rank > 4)
        return M3_ERR_UNSUPPORTED;
    // every grid dimension and element offset must stay in range
    const double bh = double(s->batch) * double(s->nheads);
    const double T = decode ? 1.0 : double(s->seqlen);
    const double elems = bh * T * double(s->rank) * double(s->dstate > s->headdim ? s->dstate : s->headdim);
    if (elems > 4.0e18) return M3_ERR_UNSUPPORTED;
    if (!decode) {
        // the prefill kernel stages a whole chunk in LDS
        const size_t lds = m3::prefill_lds_bytes(s->io_dtype == M3_DTYPE_BF16, s->dstate, s->headdim, s->rank);
        if (lds == 0 || lds > m3::kMaxLdsBytes) return M3_ERR_UNSUPPORTED;
    }
    if (bh * ((T + 63.0) / 64.0) > double(std::numeric_limits<unsigned>::max()) / 2) return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

// Workgroup slots the prefill aims to fill (MI355X has 256 compute units).
constexpr int64_t kSlots = 256;

// Segments per sequence: enough (batch, head, segment) workgroups to fill the
// chip, never an empty segment.  Depends on the shape only.
void segments(int64_t bh, int64_t T, int32_t &S, int32_t &cps) {
    const int64_t nC = (T + 63) / 64;
    int64_t s = bh >= kSlots ? 1 : kSlots / bh;
    if (s > nC) s = nC;
    if (s < 1) s = 1;
    const int64_t c = (nC + s - 1) / s;
    cps = int32_t(c);
    S = int32_t((nC + c - 1) / c);
}

WorkspaceLayout layout(const m3_shape_t *s) {
    const size_t bh = size_t(s->batch) * size_t(s->nheads);
    int32_t S, cps;
    segments(int64_t(bh), s->seqlen, S, cps);
    const size_t N = size_t(s->dstate), P = size_t(s->headdim), K = N / 2;
    WorkspaceLayout w;
    size_t off = 0;
    w.segU = off; off += round_up(bh * S * N * P * sizeof(float));
    w.segG = off; off += round_up(bh * S * sizeof(float));
    w.segTh = off; off += round_up(bh * S * K * sizeof(double));
    w.hinit = off; off += round_up(bh * N * P * sizeof(float));
    w.phi0 = off; off += round_up(bh * K * sizeof(double));
    w.total = off;
    return w;
}

// Backward workspace: the state and angle entering each chunk, the
// per-sequence partials of dA.
struct BwdLayout {
    size_t ck_h, ck_phi, gA, total;
};
BwdLayout bwd_layout(const m3_shape_t *s) {
    const size_t bh = size_t(s->batch) * size_t(s->nheads);
    const size_t Q = size_t(m3::kBwdV / s->rank);
    const size_t nC = (size_t(s->seqlen) + Q - 1) / Q;
    const size_t N = size_t(s->dstate), P = size_t(s->headdim), K = N / 2;
    BwdLayout w;
    size_t off = 0;
    w.ck_h = off; off += round_up(bh * nC * N * P * sizeof(float));
    w.ck_phi = off; off += round_up(bh * nC * K * sizeof(double));
    w.gA = off; off += round_up(bh * sizeof(float));
    w.total = off;
    return w;
}

m3_status_t check_backward_shape(const m3_shape_t *s) {
    const m3_status_t sc = check_shape(s, false);
    if (sc != M3_OK) return sc;
    if (s->ngroups != 0 && s->ngroups != s->nheads) return M3_ERR_UNSUPPORTED;
    if (s->state_dtype != M3_DTYPE_F32) return M3_ERR_UNSUPPORTED;
    if (double(s->batch) * double(s->nheads) > 2.0e9) return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

bool state_ok(const m3_state_t *st) {
    return st->h && st->phi && st->prev_B && st->prev_x && aligned16(st->h) && aligned16(st->phi) &&
           aligned16(st->prev_B) && aligned16(st->prev_x);
}

} // namespace

namespace m3 {

template <typename IO, int N, bool BLK>
static size_t lds_np(int P, int R) {
#define M3_LDS_R(PP)                                                                     \
    switch (R) {                                                                         \
    case 1: return Cfg<IO, N, PP, 1, BLK>::bytes;                                        \
    case 2: return Cfg<IO, N, PP, 2, BLK>::bytes;                                        \
    case 3: return Cfg<IO, N, PP, 3, BLK>::bytes;                                        \
    case 4: return Cfg<IO, N, PP, 4, BLK>::bytes;                                        \
    }                                                                                    \
    return 0;
    switch (P) {
    case 16: M3_LDS_R(16)
    case 32: M3_LDS_R(32)
    case 64: M3_LDS_R(64)
    }
#undef M3_LDS_R
    return 0;
}

template <bool BLK>
static size_t lds_n(bool is_bf16, int N, int P, int R) {
    switch (N) {
    case 16: return is_bf16 ? lds_np<bf16, 16, BLK>(P, R) : lds_np<float, 16, BLK>(P, R);
    case 32: return is_bf16 ? lds_np<bf16, 32, BLK>(P, R) : lds_np<float, 32, BLK>(P, R);
    case 64: return is_bf16 ? lds_np<bf16, 64, BLK>(P, R) : lds_np<float, 64, BLK>(P, R);
    case 128: return is_bf16 ? lds_np<bf16, 128, BLK>(P, R) : lds_np<float, 128, BLK>(P, R);
    }
    return 0;
}

size_t prefill_lds_bytes(bool is_bf16, int N, int P, int R, bool blk) {
    return blk ? lds_n<true>(is_bf16, N, P, R) : lds_n<false>(is_bf16, N, P, R);
}

} // namespace m3

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

// Validates the optional block prologue/epilogue and resolves it.
static m3_status_t resolve_block(const m3_block_t *blk, m3::BlockParams &b) {
    b = m3::BlockParams{};
    if (!blk) return M3_OK;
    const void *ptrs[] = {blk->B_weight, blk->B_bias, blk->C_weight, blk->C_bias, blk->z};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    if (blk->bc_norm && !(blk->norm_eps >= 0.f && blk->norm_eps <= 3.0e38f)) return M3_ERR_INVALID_ARGUMENT;
    b.norm = blk->bc_norm != 0;
    b.eps = blk->norm_eps;
    b.bw = blk->B_weight; b.bb = blk->B_bias; b.cw = blk->C_weight; b.cb = blk->C_bias;
    b.z = blk->z;
    b.on = b.norm || b.bw || b.bb || b.cw || b.cb || b.z;
    return M3_OK;
}

// Validates a prefill call and resolves its parameters.
static m3_status_t prepare_prefill(const m3_shape_t *shape, const void *x, const void *dt,
                                   const float *A, const void *lam, const void *theta,
                                   const void *B, const void *C, const m3_state_t *init,
                                   m3_state_t *final_state, void *y, void *workspace,
                                   size_t workspace_bytes, PrefillParams &p,
                                   const m3_block_t *block = nullptr) {
    const m3_status_t sc = check_shape(shape, false);
    if (sc != M3_OK) return sc;
    m3::BlockParams bp;
    const m3_status_t sb = resolve_block(block, bp);
    if (sb != M3_OK) return sb;
    if (bp.on) {
        // the block kernels also keep this head's weights and biases in LDS
        const size_t lds = m3::prefill_lds_bytes(shape->io_dtype == M3_DTYPE_BF16, shape->dstate,
                                                 shape->headdim, shape->rank, true);
        if (lds == 0 || lds > m3::kMaxLdsBytes) return M3_ERR_UNSUPPORTED;
    }
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
    p.G = shape->ngroups ? shape->ngroups : shape->nheads;
    p.hpg = p.H / p.G;
    p.sbf16 = shape->state_dtype == M3_DTYPE_BF16;
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
    segments(p.batch * p.H, p.T, p.S, p.cps);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.segU = reinterpret_cast<float *>(ws + w.segU);
    p.segG = reinterpret_cast<float *>(ws + w.segG);
    p.segTh = reinterpret_cast<double *>(ws + w.segTh);
    p.hinit = reinterpret_cast<float *>(ws + w.hinit);
    p.phi0ws = reinterpret_cast<double *>(ws + w.phi0);
    p.blk = bp;
    return M3_OK;
}

static hipError_t launch_stage(int32_t stage, const PrefillParams &p, bool bf, hipStream_t stream) {
    if (stage != M3_STAGE_SEGMENT_STATE && stage != M3_STAGE_OUTPUT) return hipErrorInvalidValue;
    const bool out = stage == M3_STAGE_OUTPUT;
    switch (p.N) {
    case 16: return bf ? m3::launch_prefill_bf16_n16(p, out, stream) : m3::launch_prefill_f32_n16(p, out, stream);
    case 32: return bf ? m3::launch_prefill_bf16_n32(p, out, stream) : m3::launch_prefill_f32_n32(p, out, stream);
    case 64: return bf ? m3::launch_prefill_bf16_n64(p, out, stream) : m3::launch_prefill_f32_n64(p, out, stream);
    case 128: return bf ? m3::launch_prefill_bf16_n128(p, out, stream) : m3::launch_prefill_f32_n128(p, out, stream);
    }
    return hipErrorInvalidValue;
}

m3_status_t m3_ssm_prefill(const m3_shape_t *shape, const void *x, const void *dt, const float *A,
                           const void *lam, const void *theta, const void *B, const void *C,
                           const m3_state_t *init, m3_state_t *final_state, void *y,
                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return m3_ssm_prefill_block(shape, x, dt, A, lam, theta, B, C, nullptr, init, final_state, y,
                                workspace, workspace_bytes, stream);
}

m3_status_t m3_ssm_prefill_block(const m3_shape_t *shape, const void *x, const void *dt,
                                 const float *A, const void *lam, const void *theta,
                                 const void *B, const void *C, const m3_block_t *block,
                                 const m3_state_t *init, m3_state_t *final_state, void *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    PrefillParams p;
    const m3_status_t sc = prepare_prefill(shape, x, dt, A, lam, theta, B, C, init, final_state, y,
                                           workspace, workspace_bytes, p, block);
    if (sc != M3_OK) return sc;
    const bool bf = shape->io_dtype == M3_DTYPE_BF16;
    for (int32_t stage = M3_STAGE_SEGMENT_STATE; stage <= M3_STAGE_OUTPUT; ++stage)
        if (launch_stage(stage, p, bf, stream) != hipSuccess) return M3_ERR_HIP;
    return M3_OK;
}

m3_status_t m3_ssm_prefill_stage(int32_t stage, const m3_shape_t *shape, const void *x,
                                 const void *dt, const float *A, const void *lam,
                                 const void *theta, const void *B, const void *C,
                                 const m3_state_t *init, m3_state_t *final_state, void *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (stage != M3_STAGE_SEGMENT_STATE && stage != M3_STAGE_OUTPUT) return M3_ERR_INVALID_ARGUMENT;
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
    return m3_ssm_decode_step_block(shape, x, dt, A, lam, theta, B, C, nullptr, state, y, stream);
}

m3_status_t m3_ssm_decode_step_block(const m3_shape_t *shape, const void *x, const void *dt,
                                     const float *A, const void *lam, const void *theta,
                                     const void *B, const void *C, const m3_block_t *block,
                                     m3_state_t *state, void *y, hipStream_t stream) {
    const m3_status_t sc = check_shape(shape, true);
    if (sc != M3_OK) return sc;
    m3::BlockParams bp;
    const m3_status_t sb = resolve_block(block, bp);
    if (sb != M3_OK) return sb;
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
    p.G = shape->ngroups ? shape->ngroups : shape->nheads;
    p.hpg = p.H / p.G;
    p.sbf16 = shape->state_dtype == M3_DTYPE_BF16;
    p.x = x; p.dt = dt; p.lam = lam; p.theta = theta; p.B = B; p.C = C; p.A = A; p.y = y;
    p.h = state->h; p.phi = state->phi; p.prevB = state->prev_B; p.prevx = state->prev_x;
    p.blk = bp;
    if ((shape->io_dtype == M3_DTYPE_BF16 ? m3::launch_decode_bf16(p, stream) : m3::launch_decode_f32(p, stream)) != hipSuccess)
        return M3_ERR_HIP;
    return M3_OK;
}

size_t m3_ssm_prefill_backward_workspace_bytes(const m3_shape_t *shape) {
    if (check_backward_shape(shape) != M3_OK) return 0;
    return bwd_layout(shape).total;
}

m3_status_t m3_ssm_prefill_backward(const m3_shape_t *shape, const void *x, const void *dt,
                                    const float *A, const void *lam, const void *theta,
                                    const void *B, const void *C, const m3_state_t *init,
                                    const void *gy, const m3_grads_t *grads, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    const m3_status_t sc = check_backward_shape(shape);
    if (sc != M3_OK) return sc;
    const void *ptrs[] = {x, dt, A, lam, theta, B, C, gy};
    for (const void *q : ptrs)
        if (!q || !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    if (!grads) return M3_ERR_INVALID_ARGUMENT;
    const void *outs[] = {grads->x, grads->dt, grads->A, grads->lam, grads->theta, grads->B, grads->C};
    for (const void *q : outs)
        if (!q || !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    const void *opt[] = {grads->h, grads->phi, grads->prev_B, grads->prev_x};
    for (const void *q : opt)
        if (q && !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    if (init && !state_ok(init)) return M3_ERR_INVALID_ARGUMENT;
    const BwdLayout w = bwd_layout(shape);
    if (!workspace || !aligned16(workspace) || workspace_bytes < w.total) return M3_ERR_WORKSPACE;
    m3::BwdParams p{};
    p.batch = shape->batch;
    p.T = shape->seqlen;
    p.H = shape->nheads;
    p.P = shape->headdim;
    p.N = shape->dstate;
    p.R = shape->rank;
    p.K = p.N / 2;
    p.nC = int32_t((p.T + m3::kBwdV / p.R - 1) / (m3::kBwdV / p.R));
    p.x = x; p.dt = dt; p.lam = lam; p.theta = theta; p.B = B; p.C = C; p.gy = gy; p.A = A;
    p.has_init = init != nullptr;
    if (init) {
        p.h0 = static_cast<const float *>(init->h); p.phi0 = init->phi; p.prevB0 = init->prev_B;
        p.prevx0 = init->prev_x;
        p.gh0 = grads->h; p.gphi0 = grads->phi; p.gprevB0 = grads->prev_B; p.gprevx0 = grads->prev_x;
    }
    p.gx = grads->x; p.gdt = grads->dt; p.glam = grads->lam; p.gtheta = grads->theta;
    p.gB = grads->B; p.gC = grads->C; p.gA = grads->A;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.ck_h = reinterpret_cast<float *>(ws + w.ck_h);
    p.ck_phi = reinterpret_cast<double *>(ws + w.ck_phi);
    p.gA_part = reinterpret_cast<float *>(ws + w.gA);
    const hipError_t e = shape->io_dtype == M3_DTYPE_BF16 ? m3::launch_backward_bf16(p, stream)
                                                          : m3::launch_backward_f32(p, stream);
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

} // extern "C"
