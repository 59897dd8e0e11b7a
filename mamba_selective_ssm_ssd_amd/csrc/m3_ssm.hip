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

#include <algorithm>
#include <limits>

namespace {

using m3::PrefillParams;
using m3::WorkspaceLayout;

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tokens per chunk the prefill kernels use for a shape (0: no compiled
// kernel), for the segment pre-pass (out = false) or the output pass.
// chunk = small_chunk(R) takes chunks of that many tokens in both passes.
// chunk = 64 takes 64-token chunks when their tiles fit in the LDS of a CU,
// else small ones; where both fit, the output pass of bf16 MIMO shapes
// takes the small chunk, which measured faster (a quarter of the quadratic
// intra-chunk work per token), and the pre-pass the 64-token chunk (it has
// no intra-chunk product, only per-chunk overheads).  small_chunk(R)
// divides 64, so segments of whole 64-token chunks are whole small chunks
// too, and every choice gives the same result up to rounding.
int chunk_tokens(const m3_shape_t *s, bool blk, bool out) {
    const bool bf = s->io_dtype == M3_DTYPE_BF16;
    const int qs = m3::small_chunk(s->rank);
    auto fits = [&](int q) {
        const size_t lds = m3::prefill_lds_bytes(bf, s->dstate, s->headdim, s->rank, blk, q);
        return lds > 0 && lds <= m3::kMaxLdsBytes;
    };
    if (s->chunk == qs) return fits(qs) ? qs : 0;
    if (s->chunk != 64) return 0;
    if (!fits(64)) return fits(qs) ? qs : 0;
    if (out && bf && s->rank == 4 && fits(qs)) return qs;
    return 64;
}

// Which entry point a shape is checked for.
enum class Use { prefill, decode, backward };

// Checks the shape.  Returns M3_OK or the error to report.  Only the
// prefill's kernels stage chunks in LDS; the backward's LDS layout fits for
// every (N, P, R) of the tile set by construction (checked at compile time).
m3_status_t check_shape(const m3_shape_t *s, Use use) {
    const bool decode = use == Use::decode;
    if (!s) return M3_ERR_INVALID_ARGUMENT;
    if (s->io_dtype != M3_DTYPE_F32 && s->io_dtype != M3_DTYPE_BF16) return M3_ERR_INVALID_ARGUMENT;
    if (s->batch < 1 || s->nheads < 1 || s->headdim < 1 || s->dstate < 2 || s->rank < 1)
        return M3_ERR_INVALID_ARGUMENT;
    if (!decode && s->seqlen < 1) return M3_ERR_INVALID_ARGUMENT;
    if (s->dstate % 2 != 0) return M3_ERR_INVALID_ARGUMENT;
    if (s->chunk < 1) return M3_ERR_INVALID_ARGUMENT;
    if (s->ngroups < 0 || (s->ngroups > 0 && s->nheads % s->ngroups != 0)) return M3_ERR_INVALID_ARGUMENT;
    if (s->state_dtype != M3_DTYPE_F32 && s->state_dtype != M3_DTYPE_BF16) return M3_ERR_INVALID_ARGUMENT;
    if (!m3::supported_N(s->dstate) || !m3::supported_P(s->headdim) || s->rank > 4)
        return M3_ERR_UNSUPPORTED;
    if (s->chunk != 64 && s->chunk != m3::small_chunk(s->rank)) return M3_ERR_UNSUPPORTED;
    // every grid dimension and element offset must stay in range: offsets
    // across tokens and sequences are 64-bit, the kernels' offsets within a
    // chunk (up to 64 tokens of the x, y, B, C, theta rows) 32-bit
    const double bh = double(s->batch) * double(s->nheads);
    const double T = decode ? 1.0 : double(s->seqlen);
    const double wide = double(s->dstate > s->headdim ? s->dstate : s->headdim);
    const double elems = bh * T * double(s->rank) * wide;
    if (elems > 4.0e18) return M3_ERR_UNSUPPORTED;
    if (64.0 * double(s->nheads) * double(s->rank) * wide >= 2147483648.0) return M3_ERR_UNSUPPORTED;
    // the prefill kernel stages a whole chunk in LDS
    if (use == Use::prefill && (chunk_tokens(s, false, false) == 0 || chunk_tokens(s, false, true) == 0))
        return M3_ERR_UNSUPPORTED;
    if (bh * ((T + 15.0) / 16.0) > double(std::numeric_limits<unsigned>::max()) / 2) return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

// Workgroup slots the prefill aims to fill (MI355X has 256 compute units).
constexpr int64_t kSlots = 256;

// Segments per sequence: enough (batch, head, segment) workgroups to fill the
// chip, never an empty segment.  Depends on the shape and the chunk length Q
// only.
void segments(int64_t bh, int64_t T, int Q, int32_t &S, int32_t &cps) {
    const int64_t nC = (T + Q - 1) / Q;
    int64_t s = bh >= kSlots ? 1 : kSlots / bh;
    if (s > nC) s = nC;
    if (s < 1) s = 1;
    const int64_t c = (nC + s - 1) / s;
    cps = int32_t(c);
    S = int32_t((nC + c - 1) / c);
}

// How one prefill call runs: chunk lengths of the two passes, S segments of
// seglen tokens per sequence (whole pre-pass chunks), and the pre-pass cut
// into kpre pieces per segment.  With S > 1 the pre-pass has (S - 1) b H
// workgroups; when that is not a whole number of rounds over the 256
// compute units, cutting each segment into kpre pieces (a power of two up to
// 8, at least two chunks each) that make it one fills every round, at
// NA = (S - 1) kpre aggregates per sequence (kept below 16 MiB in all).
struct Plan {
    int32_t Qpre, Qout, S, cps, kpre, NA;
    int64_t seglen;
};
Plan make_plan(const m3_shape_t *s, bool blk) {
    Plan pl{};
    pl.Qpre = chunk_tokens(s, blk, false);
    pl.Qout = chunk_tokens(s, blk, true);
    if (pl.Qpre == 0 || pl.Qout == 0) return pl;
    const int64_t bh = s->batch * s->nheads;
    segments(bh, s->seqlen, pl.Qpre, pl.S, pl.cps);
    pl.seglen = int64_t(pl.cps) * pl.Qpre;
    pl.kpre = 1;
    if (pl.S > 1) {
        const int64_t w = int64_t(pl.S - 1) * bh;
        const double agg = double(s->dstate) * double(s->headdim) * 4.0;
        if (w % kSlots != 0) {
            for (int k = 2; k <= 8; k *= 2) {
                if ((w * k) % kSlots == 0 && pl.cps % k == 0 && pl.cps / k >= 2 &&
                    double(w * k) * agg <= double(16 << 20)) {
                    pl.kpre = k;
                    break;
                }
            }
        }
    }
    pl.NA = (pl.S - 1) * pl.kpre;
    return pl;
}

// Sized for the plain and the block kernels' plans (their chunk lengths may
// differ), so one workspace serves both.  Only a sequence cut into S > 1
// segments uses it; otherwise it is one aligned block, unused.
WorkspaceLayout layout(const m3_shape_t *s) {
    const size_t bh = size_t(s->batch) * size_t(s->nheads);
    const Plan a = make_plan(s, false), b = make_plan(s, true);
    const size_t NA = size_t(a.NA > b.NA ? a.NA : b.NA);
    const size_t N = size_t(s->dstate), P = size_t(s->headdim), K = N / 2;
    const size_t used = NA > 0 ? 1 : 0;
    WorkspaceLayout w;
    size_t off = 0;
    w.segU = off; off += round_up(bh * NA * N * P * sizeof(float));
    w.segG = off; off += round_up(bh * NA * sizeof(float));
    w.segTh = off; off += round_up(bh * NA * K * sizeof(double));
    w.hinit = off; off += round_up(used * bh * N * P * sizeof(float));
    w.phi0 = off; off += round_up(used * bh * K * sizeof(double));
    w.total = off > kAlign ? off : kAlign;
    return w;
}

// Backward segments: with fewer than 256 (batch, head) sequences each is cut
// into S segments of whole chunks (at least two chunks each, at most 64
// segments), one workgroup per (b, h, segment), so that the grid fills the
// 256 CUs; S = 1 otherwise.
struct BwdPlan {
    int32_t S, cps, kagg; // kagg: pieces per segment of the aggregate launch
};
BwdPlan bwd_plan(const m3_shape_t *s) {
    const int64_t bh = int64_t(s->batch) * s->nheads;
    const int64_t Q = m3::kBwdV / s->rank;
    const int64_t nC = (int64_t(s->seqlen) + Q - 1) / Q;
    int64_t S = 1;
    if (bh < 256) S = std::min<int64_t>({(256 + bh - 1) / bh, nC / 2, 64});
    if (S < 2) return {1, int32_t(nC), 1};
    const int64_t cps = (nC + S - 1) / S;
    S = (nC + cps - 1) / cps;
    // the aggregate launch has 2 (S - 1) b H jobs of a segment each; cut them
    // into pieces so that the launch fills whole rounds of the 256 CUs
    int32_t kagg = 1;
    for (int32_t k = 1; k <= 8; k *= 2)
        if ((2 * (S - 1) * bh * k) % 256 == 0 && cps % k == 0) {
            kagg = k;
            break;
        }
    return {int32_t(S), int32_t(cps), kagg};
}

// Backward workspace: the state and angle entering each chunk, the
// per-(sequence, segment) partials of dA and, for split sequences, the
// segment aggregates.
struct BwdLayout {
    size_t ck_h, ck_phi, gA, segA, segGa, segg, segdd, segTh, segDphi, total;
};
BwdLayout bwd_layout(const m3_shape_t *s) {
    const size_t bh = size_t(s->batch) * size_t(s->nheads);
    const size_t Q = size_t(m3::kBwdV / s->rank);
    const size_t nC = (size_t(s->seqlen) + Q - 1) / Q;
    const size_t N = size_t(s->dstate), P = size_t(s->headdim), K = N / 2;
    const BwdPlan plan = bwd_plan(s);
    const size_t S = size_t(plan.S), nseg = S > 1 ? bh * S : 0, npc = nseg * size_t(plan.kagg);
    BwdLayout w;
    size_t off = 0;
    w.ck_h = off; off += round_up(bh * nC * N * P * sizeof(float));
    w.ck_phi = off; off += round_up(bh * nC * K * sizeof(double));
    w.gA = off; off += round_up(bh * S * sizeof(float));
    w.segA = off; off += round_up(npc * N * P * sizeof(float));
    w.segGa = off; off += round_up(npc * N * P * sizeof(float));
    w.segg = off; off += round_up(npc * sizeof(float));
    w.segdd = off; off += round_up(nseg * sizeof(float));
    w.segTh = off; off += round_up(npc * K * sizeof(double));
    w.segDphi = off; off += round_up(nseg * K * sizeof(double));
    w.total = off;
    return w;
}

m3_status_t check_backward_shape(const m3_shape_t *s) {
    const m3_status_t sc = check_shape(s, Use::backward);
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

template <typename IO, int N, int P, int R, bool BLK>
static size_t lds_q(int Q) {
    constexpr int QS = small_chunk(R);
    if (Q == 64) return Cfg<IO, N, P, R, 64, BLK>::bytes;
    if (Q == QS) return Cfg<IO, N, P, R, QS, BLK>::bytes;
    return 0;
}

template <typename IO, int N, bool BLK>
static size_t lds_np(int P, int R, int Q) {
#define M3_LDS_R(PP)                                                                     \
    switch (R) {                                                                         \
    case 1: return lds_q<IO, N, PP, 1, BLK>(Q);                                          \
    case 2: return lds_q<IO, N, PP, 2, BLK>(Q);                                          \
    case 3: return lds_q<IO, N, PP, 3, BLK>(Q);                                          \
    case 4: return lds_q<IO, N, PP, 4, BLK>(Q);                                          \
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
static size_t lds_n(bool is_bf16, int N, int P, int R, int Q) {
    switch (N) {
    case 16: return is_bf16 ? lds_np<bf16, 16, BLK>(P, R, Q) : lds_np<float, 16, BLK>(P, R, Q);
    case 32: return is_bf16 ? lds_np<bf16, 32, BLK>(P, R, Q) : lds_np<float, 32, BLK>(P, R, Q);
    case 64: return is_bf16 ? lds_np<bf16, 64, BLK>(P, R, Q) : lds_np<float, 64, BLK>(P, R, Q);
    case 128: return is_bf16 ? lds_np<bf16, 128, BLK>(P, R, Q) : lds_np<float, 128, BLK>(P, R, Q);
    }
    return 0;
}

size_t prefill_lds_bytes(bool is_bf16, int N, int P, int R, bool blk, int Q) {
    return blk ? lds_n<true>(is_bf16, N, P, R, Q) : lds_n<false>(is_bf16, N, P, R, Q);
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
    if (check_shape(shape, Use::prefill) != M3_OK) return 0;
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
    const m3_status_t sc = check_shape(shape, Use::prefill);
    if (sc != M3_OK) return sc;
    m3::BlockParams bp;
    const m3_status_t sb = resolve_block(block, bp);
    if (sb != M3_OK) return sb;
    // the block kernels also keep this head's weights and biases in LDS
    const Plan pl = make_plan(shape, bp.on);
    if (pl.Qpre == 0 || pl.Qout == 0) return M3_ERR_UNSUPPORTED;
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
    p.Qpre = pl.Qpre;
    p.Qout = pl.Qout;
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
    // segments of whole pre-pass chunks (which are whole output-pass chunks)
    p.S = pl.S;
    p.seglen = pl.seglen;
    p.kpre = pl.kpre;
    p.NA = pl.NA;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.segU = reinterpret_cast<float *>(ws + w.segU);
    p.segG = reinterpret_cast<float *>(ws + w.segG);
    p.segTh = reinterpret_cast<double *>(ws + w.segTh);
    p.hinit = reinterpret_cast<float *>(ws + w.hinit);
    p.phi0ws = reinterpret_cast<double *>(ws + w.phi0);
    p.blk = bp;
    return M3_OK;
}

// The launcher of one (I/O type, N, block variant, chunk kind).
#define M3_LAUNCHERS(IO, N)                                                                        \
    { m3::launch_prefill_##IO##_n##N, m3::launch_prefill_##IO##_n##N##_blk,                        \
      m3::launch_prefill_##IO##_n##N##_qs, m3::launch_prefill_##IO##_n##N##_blk_qs }
static const m3::prefill_launcher_t kLaunchers[2][4][4] = {
    {M3_LAUNCHERS(f32, 16), M3_LAUNCHERS(f32, 32), M3_LAUNCHERS(f32, 64), M3_LAUNCHERS(f32, 128)},
    {M3_LAUNCHERS(bf16, 16), M3_LAUNCHERS(bf16, 32), M3_LAUNCHERS(bf16, 64), M3_LAUNCHERS(bf16, 128)}};
#undef M3_LAUNCHERS

static hipError_t launch_stage(int32_t stage, const PrefillParams &p0, bool bf, hipStream_t stream) {
    if (stage != M3_STAGE_SEGMENT_STATE && stage != M3_STAGE_OUTPUT) return hipErrorInvalidValue;
    const bool out = stage == M3_STAGE_OUTPUT;
    const int ni = p0.N == 16 ? 0 : p0.N == 32 ? 1 : p0.N == 64 ? 2 : p0.N == 128 ? 3 : -1;
    if (ni < 0) return hipErrorInvalidValue;
    // this stage's chunk length, chunk count and chunks per segment
    PrefillParams p = p0;
    p.Q = out ? p.Qout : p.Qpre;
    p.nC = int32_t((p.T + p.Q - 1) / p.Q);
    p.cps = int32_t(p.seglen / p.Q / (out ? 1 : p.kpre));
    const int kind = (p.blk.on ? 1 : 0) + (p.Q != 64 ? 2 : 0);
    return kLaunchers[bf ? 1 : 0][ni][kind](p, out, stream);
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

m3_status_t m3_ssm_prefill_plan(const m3_shape_t *shape, int32_t with_block, int32_t *chunk_pre,
                                int32_t *chunk_out, int32_t *segments_out, int64_t *segment_tokens,
                                int32_t *prepass_pieces) {
    const m3_status_t sc = check_shape(shape, Use::prefill);
    if (sc != M3_OK) return sc;
    const Plan pl = make_plan(shape, with_block != 0);
    if (pl.Qpre == 0 || pl.Qout == 0) return M3_ERR_UNSUPPORTED;
    if (chunk_pre) *chunk_pre = pl.Qpre;
    if (chunk_out) *chunk_out = pl.Qout;
    if (segments_out) *segments_out = pl.S;
    if (segment_tokens) *segment_tokens = pl.seglen;
    if (prepass_pieces) *prepass_pieces = pl.kpre;
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
    const m3_status_t sc = check_shape(shape, Use::decode);
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

m3_status_t m3_ssm_prefill_backward_plan(const m3_shape_t *shape, int32_t *segments, int64_t *segment_tokens) {
    const m3_status_t sc = check_backward_shape(shape);
    if (sc != M3_OK) return sc;
    const BwdPlan plan = bwd_plan(shape);
    if (segments) *segments = plan.S;
    if (segment_tokens) *segment_tokens = int64_t(plan.cps) * (m3::kBwdV / shape->rank);
    return M3_OK;
}

m3_status_t m3_ssm_prefill_backward(const m3_shape_t *shape, const void *x, const void *dt,
                                    const float *A, const void *lam, const void *theta,
                                    const void *B, const void *C, const m3_state_t *init,
                                    const void *gy, const m3_grads_t *grads, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    return m3_ssm_prefill_backward_ex(shape, x, dt, A, lam, theta, B, C, init, gy, nullptr, grads,
                                      workspace, workspace_bytes, stream);
}

m3_status_t m3_ssm_prefill_backward_ex(const m3_shape_t *shape, const void *x, const void *dt,
                                       const float *A, const void *lam, const void *theta,
                                       const void *B, const void *C, const m3_state_t *init,
                                       const void *gy, const m3_final_grads_t *gfinal,
                                       const m3_grads_t *grads, void *workspace,
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
    if (gfinal) {
        const void *gf[] = {gfinal->h, gfinal->phi, gfinal->prev_B, gfinal->prev_x};
        for (const void *q : gf)
            if (q && !aligned16(q)) return M3_ERR_INVALID_ARGUMENT;
    }
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
    if (gfinal) {
        p.ghT = gfinal->h; p.gphiT = gfinal->phi; p.gBpT = gfinal->prev_B; p.gxpT = gfinal->prev_x;
    }
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.ck_h = reinterpret_cast<float *>(ws + w.ck_h);
    p.ck_phi = reinterpret_cast<double *>(ws + w.ck_phi);
    p.gA_part = reinterpret_cast<float *>(ws + w.gA);
    const BwdPlan plan = bwd_plan(shape);
    p.S = plan.S;
    p.cps = plan.cps;
    p.kagg = plan.kagg;
    p.segA = reinterpret_cast<float *>(ws + w.segA);
    p.segGa = reinterpret_cast<float *>(ws + w.segGa);
    p.segg = reinterpret_cast<float *>(ws + w.segg);
    p.segdd = reinterpret_cast<float *>(ws + w.segdd);
    p.segTh = reinterpret_cast<double *>(ws + w.segTh);
    p.segDphi = reinterpret_cast<double *>(ws + w.segDphi);
    const hipError_t e = shape->io_dtype == M3_DTYPE_BF16 ? m3::launch_backward_bf16(p, stream)
                                                          : m3::launch_backward_f32(p, stream);
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

} // extern "C"
