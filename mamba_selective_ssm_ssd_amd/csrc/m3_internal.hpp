// m3_internal.hpp -- parameters passed from the host dispatch to the kernels,
// and the kernel launchers each translation unit provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

// Block prologue and epilogue around the mixer (Mamba-3 review, section 3.4):
// B and C rows RMS-normalised over N, then weight and bias per (head, rank,
// channel); y gated by silu(z).  Absent pieces are null / zero.
struct BlockParams {
    int32_t on;                     // any piece present: the block kernels run
    int32_t norm;                   // RMS-normalise the B and C rows
    float eps;                      // inside the square root
    const float *bw, *bb, *cw, *cb; // [H][R][N] fp32: B weight, B bias, C weight, C bias
    const void *z;                  // gate, shaped like y (I/O dtype)
};

// Everything one prefill call needs, resolved to device pointers.
struct PrefillParams {
    int64_t batch, T;
    int32_t H, P, N, R, K;     // K = N/2 rotation pairs
    int32_t Q, nC;             // tokens per chunk of the launched pass (64 or small_chunk(R)), ceil(T/Q) chunks
    int32_t G, hpg;            // B/C groups, heads per group (head h reads group h / hpg)
    int32_t sbf16;             // carried state h~ stored in bf16
    int32_t S, cps;            // segments per sequence, chunks of the launched pass per segment (piece)
    int32_t kpre, NA;          // pre-pass pieces per segment, aggregates per sequence ((S - 1) kpre)
    int32_t Qpre, Qout;        // tokens per chunk of the pre-pass and of the output pass (host)
    int64_t seglen;            // tokens per segment, a multiple of both (host)
    // inputs (I/O dtype unless noted)
    const void *x, *dt, *lam, *theta, *B, *C;
    const float *A; // [H]
    void *y;
    // initial carried state; read only by the first workgroup of a sequence
    // (S == 1) or by the pre-pass (S > 1)
    int32_t has_init;
    const void *h0; // state_dtype (sbf16: bf16, else fp32)
    const float *phi0, *prevB0;
    const void *prevx0;
    // final carried state; written only by the last segment's workgroup
    int32_t has_final;
    void *hT; // state_dtype
    float *phiT, *prevBT;
    void *prevxT;
    // workspace (used when S > 1)
    float *segU;    // [b][H][NA][N][P] aggregate of each pre-pass piece: its state from a zero start
    float *segG;    // [b][H][NA]       summed log decay of the piece
    double *segTh;  // [b][H][NA][K]    summed rotary angle of the piece
    float *hinit;   // [b][H][N][P]     carried state in its own frame at the sequence start
    double *phi0ws; // [b][H][K]        Phi_{-1}
    BlockParams blk;
};

struct DecodeParams {
    int64_t batch;
    int32_t H, P, N, R, K;
    int32_t G, hpg; // B/C groups, heads per group
    int32_t sbf16;  // state h~ stored in bf16
    const void *x, *dt, *lam, *theta, *B, *C;
    const float *A;
    void *y;
    void *h; // state_dtype
    float *phi, *prevB;
    void *prevx;
    BlockParams blk;
};

// Backward pass (one workgroup per (batch, head), chunks of kBwdV / R
// tokens processed last to first): kBwdV rows (token, rank) per chunk.
constexpr int kBwdV = 32;

struct BwdParams {
    int64_t batch, T;
    int32_t H, P, N, R, K, nC;
    const void *x, *dt, *lam, *theta, *B, *C, *gy; // I/O dtype
    const float *A;
    int32_t has_init;
    const float *h0, *phi0, *prevB0; // rotated frame, fp32
    const void *prevx0;             // I/O dtype
    // incoming gradients of the final carried state (fp32, rotated frame;
    // null: zero): h~_T [N][P], Phi_T [K], B~_{T-1} [R][N], x_{T-1} [R][P] per (b, h)
    const float *ghT, *gphiT, *gBpT, *gxpT;
    // outputs (fp32); the carried-state ones may be null
    float *gx, *gdt, *glam, *gtheta, *gB, *gC, *gA;
    float *gh0, *gphi0, *gprevB0, *gprevx0;
    // workspace
    float *ck_h;    // [b][H][nC][N x P] state entering each chunk (tile-major)
    double *ck_phi; // [b][H][nC][K]     angle before each chunk
    float *gA_part; // [b][H][S]
    // sequences split into S segments of cps chunks (S = 1: no split).
    // mode 0: the gradients of each (b, h, segment); mode 1: the segment
    // aggregates, (S - 1) b H workgroups of forward state (segments 0 .. S-2)
    // then as many of adjoint state (segments 1 .. S-1).
    // The aggregates are taken per piece: kagg pieces of cps / kagg chunks per
    // segment, S kagg pieces per sequence.
    int32_t S, cps, mode, kagg;
    float *segA;     // [b][H][S kagg][N][P] state at a piece's end from zero, frame of its start
    float *segGa;    // [b][H][S kagg][N][P] adjoint at a piece's start from zero at its end, same frame
    float *segg;     // [b][H][S kagg] summed log decay of a piece
    float *segdd;    // [b][H][S] gradient of delta of a segment's first token from the segment before
    double *segTh;   // [b][H][S kagg][K] summed theta of a piece (wrapped)
    double *segDphi; // [b][H][S][K] summed dPhi of a segment
};

// Workspace layout (byte offsets of each region, 256-byte aligned).
struct WorkspaceLayout {
    size_t segU, segG, segTh, hinit, phi0, total;
};

// Tokens per chunk of the small MIMO chunk: 64/R tokens, i.e. 64 virtual
// (token, rank) rows (R = 3: 32 tokens, 96 rows, since the products take
// rows 32 at a time); 64 for R = 1.
constexpr int small_chunk(int R) { return R == 4 ? 16 : R >= 2 ? 32 : 64; }

// Fused prefill launchers, one per (I/O type, N, block variant, chunk kind):
// out = false runs the segment pre-pass (nothing to do when S == 1), out =
// true the output pass.  "_blk": the block prologue/epilogue kernels
// (p.blk.on); "_qs": chunks of small_chunk(R) tokens instead of 64.
typedef hipError_t (*prefill_launcher_t)(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n16(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n16_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n16_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n16_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n32(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n32_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n32_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n32_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n64(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n64_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n64_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n64_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n128(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n128_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n128_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_bf16_n128_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n16(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n16_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n16_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n16_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n32(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n32_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n32_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n32_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n64(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n64_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n64_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n64_blk_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n128(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n128_blk(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n128_qs(const PrefillParams &p, bool out, hipStream_t s);
hipError_t launch_prefill_f32_n128_blk_qs(const PrefillParams &p, bool out, hipStream_t s);

hipError_t launch_decode_bf16(const DecodeParams &p, hipStream_t s);
hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t s);
// the same with the block prologue/epilogue (p.blk.on)
hipError_t launch_decode_bf16_blk(const DecodeParams &p, hipStream_t s);
hipError_t launch_decode_f32_blk(const DecodeParams &p, hipStream_t s);
// the same with a bf16 carried state (p.sbf16), plain and with the block ops
hipError_t launch_decode_bf16_sb(const DecodeParams &p, hipStream_t s);
hipError_t launch_decode_f32_sb(const DecodeParams &p, hipStream_t s);
hipError_t launch_decode_bf16_blk_sb(const DecodeParams &p, hipStream_t s);
hipError_t launch_decode_f32_blk_sb(const DecodeParams &p, hipStream_t s);

hipError_t launch_backward_bf16(const BwdParams &p, hipStream_t s);
hipError_t launch_backward_f32(const BwdParams &p, hipStream_t s);

// Dynamic LDS bytes of the fused prefill kernel for a shape and chunk length
// Q (64 or small_chunk(R)); 0: not compiled.
size_t prefill_lds_bytes(bool is_bf16, int N, int P, int R, bool blk, int Q);
constexpr size_t kMaxLdsBytes = 160 * 1024; // LDS per workgroup on gfx950

// Sizes handled by the compiled kernels.
inline bool supported_P(int P) { return P == 16 || P == 32 || P == 64; }
inline bool supported_N(int N) { return N == 16 || N == 32 || N == 64 || N == 128; }

} // namespace m3

// Expand MACRO(IO, N, P) for every compiled (N, P) pair and both I/O types,
// as a switch that returns from the enclosing launcher.
#define M3_DISPATCH(IS_BF16, NV, PV, MACRO)                                          \
    do {                                                                             \
        if (IS_BF16) {                                                               \
            M3_DISPATCH_NP(::m3::bf16, NV, PV, MACRO);                               \
        } else {                                                                     \
            M3_DISPATCH_NP(float, NV, PV, MACRO);                                    \
        }                                                                            \
        return hipErrorInvalidValue;                                                 \
    } while (0)

#define M3_DISPATCH_P(IO, NC, PV, MACRO)                                             \
    switch (PV) {                                                                    \
    case 16: MACRO(IO, NC, 16);                                                      \
    case 32: MACRO(IO, NC, 32);                                                      \
    case 64: MACRO(IO, NC, 64);                                                      \
    default: break;                                                                  \
    }

#define M3_DISPATCH_NP(IO, NV, PV, MACRO)                                            \
    switch (NV) {                                                                    \
    case 16: M3_DISPATCH_P(IO, 16, PV, MACRO); break;                                \
    case 32: M3_DISPATCH_P(IO, 32, PV, MACRO); break;                                \
    case 64: M3_DISPATCH_P(IO, 64, PV, MACRO); break;                                \
    case 128: M3_DISPATCH_P(IO, 128, PV, MACRO); break;                              \
    default: break;                                                                  \
    }
