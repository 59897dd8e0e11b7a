// m3_internal.hpp -- parameters passed from the host dispatch to the kernels,
// and the kernel launchers each translation unit provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

// Everything one prefill call needs, resolved to device pointers.
struct PrefillParams {
    int64_t batch, T;
    int32_t H, P, N, R, K, nC; // K = N/2 rotation pairs, nC = ceil(T/64) chunks
    // inputs (I/O dtype unless noted)
    const void *x, *dt, *lam, *theta, *B, *C;
    const float *A; // [H]
    void *y;
    // initial carried state (read by the coefficient kernel only)
    int32_t has_init;
    const float *h0, *phi0, *prevB0;
    const void *prevx0;
    // final carried state (written by the state-scan kernel only)
    int32_t has_final;
    float *hT, *phiT, *prevBT;
    void *prevxT;
    // workspace
    float *ell;        // [b][H][T]   within-chunk inclusive cumsum of dt*A
    float *gam;        // [b][H][T]   gamma_t = lam_t dt_t
    float *wgt;        // [b][H][T]   gamma_t + delta_{t+1} (delta_T = 0)
    float *ubuf;       // [b][H][nC][N][P]  chunk state, then incoming state
    double *thetaC;    // [b][H][nC][K]     chunk angle totals
    float2 *thetaCS;   // [b][H][nC][K]     (cos, sin) of the wrapped totals
    float *hinit;      // [b][H][N][P]      incoming state of chunk 0
    double *phi0ws;    // [b][H][K]         Phi_{-1}
};

struct DecodeParams {
    int64_t batch;
    int32_t H, P, N, R, K;
    const void *x, *dt, *lam, *theta, *B, *C;
    const float *A;
    void *y;
    float *h, *phi, *prevB;
    void *prevx;
};

// Workspace layout (byte offsets of each region, 256-byte aligned).
struct WorkspaceLayout {
    size_t ell, gam, wgt, ubuf, thetaC, thetaCS, hinit, phi0, total;
};

// Launchers: dispatch on (io dtype, N, P) and enqueue one kernel.
// Return hipSuccess, or the launch error.  is_bf16 selects the I/O type.
hipError_t launch_chunk_coef(const PrefillParams &p, bool is_bf16, hipStream_t s);
hipError_t launch_chunk_state(const PrefillParams &p, bool is_bf16, hipStream_t s);
hipError_t launch_state_scan(const PrefillParams &p, bool is_bf16, hipStream_t s);
hipError_t launch_chunk_output(const PrefillParams &p, bool is_bf16, hipStream_t s);
hipError_t launch_decode_step(const DecodeParams &p, bool is_bf16, hipStream_t s);

// Dynamic LDS bytes of the chunk kernels for a shape (0 if not compiled).
size_t chunk_state_lds_bytes(bool is_bf16, int N, int P, int R);
size_t chunk_output_lds_bytes(bool is_bf16, int N, int P, int R);
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
