// m3_chunk.hpp -- per-chunk prologue shared by the chunk-state and the
// chunk-output kernels: which (b, h, c) a workgroup owns, the chunk's decay
// coefficients, and the within-chunk cumulative rotary angles.
//
// Within chunk c (tokens t0 .. t0+Tc-1) every B and C is rotated by the local
// cumulative angle phi_loc[s][k] = sum_{t0 <= u <= s} theta_u,k (the RoPE form
// of the complex state, Mamba-3 review section 3.2, Props. 3.2.2-3.2.3, taken
// relative to the chunk start).  The rotation by the angle accumulated before
// the chunk is carried by the inter-chunk state kernel, so no global angle ever
// reaches fp32.
#pragma once

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

struct ChunkId {
    int64_t b, bh; // batch index, b * H + h
    int32_t h, c;  // head, chunk
    int64_t t0;    // first token
    int32_t Tc;    // valid tokens in this chunk (64 except a ragged tail)
};

__device__ __forceinline__ ChunkId chunk_id(const PrefillParams &p) {
    ChunkId id;
    const int64_t wg = blockIdx.x;
    id.c = int32_t(wg % p.nC);
    id.bh = wg / p.nC;
    id.h = int32_t(id.bh % p.H);
    id.b = id.bh / p.H;
    id.t0 = int64_t(id.c) * kQ;
    const int64_t rem = p.T - id.t0;
    id.Tc = int32_t(rem < kQ ? rem : kQ);
    return id;
}

// Element offset of token t of (b, h) in a [b][T][H][R][D] tensor, rank r.
__device__ __forceinline__ int64_t tok_off(const PrefillParams &p, const ChunkId &id, int64_t t,
                                           int r, int D) {
    return (((id.b * p.T + t) * p.H + id.h) * p.R + r) * int64_t(D);
}

// Loads theta of the chunk into phi_s[s * KP + k] (fp32; 0 beyond Tc), then
// replaces it by the wrapped within-chunk inclusive cumulative angle.  The
// scan runs over the 64 tokens of a wavefront (one lane per token) in fp64;
// waves own pairs k = wave, wave + 4, ...  Returns nothing; the chunk totals
// Theta_c,k (fp64, unwrapped) are written to thetaC/thetaCS when
// write_totals is set.  Two __syncthreads inside; all threads must call.
template <typename IO, int K>
__device__ __forceinline__ void chunk_angles(const PrefillParams &p, const ChunkId &id, float *phi_s,
                                             bool write_totals) {
    constexpr int KP = K + 1;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const IO *theta = static_cast<const IO *>(p.theta);
    for (int i = tid; i < kQ * K; i += kThreads) {
        const int s = i / K, k = i - s * K;
        float v = 0.f;
        if (s < id.Tc) v = io<IO>::get(theta + ((id.b * p.T + id.t0 + s) * p.H + id.h) * K + k);
        phi_s[s * KP + k] = v;
    }
    __syncthreads();
    for (int k = wave; k < K; k += kThreads / kWave) {
        double v = double(phi_s[lane * KP + k]);
        v = wave_inclusive_sum(v, lane);
        const double w = wrap_angle(v);
        phi_s[lane * KP + k] = float(w);
        if (write_totals && lane == kWave - 1) {
            const int64_t o = (id.bh * p.nC + id.c) * K + k;
            p.thetaC[o] = v;
            double sn, cs;
            sincos(w, &sn, &cs);
            p.thetaCS[o] = make_float2(float(cs), float(sn));
        }
    }
    __syncthreads();
}

// Loads row v (= s * R + r) elements [8 q, 8 q + 8) of B or C of this chunk,
// rotated by R(-phi_loc[s]) pairwise and multiplied by `scale`; zeros for
// tokens beyond Tc.
template <typename IO, int K>
__device__ __forceinline__ void load_rotated8(const PrefillParams &p, const ChunkId &id, const IO *src,
                                              const float *phi_s, int v, int q, float scale,
                                              float out[8]) {
    constexpr int KP = K + 1;
    constexpr int N = 2 * K;
    const int s = v / p.R, r = v - s * p.R;
    if (s >= id.Tc) {
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = 0.f;
        return;
    }
    io<IO>::load8(src + tok_off(p, id, id.t0 + s, r, N) + 8 * q, out);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float sn, cs;
        __sincosf(phi_s[s * KP + 4 * q + j], &sn, &cs);
        rot_neg(cs, sn, out[2 * j], out[2 * j + 1]);
        out[2 * j] *= scale;
        out[2 * j + 1] *= scale;
    }
}

// Loads row v of x (elements [8 q, 8 q + 8)); zeros beyond Tc.
template <typename IO>
__device__ __forceinline__ void load_x8(const PrefillParams &p, const ChunkId &id, int v, int q,
                                        float out[8]) {
    const int s = v / p.R, r = v - s * p.R;
    if (s >= id.Tc) {
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = 0.f;
        return;
    }
    io<IO>::load8(static_cast<const IO *>(p.x) + tok_off(p, id, id.t0 + s, r, p.P) + 8 * q, out);
}

} // namespace m3
