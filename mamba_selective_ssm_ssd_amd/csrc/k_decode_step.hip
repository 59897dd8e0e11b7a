// k_decode_step.hip -- one fused decode step per (batch, head).
//
// In the rotated (RoPE) frame of the Mamba-3 review, section 3.2.2,
// Prop. 3.2.3, with the exponential-trapezoidal coefficients of section
// 3.1.1, eq. (6), and the rank-R MIMO update of section 3.3:
//   Phi   <- wrap(Phi + theta_t)                       (per rotation pair)
//   B~    =  R(-Phi) B_t,   C~ = R(-Phi) C_t
//   h~    <- alpha h~ + beta B~_prev x_prev^T + gamma B~ x_t^T
//   y_t   =  C~^T h~
//   B~_prev <- B~,  x_prev <- x_t
// with alpha = exp(dt A), beta = (1 - lam) dt alpha, gamma = lam dt.
//
// Decode is bound by the read-modify-write of the fp32 state (N x P per
// head).  One workgroup of 256 threads owns one (b, h); each thread owns
// float4 runs along P, so every state access is a coalesced 16-byte access,
// and the loads of all its rows are issued before any arithmetic.  The small
// per-head vectors (B~, B~_prev, C~, x, x_prev) are staged in LDS; the output
// reduction over N goes through LDS.
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

template <int N, int P>
struct DecodeLds {
    static constexpr int P4 = P / 4;
    static constexpr int G = kThreads / P4; // row groups
    // floats: bt, bp, ct [4][N]; x, xp [4][P]; cs [N/2][2]; red [G][4][P]
    static constexpr size_t floats = 3 * 4 * N + 2 * 4 * P + N + size_t(G) * 4 * P;
    static constexpr size_t bytes = floats * sizeof(float);
};

template <typename IO, int N, int P>
__global__ __launch_bounds__(kThreads) void k_decode_step(const DecodeParams p) {
    typedef DecodeLds<N, P> L;
    constexpr int K = N / 2, P4 = L::P4, G = L::G;
    constexpr int SLOTS = N * P4;                                  // float4 runs in the state
    constexpr int SPT = (SLOTS + kThreads - 1) / kThreads;         // runs per thread
    __shared__ __align__(16) float sm[L::floats];
    float *bt_s = sm, *bp_s = bt_s + 4 * N, *ct_s = bp_s + 4 * N;
    float *x_s = ct_s + 4 * N, *xp_s = x_s + 4 * P;
    float *cs_s = xp_s + 4 * P;
    float *red = cs_s + N;

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int h = int(bh % p.H);
    const int R = p.R;
    const IO *xin = static_cast<const IO *>(p.x) + bh * R * P;
    IO *prevx = static_cast<IO *>(p.prevx) + bh * R * P;
    float *hs = p.h + bh * int64_t(N) * P;

    // state loads first: they are the bulk of the traffic
    const int pg = tid % P4, rg = tid / P4;
    float4 hv[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int slot = tid + j * kThreads;
        if (slot < SLOTS) hv[j] = *reinterpret_cast<const float4 *>(hs + (slot / P4) * P + 4 * pg);
    }

    const float dtv = io<IO>::get(static_cast<const IO *>(p.dt) + bh);
    const float lamv = io<IO>::get(static_cast<const IO *>(p.lam) + bh);
    const float alpha = expf(dtv * p.A[h]);
    const float beta = (1.f - lamv) * dtv * alpha;
    const float gamma = lamv * dtv;

    if (tid < K) {
        const double ph = wrap_angle(double(p.phi[bh * K + tid]) +
                                     double(io<IO>::get(static_cast<const IO *>(p.theta) + bh * K + tid)));
        float sn, cs;
        sincos_wrapped(ph, &sn, &cs);
        cs_s[2 * tid] = cs;
        cs_s[2 * tid + 1] = sn;
        p.phi[bh * K + tid] = float(ph);
    }
    for (int i = tid; i < R * N; i += kThreads) bp_s[i] = p.prevB[bh * R * N + i];
    for (int i = tid; i < R * P; i += kThreads) {
        xp_s[i] = io<IO>::get(prevx + i);
        x_s[i] = io<IO>::get(xin + i);
    }
    __syncthreads();

    // rotate B and C by -Phi; the new B~ and x become the carried previous token
    const IO *Bin = static_cast<const IO *>(p.B) + bh * R * N;
    const IO *Cin = static_cast<const IO *>(p.C) + bh * R * N;
    for (int i = tid; i < 2 * R * K; i += kThreads) {
        const bool isC = i >= R * K;
        const int j = isC ? i - R * K : i;
        const int r = j / K, k = j - r * K;
        const IO *src = (isC ? Cin : Bin) + r * N + 2 * k;
        float u = io<IO>::get(src), v = io<IO>::get(src + 1);
        rot_neg(cs_s[2 * k], cs_s[2 * k + 1], u, v);
        float *dst = (isC ? ct_s : bt_s) + r * N + 2 * k;
        dst[0] = u;
        dst[1] = v;
        if (!isC) {
            p.prevB[(bh * R + r) * N + 2 * k] = u;
            p.prevB[(bh * R + r) * N + 2 * k + 1] = v;
        }
    }
    for (int i = tid; i < R * P; i += kThreads) prevx[i] = xin[i];
    __syncthreads();

    // state update and partial outputs
    float yp[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) yp[i][q] = 0.f;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int slot = tid + j * kThreads;
        if (slot >= SLOTS) continue;
        const int n = slot / P4;
        float u[4] = {alpha * hv[j].x, alpha * hv[j].y, alpha * hv[j].z, alpha * hv[j].w};
        for (int r = 0; r < R; ++r) {
            const float cb = beta * bp_s[r * N + n], cg = gamma * bt_s[r * N + n];
            const float4 xp4 = *reinterpret_cast<const float4 *>(xp_s + r * P + 4 * pg);
            const float4 x4 = *reinterpret_cast<const float4 *>(x_s + r * P + 4 * pg);
            u[0] += cb * xp4.x + cg * x4.x;
            u[1] += cb * xp4.y + cg * x4.y;
            u[2] += cb * xp4.z + cg * x4.z;
            u[3] += cb * xp4.w + cg * x4.w;
        }
        *reinterpret_cast<float4 *>(hs + n * P + 4 * pg) = make_float4(u[0], u[1], u[2], u[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < R) {
                const float cc = ct_s[i * N + n];
#pragma unroll
                for (int q = 0; q < 4; ++q) yp[i][q] += cc * u[q];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < R)
            *reinterpret_cast<float4 *>(red + (rg * 4 + i) * P + 4 * pg) =
                make_float4(yp[i][0], yp[i][1], yp[i][2], yp[i][3]);
    __syncthreads();

    IO *y = static_cast<IO *>(p.y) + bh * R * P;
    constexpr int GACT = G < N ? G : N; // row groups that own at least one row
    for (int o = tid; o < R * P; o += kThreads) {
        const int i = o / P, pc = o - i * P;
        float s = 0.f;
        for (int r = 0; r < GACT; ++r) s += red[(r * 4 + i) * P + pc];
        io<IO>::put(y + o, s);
    }
}

#define M3_LAUNCH_DECODE(IO, NN, PP)                                                        \
    {                                                                                       \
        hipLaunchKernelGGL((k_decode_step<IO, NN, PP>), grid, block, 0, s, p);              \
        return hipGetLastError();                                                           \
    }

hipError_t launch_decode_step(const DecodeParams &p, bool is_bf16, hipStream_t s) {
    const dim3 grid(unsigned(p.batch * p.H)), block(kThreads);
    M3_DISPATCH(is_bf16, p.N, p.P, M3_LAUNCH_DECODE);
}

} // namespace m3
