// k_decode_step.hip -- one fused decode step for every (batch, head).
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
// head).  Workgroups of 256 threads walk the (b, h) items grid-stride; each
// thread owns float4 runs along P of the state, so every state access is a
// coalesced 16-byte access, and the state of the workgroup's next item is
// loaded while the current one is computed, so state loads are always in
// flight.  The small per-item vectors (B, C, x, x_prev, B~_prev) are read as
// 16-byte units spread over the threads; a thread holding a unit of B or C
// advances Phi for that unit's pairs (fp64 add and wrap, sin/cos of the angle
// in turns) and rotates it.  Values read from the carried state are written
// back only after the workgroup barrier, so no thread overwrites an input
// another thread still reads.
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

constexpr int kDecodeCus = 256; // compute units of an MI355X
// Resident decode workgroups per compute unit: each holds the state of two
// items (current and prefetched) in registers.
constexpr int decode_wg_per_cu(int N, int P) { return N * P > 4096 || (N > 64 && N * P >= 4096) ? 2 : 4; }

template <int N, int P>
struct DecodeLds {
    static constexpr int K = N / 2, P4 = P / 4;
    static constexpr int G = kThreads / P4; // row groups of the state
    // floats: bt, bp, ct [4][N]; x, xp [4][P]; phi' [K]; red [G][4][P]
    static constexpr int o_bt = 0, o_bp = o_bt + 4 * N, o_ct = o_bp + 4 * N;
    static constexpr int o_x = o_ct + 4 * N, o_xp = o_x + 4 * P, o_ph = o_xp + 4 * P;
    static constexpr int o_red = o_ph + (K + 3) / 4 * 4;
    static constexpr size_t floats = size_t(o_red) + size_t(G) * 4 * P;
};

// Rotation of one unit of B or C: EPU elements (EPU/2 pairs starting at
// pair k0) by -Phi' with Phi' = wrap(Phi + theta) (fp64 add and wrap; sin
// and cos of the angle in turns).  Writes Phi' of the pairs to phn when given.
template <typename IO>
__device__ __forceinline__ void rotate_unit(float *e, const float *phi, const IO *theta, int k0, float *phn) {
    constexpr int EPU = 16 / int(sizeof(IO));
    float ph[EPU / 2], th[EPU / 2];
    if constexpr (EPU == 8) {
        const float4 a = *reinterpret_cast<const float4 *>(phi + k0);
        ph[0] = a.x; ph[1] = a.y; ph[2] = a.z; ph[3] = a.w;
        io<IO>::load4(theta + k0, th);
    } else {
        const float2 a = *reinterpret_cast<const float2 *>(phi + k0);
        const float2 b = *reinterpret_cast<const float2 *>(theta + k0);
        ph[0] = a.x; ph[1] = a.y; th[0] = b.x; th[1] = b.y;
    }
#pragma unroll
    for (int j = 0; j < EPU / 2; ++j) {
        const double a = wrap_angle(double(ph[j]) + double(th[j]));
        float tf = float(a * (1.0 / kTwoPi));
        tf -= rintf(tf);
        const float sn = __builtin_amdgcn_sinf(tf), cs = __builtin_amdgcn_cosf(tf);
        rot_neg(cs, sn, e[2 * j], e[2 * j + 1]);
        if (phn) phn[j] = float(a);
    }
}

__device__ __forceinline__ void unpack16(const uint4 &u, float *v, bf16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(const uint4 &u, float *v, float) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}

template <typename IO, int N, int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_wg_per_cu(N, P)))) void k_decode_step(const DecodeParams p) {
    typedef DecodeLds<N, P> L;
    constexpr int K = N / 2, P4 = L::P4, G = L::G;
    constexpr int SZ = int(sizeof(IO)), EPU = 16 / SZ;
    constexpr int SLOTS = N * P4;                          // float4 runs in the state
    constexpr int SPT = (SLOTS + kThreads - 1) / kThreads; // runs per thread
    constexpr int URN = N * SZ / 16, URP = P * SZ / 16;    // 16-byte units per row of B/C and of x
    __shared__ __align__(16) float sm[L::floats];
    float *bt_s = sm + L::o_bt, *bp_s = sm + L::o_bp, *ct_s = sm + L::o_ct;
    float *x_s = sm + L::o_x, *xp_s = sm + L::o_xp, *ph_s = sm + L::o_ph, *red = sm + L::o_red;

    const int tid = threadIdx.x;
    const int R = p.R;
    const int64_t BH = p.batch * p.H;
    const int UB = R * URN, UX = R * URP, UPB = R * N / 4;
    const int pg = tid % P4, rg = tid / P4;

    auto load_state = [&](int64_t item, float4 *hv) {
        const float *hs = p.h + item * int64_t(N) * P;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int slot = tid + j * kThreads;
            if (slot < SLOTS) hv[j] = *reinterpret_cast<const float4 *>(hs + (slot / P4) * P + 4 * pg);
        }
    };

    float4 hv[SPT], hn[SPT];
    int64_t item = blockIdx.x;
    if (item < BH) load_state(item, hv);
    for (; item < BH; item += gridDim.x) {
        const int64_t next = item + gridDim.x;
        if (next < BH) load_state(next, hn);
        const int h = int(item % p.H);
        const float dtv = io<IO>::get(static_cast<const IO *>(p.dt) + item);
        const float lamv = io<IO>::get(static_cast<const IO *>(p.lam) + item);
        const float *phi = p.phi + item * K;
        const IO *theta = static_cast<const IO *>(p.theta) + item * K;

        // ---- small vectors: rotate B and C, stage them and x, x_prev, B~_prev
        for (int u = tid; u < 2 * UB + 2 * UX + UPB; u += kThreads) {
            if (u < 2 * UB) {
                const bool isC = u >= UB;
                const int w = isC ? u - UB : u;
                const int r = w / URN, q = w - r * URN;
                const IO *src = static_cast<const IO *>(isC ? p.C : p.B) + (item * R + r) * N + q * EPU;
                float e[EPU];
                unpack16(*reinterpret_cast<const uint4 *>(src), e, IO());
                rotate_unit<IO>(e, phi, theta, q * (EPU / 2), (!isC && r == 0) ? ph_s + q * (EPU / 2) : nullptr);
                float *dst = (isC ? ct_s : bt_s) + r * N + q * EPU;
#pragma unroll
                for (int i = 0; i < EPU; i += 4) *reinterpret_cast<float4 *>(dst + i) = make_float4(e[i], e[i + 1], e[i + 2], e[i + 3]);
            } else if (u < 2 * UB + 2 * UX) {
                const bool isP = u >= 2 * UB + UX;
                const int w = u - 2 * UB - (isP ? UX : 0);
                const IO *src = static_cast<const IO *>(isP ? p.prevx : p.x) + item * R * P + w * EPU;
                float e[EPU];
                unpack16(*reinterpret_cast<const uint4 *>(src), e, IO());
                float *dst = (isP ? xp_s : x_s) + w * EPU;
#pragma unroll
                for (int i = 0; i < EPU; i += 4) *reinterpret_cast<float4 *>(dst + i) = make_float4(e[i], e[i + 1], e[i + 2], e[i + 3]);
            } else {
                const int w = u - 2 * UB - 2 * UX;
                *reinterpret_cast<float4 *>(bp_s + 4 * w) = *reinterpret_cast<const float4 *>(p.prevB + item * R * N + 4 * w);
            }
        }
        __syncthreads();

        // ---- carried small state: B~_prev <- B~, x_prev <- x, Phi <- Phi'
        for (int w = tid; w < UPB; w += kThreads)
            *reinterpret_cast<float4 *>(p.prevB + item * R * N + 4 * w) = *reinterpret_cast<const float4 *>(bt_s + 4 * w);
        for (int w = tid; w < UX; w += kThreads) {
            const float *s = x_s + w * EPU;
            IO *d = static_cast<IO *>(p.prevx) + item * R * P + w * EPU;
#pragma unroll
            for (int i = 0; i < EPU; i += 4) io<IO>::store4(d + i, s + i);
        }
        for (int k = tid; k < K; k += kThreads) p.phi[item * K + k] = ph_s[k];

        // ---- state update and partial outputs
        const float alpha = __expf(dtv * p.A[h]);
        const float beta = (1.f - lamv) * dtv * alpha;
        const float gamma = lamv * dtv;
        float *hs = p.h + item * int64_t(N) * P;
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

        // y: four consecutive outputs per thread, one 4-element store
        IO *y = static_cast<IO *>(p.y) + item * R * P;
        constexpr int GACT = G < N ? G : N; // row groups that own at least one row
        for (int o = 4 * tid; o < R * P; o += 4 * kThreads) {
            const int i = o / P, pc = o - i * P;
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int r = 0; r < GACT; ++r) {
                const float4 v = *reinterpret_cast<const float4 *>(red + (r * 4 + i) * P + pc);
                s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
            }
            const float sv[4] = {s.x, s.y, s.z, s.w};
            io<IO>::store4(y + o, sv);
        }
#pragma unroll
        for (int j = 0; j < SPT; ++j) hv[j] = hn[j];
    }
}

#define M3_LAUNCH_DECODE(IO, NN, PP)                                                        \
    {                                                                                       \
        const int64_t cap = int64_t(kDecodeCus) * decode_wg_per_cu(NN, PP);                 \
        const dim3 grid{static_cast<unsigned>(bh < cap ? bh : cap)}, block{kThreads};       \
        hipLaunchKernelGGL((k_decode_step<IO, NN, PP>), grid, block, 0, s, p);              \
        return hipGetLastError();                                                           \
    }

hipError_t launch_decode_step(const DecodeParams &p, bool is_bf16, hipStream_t s) {
    const int64_t bh = p.batch * p.H;
    M3_DISPATCH(is_bf16, p.N, p.P, M3_LAUNCH_DECODE);
}

} // namespace m3
