// k_backward.hpp -- gradients of the mixer: one workgroup per (batch, head),
// sequential in time (the adjoint recurrence), fp32 arithmetic, fp64 angles.
//
// The forward map is the rotated-frame form of the Mamba-3 review, section
// 3.2.2, Prop. 3.2.3, with the coefficients of section 3.1.1, eq. (6), and
// the rank-R products of section 3.3:
//   h~_t = a_t h~_{t-1} + b_t B~_{t-1} x_{t-1}^T + g_t B~_t x_t^T,  y_t = C~_t^T h~_t,
//   B~_t = R(-Phi_t) B_t, C~_t = R(-Phi_t) C_t, Phi_t = Phi_{t-1} + theta_t,
//   a_t = exp(dt_t A), b_t = (1 - lam_t) dt_t a_t, g_t = lam_t dt_t.
// For L = sum <gy_t, y_t> the adjoint of h~_t is
//   G_t = C~_t gy_t + a_{t+1} G_{t+1}                      (G_T = 0)
// and, with M_t = g_t G_t + b_{t+1} G_{t+1},
//   d a_t = <G_t, h~_{t-1}>,  d b_t = <G_t, B~_{t-1} x_{t-1}^T>,  d g_t = <G_t, B~_t x_t^T>,
//   dB~_t = M_t x_t^T,  dx_t = B~_t^T M_t,  dC~_t = h~_t gy_t^T,
//   dB_t = R(Phi_t) dB~_t (same for C), and per row pair k
//   dPhi_t = sum_r (dB~[2k] B~[2k+1] - dB~[2k+1] B~[2k]) + (the same for C),
//   dtheta_t = sum_{s >= t} dPhi_s,
//   d dt = d a A a + d b (1 - lam)(a + dt A a) + d g lam,
//   d lam = -d b dt a + d g dt,  dA = sum_t (d a dt a + d b (1 - lam) dt^2 a);
// the carried state gets dh~_{-1} = a_0 G_0, dB~_{-1} = b_0 G_0 x_{-1}^T,
// dx_{-1} = b_0 B~_{-1}^T G_0 and dPhi_{-1} = sum_t dPhi_t.
//
// The states the adjoint needs are rebuilt chunk by chunk: a forward sweep
// stores the state and angle at every chunk start (workspace), then for each
// chunk, last to first, the chunk's states are recomputed into a per-sequence
// slab (workspace) with their angles' cos/sin in LDS, and the chunk's tokens
// are processed backwards.  Each thread owns float4 runs of the N x P state
// (along P); the small per-token vectors are staged in LDS, the next token's
// ones loaded into registers one step ahead.
#pragma once
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

constexpr int kQB = kBwdQ; // tokens per recomputed stretch

// Threads per workgroup: 512 for the larger MIMO states (measured on the
// b4 T2048 H64 P64 N64 R4 workload: 14.7 vs 17.8 ms), else 256 (SISO N128:
// 11.1 vs 12.1 ms).
constexpr int bwd_threads(int N, int P, int R) { return R >= 2 && N * P >= 4096 ? 512 : 256; }

template <int N, int P, int R>
struct BwdCfg {
    static constexpr int N_ = N, P_ = P, R_ = R;
    static constexpr int kBT = bwd_threads(N, P, R);
    static constexpr int K = N / 2, P4 = P / 4, RG = kBT / P4;
    static constexpr int SLOTS = N * P / 4, SPT = (SLOTS + kBT - 1) / kBT;
    // token buffer (floats): B~ [R][N], C~ [R][N], x [R][P], gy [R][P], theta [K], dt, lam
    static constexpr int t_b = 0, t_c = R * N, t_x = 2 * R * N, t_gy = t_x + R * P, t_th = t_gy + R * P;
    static constexpr int t_dt = t_th + K, t_lam = t_dt + 1, TB = (t_lam + 1 + 3) / 4 * 4;
    static constexpr int SV = t_lam + 1;                 // staged values per token
    static constexpr int SVPT = (SV + kBT - 1) / kBT;
    // LDS (floats): two token buffers, cos/sin table [kQB + 1][K] float2, dx
    // partials [RG][R][P], dB~ and dC~ [R][N], scalar partials
    static constexpr int o_tok = 0, o_cs = 2 * TB, o_red = o_cs + 2 * (kQB + 1) * K;
    static constexpr int o_gb = o_red + RG * R * P, o_gc = o_gb + R * N, o_sc = o_gc + R * N;
    static constexpr int floats = o_sc + 4 * (kBT / kWave);
    static constexpr size_t bytes = size_t(floats) * 4;
};

// Raw bits of one staged value of token t (t = -1: the carried previous
// token; values absent there read as zero).  The index is clamped, so every
// thread issues its loads.
template <class Cf, typename IO>
__device__ __forceinline__ uint32_t bwd_raw(const BwdParams &p, int64_t b, int h, int64_t t, int e) {
    constexpr int R = Cf::R_, N = Cf::N_, P = Cf::P_, K = Cf::K;
    const int i = min(e, Cf::SV - 1);
    if (t < 0) {
        const int64_t bh = b * p.H + h;
        if (!p.has_init || (i >= Cf::t_c && i < Cf::t_x) || i >= Cf::t_gy) return 0u;
        if (i < Cf::t_c) return __float_as_uint(p.prevB0[bh * R * N + i]);
        return io<IO>::raw(static_cast<const IO *>(p.prevx0) + bh * R * P + (i - Cf::t_x));
    }
    const int64_t tok = (b * p.T + t) * p.H + h;
    if (i < Cf::t_c) return io<IO>::raw(static_cast<const IO *>(p.B) + tok * R * N + i);
    if (i < Cf::t_x) return io<IO>::raw(static_cast<const IO *>(p.C) + tok * R * N + (i - Cf::t_c));
    if (i < Cf::t_gy) return io<IO>::raw(static_cast<const IO *>(p.x) + tok * R * P + (i - Cf::t_x));
    if (i < Cf::t_th) return io<IO>::raw(static_cast<const IO *>(p.gy) + tok * R * P + (i - Cf::t_gy));
    if (i < Cf::t_dt) return io<IO>::raw(static_cast<const IO *>(p.theta) + tok * K + (i - Cf::t_th));
    if (i == Cf::t_dt) return io<IO>::raw(static_cast<const IO *>(p.dt) + tok);
    return io<IO>::raw(static_cast<const IO *>(p.lam) + tok);
}

template <typename IO, int N, int P, int R>
__global__ __launch_bounds__(bwd_threads(N, P, R)) void k_backward(const BwdParams p) {
    typedef BwdCfg<N, P, R> Cf;
    constexpr int kBT = Cf::kBT;
    constexpr int K = Cf::K, P4 = Cf::P4, RG = Cf::RG, SLOTS = Cf::SLOTS, SPT = Cf::SPT, SVPT = Cf::SVPT;
    constexpr int TB = Cf::TB;
    extern __shared__ __align__(16) float sm[];
    float2 *cs = reinterpret_cast<float2 *>(sm + Cf::o_cs);
    float *red = sm + Cf::o_red, *gbs = sm + Cf::o_gb, *gcs = sm + Cf::o_gc, *scs = sm + Cf::o_sc;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t bh = blockIdx.x;
    const int h = int(bh % p.H);
    const int64_t b = bh / p.H;
    const float Ah = p.A[h];
    const int pg = tid % P4, rg = tid / P4;
    const int tslot = min(tid, SLOTS - 1);
    const bool own = tid < SLOTS || SLOTS % kBT == 0;

    // ---- small-vector staging: raw bits of one token into registers, then
    // into a token buffer as floats (B and C rotated in place by the owner of
    // each row pair, unless the token is the carried one, already rotated)
    auto tok_of = [&](int64_t t) -> float * { return sm + Cf::o_tok + (int(t & 1)) * TB; };
    uint32_t rv[SVPT];
    auto load_raw = [&](int64_t t) {
#pragma unroll
        for (int j = 0; j < SVPT; ++j) rv[j] = bwd_raw<Cf, IO>(p, b, h, t, tid + j * kBT);
    };
    auto store_raw = [&](int64_t t) {
        float *tb = tok_of(t);
#pragma unroll
        for (int j = 0; j < SVPT; ++j) {
            const int e = tid + j * kBT;
            if (e >= Cf::SV) continue;
            const bool fp = t < 0 && e < Cf::t_c; // carried B~ is fp32
            tb[e] = fp ? __uint_as_float(rv[j]) : io<IO>::value(rv[j]);
        }
    };
    // rotate token t's B and C by -Phi (cos/sin entry c)
    auto rotate_tok = [&](int64_t t, float2 c) {
        float *tb = tok_of(t);
        const int k = tid;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            rot_neg(c.x, c.y, tb[Cf::t_b + r * N + 2 * k], tb[Cf::t_b + r * N + 2 * k + 1]);
            rot_neg(c.x, c.y, tb[Cf::t_c + r * N + 2 * k], tb[Cf::t_c + r * N + 2 * k + 1]);
        }
    };
    auto cs_of = [](double a) {
        float tf = float(a * (1.0 / kTwoPi));
        tf -= rintf(tf);
        return make_float2(__builtin_amdgcn_cosf(tf), __builtin_amdgcn_sinf(tf));
    };
    // coefficients of token t from its buffer
    auto coef = [&](const float *tb, float &a, float &bt, float &g) {
        const float d = tb[Cf::t_dt], l = tb[Cf::t_lam];
        a = __expf(d * Ah);
        bt = (1.f - l) * d * a;
        g = l * d;
    };

    float4 hv[SPT];                 // running state (forward sweeps)
    double phi = 0.0;               // Phi of the last processed token (owners of a pair)

    // state of slot j into/out of a buffer of N x P floats
    auto ld_state = [&](const float *src, float4 *dst) {
#pragma unroll
        for (int j = 0; j < SPT; ++j) dst[j] = reinterpret_cast<const float4 *>(src)[j * kBT + tslot];
    };
    auto st_state = [&](float *dstp, const float4 *src) {
#pragma unroll
        for (int j = 0; j < SPT; ++j)
            if (own || j * kBT + tid < SLOTS) reinterpret_cast<float4 *>(dstp)[j * kBT + tid] = src[j];
    };

    // forward over tokens t0 .. t1-1 from hv, phi (token t0-1 staged and
    // rotated in its buffer); writes cos/sin of Phi_t to cs[t - t0 + 1] and,
    // with slab, the states after each token to slab[t - t0 + 1]
    auto forward = [&](int64_t t0, int64_t t1, float *slab) {
        load_raw(t0);
        for (int64_t t = t0; t < t1; ++t) {
            __syncthreads(); // buffer of token t is free (token t-2 consumed)
            store_raw(t);
            if (t + 1 < t1) load_raw(t + 1);
            __syncthreads();
            float *tb = tok_of(t);
            if (tid < K) {
                phi = wrap_angle(phi + double(tb[Cf::t_th + tid]));
                const float2 c = cs_of(phi);
                cs[int(t - t0 + 1) * K + tid] = c;
                rotate_tok(t, c);
            }
            __syncthreads();
            const float *tp = tok_of(t - 1);
            float a, bb, g;
            coef(tb, a, bb, g);
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                const int slot = j * kBT + tslot;
                const int n = slot / P4;
                float u[4] = {a * hv[j].x, a * hv[j].y, a * hv[j].z, a * hv[j].w};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float cb = bb * tp[Cf::t_b + r * N + n], cg = g * tb[Cf::t_b + r * N + n];
                    const float4 xp = *reinterpret_cast<const float4 *>(tp + Cf::t_x + r * P + 4 * pg);
                    const float4 xc = *reinterpret_cast<const float4 *>(tb + Cf::t_x + r * P + 4 * pg);
                    u[0] += cb * xp.x + cg * xc.x;
                    u[1] += cb * xp.y + cg * xc.y;
                    u[2] += cb * xp.z + cg * xc.z;
                    u[3] += cb * xp.w + cg * xc.w;
                }
                hv[j] = make_float4(u[0], u[1], u[2], u[3]);
            }
            if (slab) st_state(slab + (t - t0 + 1) * int64_t(N) * P, hv);
        }
    };
    // stage token t (t >= -1) synchronously, rotated with cos/sin entry c
    auto stage_sync = [&](int64_t t, float2 c) {
        load_raw(t);
        __syncthreads();
        store_raw(t);
        __syncthreads();
        if (tid < K && t >= 0) rotate_tok(t, c);
    };

    // ---- forward sweep: chunk-start checkpoints
    const int64_t T = p.T;
    const int nC = p.nC;
    float *ckh = p.ck_h + bh * nC * int64_t(N) * P;
    double *ckp = p.ck_phi + bh * nC * int64_t(K);
    float *slab = p.slab + bh * (kQB + 1) * int64_t(N) * P;
    if (p.has_init) ld_state(p.h0 + bh * int64_t(N) * P, hv);
    else
#pragma unroll
        for (int j = 0; j < SPT; ++j) hv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < K) phi = p.has_init ? double(p.phi0[bh * K + tid]) : 0.0;
    stage_sync(-1, make_float2(1.f, 0.f));
    for (int c = 0; c < nC; ++c) {
        st_state(ckh + c * int64_t(N) * P, hv);
        if (tid < K) ckp[c * K + tid] = phi;
        forward(int64_t(c) * kQB, min<int64_t>(T, int64_t(c + 1) * kQB), nullptr);
    }

    // ---- backward, chunk by chunk
    float4 Gn[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) Gn[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    float a1 = 0.f, b1 = 0.f; // a_{t+1}, b_{t+1}
    double acc = 0.0;         // running sum of dPhi (owners of a pair)
    float gA = 0.f;
    for (int c = nC - 1; c >= 0; --c) {
        const int64_t t0 = int64_t(c) * kQB, t1 = min<int64_t>(T, t0 + kQB);
        const int Tc = int(t1 - t0);
        // recompute the chunk's states from its checkpoint
        __syncthreads();
        ld_state(ckh + c * int64_t(N) * P, hv);
        if (tid < K) {
            phi = ckp[c * K + tid];
            cs[tid] = cs_of(phi);
        }
        st_state(slab, hv);
        __syncthreads();
        stage_sync(t0 - 1, t0 >= 1 ? cs[tid < K ? tid : 0] : make_float2(1.f, 0.f));
        forward(t0, t1, slab);
        __syncthreads(); // slab and cos/sin table complete
        // stage tokens t1-1 and t1-2 (rotated), the first two the loop reads
        float4 hc[SPT], hp[SPT];
        ld_state(slab + Tc * int64_t(N) * P, hc);
        ld_state(slab + (Tc - 1) * int64_t(N) * P, hp);
        stage_sync(t1 - 1, cs[Tc * K + (tid < K ? tid : 0)]);
        stage_sync(t1 - 2, cs[(Tc - 1) * K + (tid < K ? tid : 0)]);
        __syncthreads();
        if (t1 - 3 >= t0 - 1) load_raw(t1 - 3);
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const int i = int(t - t0);
            const float *tb = tok_of(t), *tp = tok_of(t - 1);
            float a, bb, g;
            coef(tb, a, bb, g);
            float4 hn[SPT];
            if (i >= 1) ld_state(slab + (i - 1) * int64_t(N) * P, hn); // h~_{t-2}, next step's h~_{t-1}
            float sa = 0.f, sb = 0.f, sg = 0.f;
            float gxp[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) gxp[r][q] = 0.f;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                const int slot = j * kBT + tslot;
                const int n = slot / P4;
                float G[4] = {a1 * Gn[j].x, a1 * Gn[j].y, a1 * Gn[j].z, a1 * Gn[j].w};
                float bx[4] = {0.f, 0.f, 0.f, 0.f}, bxp[4] = {0.f, 0.f, 0.f, 0.f};
                float4 xr[R], gyr[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    xr[r] = *reinterpret_cast<const float4 *>(tb + Cf::t_x + r * P + 4 * pg);
                    gyr[r] = *reinterpret_cast<const float4 *>(tb + Cf::t_gy + r * P + 4 * pg);
                    const float4 xq = *reinterpret_cast<const float4 *>(tp + Cf::t_x + r * P + 4 * pg);
                    const float cc = tb[Cf::t_c + r * N + n], bc = tb[Cf::t_b + r * N + n], bq = tp[Cf::t_b + r * N + n];
                    G[0] += cc * gyr[r].x; G[1] += cc * gyr[r].y; G[2] += cc * gyr[r].z; G[3] += cc * gyr[r].w;
                    bx[0] += bc * xr[r].x; bx[1] += bc * xr[r].y; bx[2] += bc * xr[r].z; bx[3] += bc * xr[r].w;
                    bxp[0] += bq * xq.x; bxp[1] += bq * xq.y; bxp[2] += bq * xq.z; bxp[3] += bq * xq.w;
                }
                const float hq[4] = {hp[j].x, hp[j].y, hp[j].z, hp[j].w};
                const float gn[4] = {Gn[j].x, Gn[j].y, Gn[j].z, Gn[j].w};
                const float hcv[4] = {hc[j].x, hc[j].y, hc[j].z, hc[j].w};
                float M[4];
                const bool live = own || slot == j * kBT + tid;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sa += live ? G[q] * hq[q] : 0.f;
                    sb += live ? G[q] * bxp[q] : 0.f;
                    sg += live ? G[q] * bx[q] : 0.f;
                    M[q] = g * G[q] + b1 * gn[q];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float vb = M[0] * xr[r].x + M[1] * xr[r].y + M[2] * xr[r].z + M[3] * xr[r].w;
                    float vc = hcv[0] * gyr[r].x + hcv[1] * gyr[r].y + hcv[2] * gyr[r].z + hcv[3] * gyr[r].w;
                    vb = row_sum<P4>(vb);
                    vc = row_sum<P4>(vc);
                    if (pg == 0 && live) {
                        gbs[r * N + n] = vb;
                        gcs[r * N + n] = vc;
                    }
                    const float bc = tb[Cf::t_b + r * N + n];
#pragma unroll
                    for (int q = 0; q < 4; ++q) gxp[r][q] += live ? bc * M[q] : 0.f;
                }
                Gn[j] = make_float4(G[0], G[1], G[2], G[3]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                *reinterpret_cast<float4 *>(red + (rg * R + r) * P + 4 * pg) = make_float4(gxp[r][0], gxp[r][1], gxp[r][2], gxp[r][3]);
            // scalar partials: wave sums, then one value per wave in LDS
            sa = row_sum<16>(sa); sb = row_sum<16>(sb); sg = row_sum<16>(sg);
            sa += __shfl_xor(sa, 16); sb += __shfl_xor(sb, 16); sg += __shfl_xor(sg, 16);
            sa += __shfl_xor(sa, 32); sb += __shfl_xor(sb, 32); sg += __shfl_xor(sg, 32);
            if (lane == 0) {
                scs[wave * 4 + 0] = sa;
                scs[wave * 4 + 1] = sb;
                scs[wave * 4 + 2] = sg;
            }
            __syncthreads();
            const int64_t tok = (b * T + t) * p.H + h;
            if (tid == 0) {
                float da = 0.f, db = 0.f, dg = 0.f;
#pragma unroll
                for (int w = 0; w < kBT / kWave; ++w) da += scs[w * 4], db += scs[w * 4 + 1], dg += scs[w * 4 + 2];
                const float d = tb[Cf::t_dt], l = tb[Cf::t_lam];
                p.gdt[tok] = da * Ah * a + db * (1.f - l) * (a + d * Ah * a) + dg * l;
                p.glam[tok] = -db * d * a + dg * d;
                gA += da * d * a + db * (1.f - l) * d * d * a;
            }
            for (int o = tid; o < R * P; o += kBT) {
                float s = 0.f;
                for (int q = 0; q < RG && q * P4 < N * P4; ++q) s += red[q * R * P + o];
                p.gx[tok * R * P + o] = s;
            }
            if (tid < K) {
                const int k = tid;
                const float2 c = cs[(i + 1) * K + k];
                float dphi = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float gb0 = gbs[r * N + 2 * k], gb1 = gbs[r * N + 2 * k + 1];
                    const float gc0 = gcs[r * N + 2 * k], gc1 = gcs[r * N + 2 * k + 1];
                    const float b0 = tb[Cf::t_b + r * N + 2 * k], b1v = tb[Cf::t_b + r * N + 2 * k + 1];
                    const float c0 = tb[Cf::t_c + r * N + 2 * k], c1 = tb[Cf::t_c + r * N + 2 * k + 1];
                    dphi += gb0 * b1v - gb1 * b0 + gc0 * c1 - gc1 * c0;
                    // dB = R(Phi) dB~
                    p.gB[(tok * R + r) * N + 2 * k] = c.x * gb0 - c.y * gb1;
                    p.gB[(tok * R + r) * N + 2 * k + 1] = c.y * gb0 + c.x * gb1;
                    p.gC[(tok * R + r) * N + 2 * k] = c.x * gc0 - c.y * gc1;
                    p.gC[(tok * R + r) * N + 2 * k + 1] = c.y * gc0 + c.x * gc1;
                }
                acc += double(dphi);
                p.gtheta[tok * K + k] = float(acc);
            }
            a1 = a;
            b1 = bb;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                hc[j] = hp[j];
                if (i >= 1) hp[j] = hn[j];
            }
            __syncthreads(); // token t's buffer, gbs, gcs, red consumed
            if (t - 2 >= t0 - 1) {
                store_raw(t - 2);
                if (t - 3 >= t0 - 1) load_raw(t - 3);
                __syncthreads();
                if (tid < K && t - 2 >= 0) rotate_tok(t - 2, cs[(i - 1) * K + tid]);
            }
            __syncthreads();
        }
    }
    if (tid == 0) p.gA_part[bh] = gA;

    // ---- the carried state: G_0 is in Gn, a_0 = a1, b_0 = b1, token -1 in its buffer
    if (p.gh0) {
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const float4 v = make_float4(a1 * Gn[j].x, a1 * Gn[j].y, a1 * Gn[j].z, a1 * Gn[j].w);
            if (own || j * kBT + tid < SLOTS) reinterpret_cast<float4 *>(p.gh0 + bh * int64_t(N) * P)[j * kBT + tid] = v;
        }
    }
    if (p.gphi0 && tid < K) p.gphi0[bh * K + tid] = float(acc);
    if (p.gprevB0 || p.gprevx0) {
        const float *tp = tok_of(-1);
        float gxp[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) gxp[r][q] = 0.f;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int slot = j * kBT + tslot;
            const int n = slot / P4;
            const bool live = own || slot == j * kBT + tid;
            const float M[4] = {b1 * Gn[j].x, b1 * Gn[j].y, b1 * Gn[j].z, b1 * Gn[j].w};
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float4 xq = *reinterpret_cast<const float4 *>(tp + Cf::t_x + r * P + 4 * pg);
                float vb = M[0] * xq.x + M[1] * xq.y + M[2] * xq.z + M[3] * xq.w;
                vb = row_sum<P4>(vb);
                if (pg == 0 && live && p.gprevB0) p.gprevB0[(bh * R + r) * N + n] = vb;
                const float bq = tp[Cf::t_b + r * N + n];
#pragma unroll
                for (int q = 0; q < 4; ++q) gxp[r][q] += live ? bq * M[q] : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            *reinterpret_cast<float4 *>(red + (rg * R + r) * P + 4 * pg) = make_float4(gxp[r][0], gxp[r][1], gxp[r][2], gxp[r][3]);
        __syncthreads();
        if (p.gprevx0)
            for (int o = tid; o < R * P; o += kBT) {
                float s = 0.f;
                for (int q = 0; q < RG && q * P4 < N * P4; ++q) s += red[q * R * P + o];
                p.gprevx0[bh * R * P + o] = s;
            }
    }
}

} // namespace m3

namespace m3 {

// Sum of the per-(batch, head) partials of dA over the batch.
static __global__ void k_backward_gA(const BwdParams p) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= p.H) return;
    float s = 0.f;
    for (int64_t b = 0; b < p.batch; ++b) s += p.gA_part[b * p.H + h];
    p.gA[h] = s;
}

template <typename IO, int N, int P, int R>
hipError_t launch_backward_inst(const BwdParams &p, hipStream_t s) {
    typedef BwdCfg<N, P, R> Cf;
    if (Cf::bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_backward<IO, N, P, R>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(Cf::bytes));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_backward<IO, N, P, R>), dim3(unsigned(p.batch * p.H)), dim3(Cf::kBT), Cf::bytes, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_backward_gA, dim3(unsigned((p.H + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_backward_io(const BwdParams &p, hipStream_t s) {
#define M3_BWD_R(NN, PP)                                                      \
    switch (p.R) {                                                            \
    case 1: return launch_backward_inst<IO, NN, PP, 1>(p, s);                 \
    case 2: return launch_backward_inst<IO, NN, PP, 2>(p, s);                 \
    case 3: return launch_backward_inst<IO, NN, PP, 3>(p, s);                 \
    case 4: return launch_backward_inst<IO, NN, PP, 4>(p, s);                 \
    default: return hipErrorInvalidValue;                                     \
    }
#define M3_BWD_P(NN)                                                          \
    switch (p.P) {                                                            \
    case 16: M3_BWD_R(NN, 16)                                                 \
    case 32: M3_BWD_R(NN, 32)                                                 \
    case 64: M3_BWD_R(NN, 64)                                                 \
    default: return hipErrorInvalidValue;                                     \
    }
    switch (p.N) {
    case 16: M3_BWD_P(16)
    case 32: M3_BWD_P(32)
    case 64: M3_BWD_P(64)
    case 128: M3_BWD_P(128)
    default: return hipErrorInvalidValue;
    }
#undef M3_BWD_P
#undef M3_BWD_R
}

} // namespace m3
