// k_prefill.hpp -- the chunked prefill as one persistent kernel per
// (batch, head, segment of chunks).
//
// Method (Mamba-3 review, junhanzang.github.io): the exponential-trapezoidal
// recurrence of section 3.1.1 (Prop. 3.1.1, eqs. (5)-(6)) with the complex
// state of section 3.2 realised as a data-dependent rotation of B and C
// (Props. 3.2.1-3.2.3) and the rank-R MIMO update of section 3.3, evaluated
// in the chunked SSD form: section 2.3 (Y = (L o C B^T) X) with the mask of
// section 3.1.3, eq. (7) (decay matrix times 2-band matrix), chunk by chunk,
// intra-chunk by matrix products and inter-chunk by passing the state at the
// chunk ends (the "20.2 Mamba and S6" page, sungeuns.github.io, section 2).
//
// Per chunk c (tokens t0 .. t0+Tc-1, virtual rows v = s*R + r):
//  a1  cumsum: ell_t = sum_{t0<=u<=t} dt_u A (one lane per token, wave scan),
//      gam_t = lam_t dt_t, wgt_t = gam_t + delta_{t+1}, delta = (1-lam) dt,
//      g_c = ell at the last token; angle prefix phi_t,k = sum theta (fp64
//      wave scan, wrapped to [-pi, pi)) and the chunk total Theta_c,k.
//  a2  rotate: Bhat = R(-phi_t) B_t, Chat = R(-phi_t) C_t, i.e. the RoPE form
//      relative to the chunk start.  The rotation accumulated before the chunk
//      is carried by the state, which is kept in the frame of the chunk start.
//  a3  intra-chunk (MFMA): S = Chat Bhat^T per 16x16 block,
//      M = S * Lmask(tt, ts) with Lmask = gam_tt on the diagonal token,
//      exp(ell_tt - ell_ts) wgt_ts below it, 0 above (the closed form of
//      Decay . Band, every factor <= 1), y_intra = M x.
//  a4  inter-chunk (MFMA + registers): the state entering the next chunk,
//      H <- R(Theta_c) (exp(g_c) H + sum_v exp(g_c - ell_s) wgt_s Bhat[v] x[v]^T),
//      kept in fp32 registers across chunks (never written to memory).
//  a5  combine: y = y_intra + exp(ell_tt) Chat H  (H of the previous chunk).
//
// A long sequence on few heads is split into segments so the grid fills the
// chip; a pre-pass (OUT = false) computes each segment's aggregate (its state
// from zero, summed log decay and angle) and each output workgroup folds the
// aggregates of the segments before it into its starting state.
//
// Data layout: one workgroup of 512 threads (8 waves).  The next chunk's
// inputs are loaded into registers while the current chunk computes.  LDS
// holds the rotated B (row-major for S, transposed and scaled for the state
// update), x transposed, the state H (bf16 or fp32, transposed) and the
// angle table; the rotated C of a wave's 16-row blocks stays in registers.
#pragma once

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

constexpr int kPT = 512;         // threads per prefill workgroup
constexpr int kPW = kPT / kWave; // waves per prefill workgroup

constexpr size_t align16(size_t v) { return (v + 15) / 16 * 16; }

template <typename IO, int N_, int P_, int R_>
struct Cfg {
    static constexpr int N = N_, P = P_, R = R_, K = N / 2, KP = K + 1, V = kQ * R;
    typedef Mma<mode<IO>::f32> M;
    typedef typename M::lds_t lds_t;
    typedef typename M::frag frag;
    static constexpr int SZ = int(sizeof(IO));
    static constexpr int EPU = 16 / SZ;                       // I/O elements per 16-byte unit
    static constexpr int PADE = 16 / int(sizeof(lds_t));      // 16 bytes of row padding
    static constexpr int NBP = N + PADE;                      // row pitch of bs, ht
    static constexpr int VP = V + PADE;                       // row pitch of bst, xt
    static constexpr int NTB = V / 16;                        // 16-row blocks of virtual rows
    static constexpr int TBW = NTB > kPW ? 2 : 1;             // blocks per wave
    static constexpr int NKS = N >= 32 ? N / 32 : 1;          // K-steps of 32 over N
    static constexpr int NT = N / 16, PT = P / 16, NTILE = NT * PT;
    static constexpr int TW = (NTILE + kPW - 1) / kPW;        // state tiles per wave
    // 16-byte units of one chunk's inputs, and units per thread
    static constexpr int URT = K * SZ / 16, UT = kQ * URT, UPT_T = (UT + kPT - 1) / kPT;
    static constexpr int URB = N * SZ / 16, UB = V * URB, UPT_B = (UB + kPT - 1) / kPT;
    static constexpr int URX = P * SZ / 16, UX = V * URX, UPT_X = (UX + kPT - 1) / kPT;
    static constexpr int FU = 8 / EPU; // units per MFMA fragment (8 elements)
    // blocked angle prefix: thread (k, blk), NB blocks of TPB tokens per pair
    static constexpr int NB = kPT / K, TPB = kQ / NB;
    static_assert(NB * TPB == kQ, "angle blocks");
    // LDS layout, bytes
    static constexpr size_t o_coef = 0;                       // ell, gam, wgt, scl [64] each
    static constexpr size_t o_misc = o_coef + 4 * kQ * 4;     // g_c, delta_0
    static constexpr size_t o_thc = o_misc + 64;              // float2 [K]: cos, sin Theta_c
    static constexpr size_t o_ths = o_thc + size_t(K) * 8;    // double [K]: running angle
    static constexpr size_t o_phi = o_ths + size_t(K) * 8;    // float [64][KP]
    static constexpr size_t o_bs = align16(o_phi + size_t(kQ) * KP * 4);    // [V][NBP]
    static constexpr size_t bst_bytes = size_t(N) * VP * sizeof(lds_t);     // [N][VP]
    static constexpr size_t rest_bytes = size_t(P) * VP * sizeof(lds_t) + size_t(P) * NBP * sizeof(lds_t);
    // The transposed, scaled copy of B (contiguous along v for the state
    // update) is kept when it fits; otherwise that operand is gathered from
    // the row-major copy.
    static constexpr bool BST = o_bs + size_t(V) * NBP * sizeof(lds_t) + bst_bytes + rest_bytes <= kMaxLdsBytes;
    static constexpr size_t o_bst = o_bs + size_t(V) * NBP * sizeof(lds_t);
    static constexpr size_t o_xt = o_bst + (BST ? bst_bytes : 0);            // [P][VP]
    static constexpr size_t o_ht = o_xt + size_t(P) * VP * sizeof(lds_t);   // [P][NBP]
    // block sums of the angle prefix (double [NB][K]) live in the staging
    // region of B and x, which is free between the end of a chunk's compute
    // and its staging
    static constexpr size_t o_blk = o_bs;
    static constexpr size_t o_pro = o_blk + size_t(kPT) * 8;  // a [64], del [65] (prologue only)
    static_assert(o_ht - o_bs >= size_t(kPT) * 8 + (2 * kQ + 4) * 4, "prologue data fits in the staging region");
    static constexpr size_t bytes = o_ht + size_t(P) * NBP * sizeof(lds_t);
    static_assert(K * SZ % 16 == 0 && N % 16 == 0 && P % 16 == 0, "tile sizes");
};

// Raw (undecoded) inputs of one chunk held in registers.
template <class C>
struct RawChunk {
    uint4 th[C::UPT_T], bb[C::UPT_B], xx[C::UPT_X];
    uint4 cc[C::TBW][C::NKS][C::FU];
    float dt, lam, deln;
};

// Unpack one 16-byte unit into EPU floats.
__device__ __forceinline__ void unpack_unit(const uint4 &u, float *v, bf16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack_unit(const uint4 &u, float *v, float) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}

// Store EPU floats as consecutive LDS elements (one 16-byte store).
__device__ __forceinline__ void st_unit(uint16_t *p, const float *v) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                                               pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
}
__device__ __forceinline__ void st_unit(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_one(uint16_t *p, float v) { *p = f32_to_bits(v); }
__device__ __forceinline__ float lds_to_f32(uint16_t v) { return bits_to_f32(v); }
__device__ __forceinline__ float lds_to_f32(float v) { return v; }
__device__ __forceinline__ void st_one(float *p, float v) { *p = v; }
// Four consecutive LDS elements.
__device__ __forceinline__ void st_four(uint16_t *p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}
__device__ __forceinline__ void st_four(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Virtual-row block i (< TBW) of a wave: blocks w and 2*kPW-1-w, so that the
// causal work of the two blocks balances across waves.
__device__ __forceinline__ int wave_block(int i, int wave) { return i == 0 ? wave : 2 * kPW - 1 - wave; }

// Loads chunk (b, h, t0 .. t0+Tc-1) into registers.  Addresses are a
// uniform per-chunk base plus a 32-bit per-thread offset, so they stay in
// scalar registers + one VGPR per load (saddr + voffset addressing).
template <class C, typename IO, bool OUT>
__device__ __forceinline__ void load_chunk(const PrefillParams &p, int64_t b, int h, int64_t t0, int Tc,
                                           RawChunk<C> &r) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, l16 = lane & 15;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const int64_t tokbase = (b * p.T + t0) * p.H + h; // token-head index of t0
    const int H = p.H;
    const IO *th = static_cast<const IO *>(p.theta) + tokbase * C::K;
    const IO *Bp = static_cast<const IO *>(p.B) + tokbase * (C::R * C::N);
    const IO *Xp = static_cast<const IO *>(p.x) + tokbase * (C::R * C::P);
    const IO *Cp = static_cast<const IO *>(p.C) + tokbase * (C::R * C::N);
#pragma unroll
    for (int j = 0; j < C::UPT_T; ++j) {
        const int u = tid + j * kPT;
        r.th[j] = z;
        if (u < C::UT) {
            const int tok = u / C::URT, q = u - tok * C::URT;
            if (tok < Tc) r.th[j] = *reinterpret_cast<const uint4 *>(th + (tok * H * C::K + q * C::EPU));
        }
    }
#pragma unroll
    for (int j = 0; j < C::UPT_B; ++j) {
        const int u = tid + j * kPT;
        r.bb[j] = z;
        if (u < C::UB) {
            const int v = u / C::URB, q = u - v * C::URB;
            const int tok = v / C::R, ch = v - tok * C::R;
            if (tok < Tc)
                r.bb[j] = *reinterpret_cast<const uint4 *>(Bp + ((tok * H * C::R + ch) * C::N + q * C::EPU));
        }
    }
#pragma unroll
    for (int j = 0; j < C::UPT_X; ++j) {
        const int u = tid + j * kPT;
        r.xx[j] = z;
        if (u < C::UX) {
            const int v = u / C::URX, q = u - v * C::URX;
            const int tok = v / C::R, ch = v - tok * C::R;
            if (tok < Tc)
                r.xx[j] = *reinterpret_cast<const uint4 *>(Xp + ((tok * H * C::R + ch) * C::P + q * C::EPU));
        }
    }
    if (OUT) {
#pragma unroll
        for (int i = 0; i < C::TBW; ++i) {
            const int tb = wave_block(i, wave);
            const int v = 16 * tb + l16;
            const int tok = v / C::R, ch = v - tok * C::R;
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                const int n0 = 32 * ks + 8 * g;
#pragma unroll
                for (int f = 0; f < C::FU; ++f) {
                    r.cc[i][ks][f] = z;
                    if (tb < C::NTB && n0 < C::N && tok < Tc)
                        r.cc[i][ks][f] = *reinterpret_cast<const uint4 *>(
                            Cp + ((tok * H * C::R + ch) * C::N + n0 + f * C::EPU));
                }
            }
        }
    }
    if (wave == 0) {
        const IO *dt = static_cast<const IO *>(p.dt) + tokbase;
        const IO *lam = static_cast<const IO *>(p.lam) + tokbase;
        r.dt = 0.f;
        r.lam = 0.f;
        r.deln = 0.f;
        if (lane < Tc) {
            r.dt = io<IO>::get(dt + lane * H);
            r.lam = io<IO>::get(lam + lane * H);
        }
        if (lane == kWave - 1 && t0 + kQ < p.T) {
            const float dn = io<IO>::get(dt + kQ * H);
            const float ln = io<IO>::get(lam + kQ * H);
            r.deln = (1.f - ln) * dn;
        }
    }
}

// State entering the sequence, as one 16x16 tile of this lane (rows
// n = 16 nt + 4 g + v, column 16 pt + l16), in the state's own frame at the
// sequence start: R(Phi_{-1}) (h~ + delta_0 B~_prev x_prev^T).
template <class C, typename IO>
__device__ __forceinline__ floatx4 fold_init(const PrefillParams &p, int64_t bh, int nt, int pt, float del0) {
    const int lane = threadIdx.x & (kWave - 1), g = lane >> 4, l16 = lane & 15;
    const int pc = 16 * pt + l16;
    const float *h0 = p.h0 + bh * int64_t(C::N) * C::P;
    const float *pb = p.prevB0 + bh * int64_t(C::R) * C::N;
    const IO *px = static_cast<const IO *>(p.prevx0) + bh * int64_t(C::R) * C::P;
    float a[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int n = 16 * nt + 4 * g + v;
        float s = h0[n * C::P + pc];
#pragma unroll
        for (int r = 0; r < C::R; ++r) s += del0 * pb[r * C::N + n] * io<IO>::get(px + r * C::P + pc);
        a[v] = s;
    }
    floatx4 o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int k = 8 * nt + 2 * g + q;
        float sn, cs;
        sincos_wrapped(wrap_angle(double(p.phi0[bh * C::K + k])), &sn, &cs);
        o[2 * q] = cs * a[2 * q] - sn * a[2 * q + 1];
        o[2 * q + 1] = sn * a[2 * q] + cs * a[2 * q + 1];
    }
    return o;
}

template <typename IO, int N, int P, int R, bool OUT>
__global__ __launch_bounds__(kPT) void k_prefill(const PrefillParams p) {
    typedef Cfg<IO, N, P, R> C;
    typedef typename C::M M;
    typedef typename C::lds_t lds_t;
    typedef typename C::frag frag;
    constexpr int K = C::K, KP = C::KP, V = C::V, NBP = C::NBP, VP = C::VP, EPU = C::EPU;
    constexpr int PT = C::PT, NKS = C::NKS;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, l16 = lane & 15;

    // workgroup -> (b, h, segment); consecutive heads land on the same XCD
    const int nseg = OUT ? p.S : p.S - 1;
    const int64_t total = p.batch * p.H * nseg;
    int64_t li = blockIdx.x;
    if (total % 8 == 0) li = int64_t(blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
    const int seg = int(li % nseg);
    const int64_t bh = li / nseg;
    const int h = int(bh % p.H);
    const int64_t b = bh / p.H;
    const int c_begin = seg * p.cps;
    const int c_end = min(p.nC, c_begin + p.cps);

    extern __shared__ __align__(16) unsigned char smem[];
    float *ell_s = reinterpret_cast<float *>(smem + C::o_coef);
    float *gam_s = ell_s + kQ, *wgt_s = gam_s + kQ, *scl_s = wgt_s + kQ;
    float *a_s = reinterpret_cast<float *>(smem + C::o_pro), *del_s = a_s + kQ;
    double *blk_s = reinterpret_cast<double *>(smem + C::o_blk);
    float *misc_s = reinterpret_cast<float *>(smem + C::o_misc);
    float2 *thc_s = reinterpret_cast<float2 *>(smem + C::o_thc);
    double *ths_s = reinterpret_cast<double *>(smem + C::o_ths);
    float *phi_s = reinterpret_cast<float *>(smem + C::o_phi);
    lds_t *bs = reinterpret_cast<lds_t *>(smem + C::o_bs);
    lds_t *bst = reinterpret_cast<lds_t *>(smem + C::o_bst);
    lds_t *xt = reinterpret_cast<lds_t *>(smem + C::o_xt);
    lds_t *ht = reinterpret_cast<lds_t *>(smem + C::o_ht);

    // running angle: Phi_{-1} plus the segments before this one (output pass)
    for (int k = tid; k < K; k += kPT) {
        double a = 0.0;
        if (OUT && p.has_init) a = p.S == 1 ? double(p.phi0[bh * K + k]) : p.phi0ws[bh * K + k];
        if (OUT)
            for (int s2 = 0; s2 < seg; ++s2) a += p.segTh[(bh * p.S + s2) * K + k];
        ths_s[k] = a;
    }

    floatx4 st[C::TW];
#pragma unroll
    for (int j = 0; j < C::TW; ++j) st[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    float gsum = 0.f;
    const float Ah = p.A[h];

    RawChunk<C> raw;
    {
        const int64_t t0 = int64_t(c_begin) * kQ;
        load_chunk<C, IO, OUT>(p, b, h, t0, int(min<int64_t>(kQ, p.T - t0)), raw);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int64_t t0 = int64_t(c) * kQ;
        const int Tc = int(min<int64_t>(kQ, p.T - t0));

        // ---- (1) theta to LDS; a1: decay and trapezoid coefficients (wave 0)
#pragma unroll
        for (int j = 0; j < C::UPT_T; ++j) {
            const int u = tid + j * kPT;
            if (u < C::UT) {
                const int tok = u / C::URT, q = u - tok * C::URT;
                float v[EPU];
                unpack_unit(raw.th[j], v, IO());
#pragma unroll
                for (int e = 0; e < EPU; ++e) phi_s[tok * KP + q * EPU + e] = v[e];
            }
        }
        if (wave == 0) {
            const float d = raw.dt, l = raw.lam;
            a_s[lane] = d * Ah;
            gam_s[lane] = l * d;
            const float del = (1.f - l) * d;
            del_s[lane] = del;
            if (lane == kWave - 1) del_s[kQ] = raw.deln; // first token of the next chunk
        }
        __syncthreads();

        // ---- a1: within-chunk prefix sums.  Rotary angles in fp64, blocked:
        // thread (k, blk) scans its TPB tokens serially, block totals go
        // through LDS.  Log decay in fp32 by wave 0 (lane = token).
        double loc[C::TPB];
        const int ak = tid % K, ablk = tid / K;
        {
            double acc = 0.0;
#pragma unroll
            for (int i = 0; i < C::TPB; ++i) {
                acc += double(phi_s[(ablk * C::TPB + i) * KP + ak]);
                loc[i] = acc;
            }
            blk_s[ablk * K + ak] = acc;
        }
        if (wave == 0) {
            float ell = 0.f;
#pragma unroll
            for (int m = 0; m < kQ / 4; ++m) {
                const float4 a4 = *reinterpret_cast<const float4 *>(a_s + 4 * m);
                ell += (4 * m + 0 <= lane ? a4.x : 0.f);
                ell += (4 * m + 1 <= lane ? a4.y : 0.f);
                ell += (4 * m + 2 <= lane ? a4.z : 0.f);
                ell += (4 * m + 3 <= lane ? a4.w : 0.f);
            }
            const float gc = __shfl(ell, Tc - 1, kWave);
            float dn = lane + 1 < kQ ? del_s[lane + 1] : del_s[kQ];
            if (t0 + lane + 1 >= p.T) dn = 0.f;
            const float w = gam_s[lane] + dn;
            ell_s[lane] = ell;
            wgt_s[lane] = w;
            scl_s[lane] = lane < Tc ? __expf(gc - ell) * w : 0.f;
            if (lane == 0) {
                misc_s[0] = gc;
                misc_s[1] = del_s[0];
            }
        }
        __syncthreads();
        {
            double off = 0.0;
            for (int b2 = 0; b2 < ablk; ++b2) off += blk_s[b2 * K + ak];
#pragma unroll
            for (int i = 0; i < C::TPB; ++i)
                phi_s[(ablk * C::TPB + i) * KP + ak] = float(wrap_angle(off + loc[i]));
            if (ablk == C::NB - 1) {
                const double tot = off + loc[C::TPB - 1];
                float sn, cs;
                sincos_wrapped(wrap_angle(tot), &sn, &cs);
                thc_s[ak] = make_float2(cs, sn);
                ths_s[ak] += tot;
            }
        }
        __syncthreads();

        // ---- a2: rotate B and C, stage B, x in LDS; C fragments to registers
#pragma unroll
        for (int j = 0; j < C::UPT_B; ++j) {
            const int u = tid + j * kPT;
            if (u < C::UB) {
                const int v = u / C::URB, q = u - v * C::URB;
                const int tok = v / R;
                float e[EPU];
                unpack_unit(raw.bb[j], e, IO());
                if (tok < Tc) {
#pragma unroll
                    for (int pp = 0; pp < EPU / 2; ++pp) {
                        float sn, cs;
                        __sincosf(phi_s[tok * KP + q * (EPU / 2) + pp], &sn, &cs);
                        rot_neg(cs, sn, e[2 * pp], e[2 * pp + 1]);
                    }
                }
                st_unit(bs + v * NBP + q * EPU, e);
                if (C::BST) {
                    const float sc = tok < Tc ? scl_s[tok] : 0.f;
#pragma unroll
                    for (int ee = 0; ee < EPU; ++ee) st_one(bst + (q * EPU + ee) * VP + v, e[ee] * sc);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < C::UPT_X; ++j) {
            const int u = tid + j * kPT;
            if (u < C::UX) {
                const int v = u / C::URX, q = u - v * C::URX;
                float e[EPU];
                unpack_unit(raw.xx[j], e, IO());
#pragma unroll
                for (int ee = 0; ee < EPU; ++ee) st_one(xt + (q * EPU + ee) * VP + v, e[ee]);
            }
        }
        frag cf[C::TBW][NKS];
        if (OUT) {
#pragma unroll
            for (int i = 0; i < C::TBW; ++i) {
                const int tb = wave_block(i, wave);
                const int tok = (16 * tb + l16) / R;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int n0 = 32 * ks + 8 * g;
                    float e[8];
#pragma unroll
                    for (int f = 0; f < C::FU; ++f) unpack_unit(raw.cc[i][ks][f], e + f * EPU, IO());
                    if (tb < C::NTB && n0 < N && tok < Tc) {
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp) {
                            float sn, cs;
                            __sincosf(phi_s[tok * KP + n0 / 2 + pp], &sn, &cs);
                            rot_neg(cs, sn, e[2 * pp], e[2 * pp + 1]);
                        }
                    }
                    cf[i][ks] = M::pack(e);
                }
            }
        }

        // state at the start of this workgroup's first chunk
        if (c == c_begin) {
            const float del0 = misc_s[1];
#pragma unroll
            for (int j = 0; j < C::TW; ++j) {
                const int tile = wave + kPW * j;
                if (tile >= C::NTILE) continue;
                const int nt = tile / PT, pt = tile - nt * PT;
                if (OUT) {
                    if (p.S == 1) {
                        if (p.has_init) st[j] = fold_init<C, IO>(p, bh, nt, pt, del0);
                    } else {
                        const int pc = 16 * pt + l16;
                        if (p.has_init) {
                            const float *hi = p.hinit + bh * int64_t(N) * P;
#pragma unroll
                            for (int v = 0; v < 4; ++v) st[j][v] = hi[(16 * nt + 4 * g + v) * P + pc];
                        }
                        for (int s2 = 0; s2 < seg; ++s2) {
                            const int64_t so = bh * p.S + s2;
                            const float eg = __expf(p.segG[so]);
                            const float *U = p.segU + so * int64_t(N) * P;
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const int k = 8 * nt + 2 * g + q;
                                float sn, cs;
                                sincos_wrapped(wrap_angle(p.segTh[so * K + k]), &sn, &cs);
                                const float a0 = eg * st[j][2 * q], a1 = eg * st[j][2 * q + 1];
                                st[j][2 * q] = cs * a0 - sn * a1 + U[(16 * nt + 4 * g + 2 * q) * P + pc];
                                st[j][2 * q + 1] = sn * a0 + cs * a1 + U[(16 * nt + 4 * g + 2 * q + 1) * P + pc];
                            }
                        }
                    }
                    st_four(ht + (16 * pt + l16) * NBP + 16 * nt + 4 * g, st[j][0], st[j][1], st[j][2], st[j][3]);
                } else if (seg == 0 && p.has_init) {
                    const floatx4 hi4 = fold_init<C, IO>(p, bh, nt, pt, del0);
                    float *hi = p.hinit + bh * int64_t(N) * P;
#pragma unroll
                    for (int v = 0; v < 4; ++v) hi[(16 * nt + 4 * g + v) * P + 16 * pt + l16] = hi4[v];
                }
            }
            if (!OUT && seg == 0 && p.has_init)
                for (int k = tid; k < K; k += kPT) p.phi0ws[bh * K + k] = double(p.phi0[bh * K + k]);
        }

        // prefetch the next chunk while this one computes
        if (c + 1 < c_end) {
            const int64_t t1 = t0 + kQ;
            load_chunk<C, IO, OUT>(p, b, h, t1, int(min<int64_t>(kQ, p.T - t1)), raw);
        }
        __syncthreads();

        const float gc = misc_s[0];
        if (OUT) {
            // ---- a3 + a5: y = M x + exp(ell) Chat H for this wave's row blocks
            IO *ybase = static_cast<IO *>(p.y) + ((b * p.T + t0) * p.H + h) * (R * P);
#pragma unroll
            for (int i = 0; i < C::TBW; ++i) {
                const int tb = wave_block(i, wave);
                if (tb >= C::NTB) continue;
                const int t0v = 16 * tb;
                if (t0v / R >= Tc) continue;
                const int tok_last = min((t0v + 15) / R, Tc - 1);
                floatx4 acc[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int n0 = 32 * ks + 8 * g;
                        const frag hb = n0 < N ? M::lds8(ht + (16 * pt + l16) * NBP + n0) : M::zero();
                        acc[pt] = M::mma(acc[pt], cf[i][ks], hb);
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int tok = (t0v + 4 * g + v) / R;
                    const float e = tok < Tc ? __expf(ell_s[tok]) : 0.f;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[pt][v] *= e;
                }
                const int tt = (t0v + l16) / R; // token of this lane's column t
                const float ell_t = ell_s[tt], gam_t = gam_s[tt];
                const bool live = tt < Tc;
                for (int s0 = 0; s0 / R <= tok_last; s0 += 32) {
                    floatx4 sb[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        sb[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) {
                            const int n0 = 32 * ks + 8 * g;
                            const frag ab = n0 < N ? M::lds8(bs + (s0 + 16 * q + l16) * NBP + n0) : M::zero();
                            sb[q] = M::mma(sb[q], ab, cf[i][ks]);
                        }
                    }
                    float m[8];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        int ts_prev = -1;
                        float w = 0.f;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int ts = (s0 + 16 * q + 4 * g + v) / R;
                            if (ts != ts_prev) {
                                w = 0.f;
                                if (live && ts <= tt) w = ts == tt ? gam_t : __expf(ell_t - ell_s[ts]) * wgt_s[ts];
                                ts_prev = ts;
                            }
                            m[4 * q + v] = sb[q][v] * w;
                        }
                    }
                    const frag mf = M::pack(m);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const lds_t *xr = xt + (16 * pt + l16) * VP + s0 + 4 * g;
                        acc[pt] = M::mma(acc[pt], mf, M::lds4x2(xr, xr + 16));
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int vr = t0v + 4 * g + v;
                    const int tok = vr / R, ch = vr - tok * R;
                    if (tok < Tc) {
                        IO *dst = ybase + ((tok * p.H * R + ch) * P + l16);
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) io<IO>::put(dst + 16 * pt, acc[pt][v]);
                    }
                }
            }
        }

        // ---- a4: H <- R(Theta_c) (exp(g_c) H + sum_v (scaled Bhat)[v] x[v]^T)
        {
            const float eg = __expf(gc);
#pragma unroll
            for (int j = 0; j < C::TW; ++j) {
                const int tile = wave + kPW * j;
                if (tile >= C::NTILE) continue;
                const int nt = tile / PT, pt = tile - nt * PT;
                floatx4 acc = st[j] * eg;
                const lds_t *br = xt + (16 * pt + l16) * VP + 8 * g;
                if (C::BST) {
                    const lds_t *ar = bst + (16 * nt + l16) * VP + 8 * g;
#pragma unroll 2
                    for (int ks = 0; ks < V / 32; ++ks) acc = M::mma(acc, M::lds8(ar + 32 * ks), M::lds8(br + 32 * ks));
                } else {
                    // gather column n of the row-major copy and apply the scale here
                    const lds_t *ac = bs + 16 * nt + l16;
#pragma unroll 1
                    for (int ks = 0; ks < V / 32; ++ks) {
                        float a[8];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            const int v = 32 * ks + 8 * g + jj;
                            a[jj] = lds_to_f32(ac[v * NBP]) * scl_s[v / R];
                        }
                        acc = M::mma(acc, M::pack(a), M::lds8(br + 32 * ks));
                    }
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float2 cs = thc_s[8 * nt + 2 * g + q];
                    st[j][2 * q] = cs.x * acc[2 * q] - cs.y * acc[2 * q + 1];
                    st[j][2 * q + 1] = cs.y * acc[2 * q] + cs.x * acc[2 * q + 1];
                }
            }
        }
        gsum += gc;
        __syncthreads();

        if (OUT) {
#pragma unroll
            for (int j = 0; j < C::TW; ++j) {
                const int tile = wave + kPW * j;
                if (tile >= C::NTILE) continue;
                const int nt = tile / PT, pt = tile - nt * PT;
                st_four(ht + (16 * pt + l16) * NBP + 16 * nt + 4 * g, st[j][0], st[j][1], st[j][2], st[j][3]);
            }
        }
    }

    if (!OUT) {
        // segment aggregate: state from zero, summed log decay and angle
        float *U = p.segU + (bh * p.S + seg) * int64_t(N) * P;
#pragma unroll
        for (int j = 0; j < C::TW; ++j) {
            const int tile = wave + kPW * j;
            if (tile >= C::NTILE) continue;
            const int nt = tile / PT, pt = tile - nt * PT;
#pragma unroll
            for (int v = 0; v < 4; ++v) U[(16 * nt + 4 * g + v) * P + 16 * pt + l16] = st[j][v];
        }
        if (tid == 0) p.segG[bh * p.S + seg] = gsum;
        for (int k = tid; k < K; k += kPT) p.segTh[(bh * p.S + seg) * K + k] = ths_s[k];
        return;
    }
    if (seg != p.S - 1 || !p.has_final) return;

    // final carried state in the rotated frame: h~ = R(-Phi_{T-1}) H
    float *hT = p.hT + bh * int64_t(N) * P;
#pragma unroll
    for (int j = 0; j < C::TW; ++j) {
        const int tile = wave + kPW * j;
        if (tile >= C::NTILE) continue;
        const int nt = tile / PT, pt = tile - nt * PT;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = 8 * nt + 2 * g + q;
            float sn, cs;
            sincos_wrapped(wrap_angle(ths_s[k]), &sn, &cs);
            float u = st[j][2 * q], v = st[j][2 * q + 1];
            rot_neg(cs, sn, u, v);
            hT[(16 * nt + 4 * g + 2 * q) * P + 16 * pt + l16] = u;
            hT[(16 * nt + 4 * g + 2 * q + 1) * P + 16 * pt + l16] = v;
        }
    }
    const int64_t tl = (b * p.T + p.T - 1) * p.H + h; // token-head index of T-1
    for (int k = tid; k < K; k += kPT) p.phiT[bh * K + k] = float(wrap_angle(ths_s[k]));
    for (int i = tid; i < R * K; i += kPT) {
        const int r = i / K, k = i - r * K;
        float sn, cs;
        sincos_wrapped(wrap_angle(ths_s[k]), &sn, &cs);
        const IO *Bl = static_cast<const IO *>(p.B) + (tl * R + r) * N + 2 * k;
        float u = io<IO>::get(Bl), v = io<IO>::get(Bl + 1);
        rot_neg(cs, sn, u, v);
        p.prevBT[(bh * R + r) * N + 2 * k] = u;
        p.prevBT[(bh * R + r) * N + 2 * k + 1] = v;
    }
    const IO *xl = static_cast<const IO *>(p.x) + tl * R * P;
    IO *px = static_cast<IO *>(p.prevxT) + bh * R * P;
    for (int i = tid; i < R * P; i += kPT) px[i] = xl[i];
}

// Host-side launch of one instantiation (pre-pass when OUT is false).
template <typename IO, int N, int P, int R, bool OUT>
hipError_t launch_prefill_inst(const PrefillParams &p, hipStream_t s) {
    typedef Cfg<IO, N, P, R> C;
    const int nseg = OUT ? p.S : p.S - 1;
    if (nseg <= 0) return hipSuccess;
    if (C::bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_prefill<IO, N, P, R, OUT>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(C::bytes));
        if (e != hipSuccess) return e;
    }
    const dim3 grid(unsigned(p.batch * p.H * nseg)), block(kPT);
    hipLaunchKernelGGL((k_prefill<IO, N, P, R, OUT>), grid, block, C::bytes, s, p);
    return hipGetLastError();
}

} // namespace m3
