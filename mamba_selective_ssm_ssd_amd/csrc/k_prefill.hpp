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
//  a1  cumsum: ell_t = sum_{t0<=u<=t} dt_u A (wave scan, lane = token),
//      gam_t = lam_t dt_t, wgt_t = gam_t + delta_{t+1}, delta = (1-lam) dt,
//      g_c = ell at the last token; angle prefix phi_t,k = sum theta (fp64
//      wave scans, wrapped to [-pi, pi)) turned into a cos/sin table, and
//      the chunk total Theta_c,k.
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
// Schedule: one workgroup of 512 threads (8 waves), two barriers per chunk.
// While chunk c computes, the next chunk's B, x, C sit in registers (loaded
// during c's staging) and the a1 prologue of chunk c+1 (wave-local DPP scans,
// no barrier of its own) fills the cos/sin table and the second half of the
// double-buffered coefficient tables.  LDS holds the rotated B, x and the
// scaled x row-major (16-byte stores, no transposed writes), the state H
// (transposed), and the tables; operands whose contraction index is the LDS
// row (x for M x, Bhat and scaled x for the state update) are read with the
// transposing LDS load.  The rotated C of a wave's 16-row blocks stays in
// registers.  bf16 I/O stages one bf16 plane per value, fp32 I/O two (hi, lo).
#pragma once

#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

constexpr int kPT = 512;         // threads per prefill workgroup
constexpr int kPW = kPT / kWave; // waves per prefill workgroup

constexpr size_t align16(size_t v) { return (v + 15) / 16 * 16; }

// Row pitch (bf16 elements) of an LDS table with n columns: padded to an odd
// multiple of 16 elements (row pitch = 8 mod 16 banks), where the row-operand,
// transposing and mask reads of this kernel are free of bank conflicts, or
// (narrow layout) by 8 elements only.
constexpr int lds_pitch(int n, bool wide) { return wide ? (n + 31) / 32 * 32 + 16 : n + 8; }

template <typename IO, int N_, int P_, int R_, int Q_, bool WIDE, bool BLK, bool BPAD = false>
struct CfgW {
    // Q tokens per chunk, V = Q R virtual rows (token, rank) per chunk
    static constexpr int N = N_, P = P_, R = R_, Q = Q_, K = N / 2, V = Q * R;
    static constexpr bool kWide = WIDE;
    // (BLK) the block prologue's weight/bias table [4][R][N] floats sits in
    // its own region, or (BPAD) one float4 per staged-B row in that row's
    // padding columns (never read or written by the staging and the products)
    static constexpr bool kBpad = BPAD;
    static constexpr int PL = mode<IO>::f32 ? 2 : 1;          // bf16 planes per staged value
    typedef Mma<PL> M;
    typedef typename M::frag frag;
    static constexpr int SZ = int(sizeof(IO));
    static constexpr int EPU = 16 / SZ;                       // I/O elements per 16-byte unit
    static constexpr int NBP = lds_pitch(N, WIDE);            // row pitch of bs, ht, cl (elements)
    static constexpr int PP = lds_pitch(P, WIDE);             // row pitch of xr, xs (elements)
    static constexpr int CSP = 2 * K + 4;                     // row pitch of the cos/sin table (floats)
    static constexpr int NTB = V / 16;                        // 16-row blocks of virtual rows
    static constexpr int TBW = NTB > kPW ? 2 : 1;             // blocks per wave
    static constexpr int NKS = N >= 32 ? N / 32 : 1;          // K-steps of 32 over N
    static constexpr int NT = N / 16, PT = P / 16, NTILE = NT * PT;
    static constexpr int TW = (NTILE + kPW - 1) / kPW;        // state tiles per wave
    // 16-byte units of one chunk's B and x, and units per thread
    static constexpr int URB = N * SZ / 16, UB = V * URB, UPT_B = (UB + kPT - 1) / kPT;
    static constexpr int URX = P * SZ / 16, UX = V * URX, UPT_X = (UX + kPT - 1) / kPT;
    static constexpr int FU = 8 / EPU; // units per MFMA fragment (8 elements)
    // prologue: the angle prefix is scanned per group of 8 pairs by one wave
    // (lane = token); GU 16-byte units hold a group of one token
    static constexpr int NG8 = K / 8, GU = 8 / EPU;
    // Angle groups go to the waves that own no intra-chunk row block when
    // there are such waves (R = 1), GPW groups each; otherwise wave w takes
    // group kPW - 1 - w.
    static constexpr int FREEW = NTB < kPW ? kPW - NTB : 0;
    static constexpr int GPW = FREEW ? (NG8 + FREEW - 1) / FREEW : 1;
    // the wave that scans the decay coefficients: the first wave without
    // intra-chunk row blocks when there is one (waves w and w + 4 share a
    // SIMD, and wave w's row block w is the lightest for w = 0)
    static constexpr int CW = FREEW ? NTB : 0;
    // plane strides (elements) of the staged arrays
    static constexpr int BS_PS = V * NBP, X_PS = V * PP, HT_PS = P * NBP;
    // LDS layout, bytes.  The MFMA operands come first so that their offsets
    // fit the LDS instructions' immediate field.  The cos/sin table is written
    // by the prologue of chunk c+1 after chunk c's staging has read it; the
    // coefficient and chunk-rotation tables are read while the next prologue
    // runs, so they are double-buffered.
    static constexpr size_t o_bs = 0;                                          // [PL][V][NBP]
    static constexpr size_t o_xr = o_bs + size_t(PL) * BS_PS * 2;              // [PL][V][PP]
    static constexpr size_t o_ht = o_xr + size_t(PL) * X_PS * 2;               // [PL][P][NBP]
    static constexpr size_t o_cs = o_ht + size_t(PL) * HT_PS * 2;              // float [Q][CSP]
    static constexpr size_t o_coef = o_cs + size_t(Q) * CSP * 4;               // [2][4][64]: ell, gam, wgt, scl (lane = token)
    static constexpr size_t o_misc = o_coef + 2 * 4 * kWave * 4;                  // [2] g_c, [2] delta_0
    static constexpr size_t o_thc = o_misc + 64;                               // float2 [2][K]: cos, sin Theta_c
    static constexpr size_t o_ths = o_thc + 2 * size_t(K) * 8;                 // double [K]: running angle
    // The chunk's token mask L[t][s] (and e^{ell_t}) is tabulated once per
    // chunk when it fits; otherwise each lane evaluates its mask entries.
    static constexpr int LWP = WIDE ? Q + 8 : Q + 4;                           // row pitch (floats)
    // block prologue tables (BLK): B weight, B bias, C weight, C bias [R][N]
    static constexpr size_t o_blk = align16(o_ths + size_t(K) * 8);
    static constexpr size_t blk_bytes = BLK && !BPAD ? 16 * size_t(R) * N : 0;
    static constexpr size_t o_lw = align16(o_blk + blk_bytes);                 // float [Q][LWP]
    static constexpr size_t lw_bytes = size_t(Q) * LWP * 4 + Q * 4;            // + e^{ell} [Q]
    static constexpr bool LWT = o_lw + lw_bytes <= kMaxLdsBytes;
    // bf16 I/O: the within-chunk angle prefix is the matrix product of the
    // lower-triangular ones matrix with the chunk's theta (MFMA, fp32
    // accumulation), read from a row-major theta table; otherwise (fp32 I/O,
    // or fewer than 16 pairs) exact fixed-point DPP scans.
    // The table has at least 32 rows (one k-step of the product); rows past
    // the chunk's last token repeat that token (finite values that meet zero
    // entries of the ones matrix).
    static constexpr int THP = lds_pitch(K, WIDE);                             // theta table pitch (elements)
    static constexpr int QTH = Q < 32 ? 32 : Q;                                // theta table rows
    static constexpr int URT = K * SZ / 16, UT = QTH * URT, UPT_T = (UT + kPT - 1) / kPT;
    static constexpr int TB = Q / 16;                                          // 16-token blocks per chunk
    static constexpr int NPB = K / 16, NTT = TB * NPB;                         // 16x16 prefix tiles
    static constexpr size_t o_th = align16(o_lw + (LWT ? lw_bytes : 0));       // bf16 [QTH][THP]
    static constexpr size_t th_bytes = size_t(QTH) * THP * 2;
    static constexpr bool MFP = PL == 1 && K % 16 == 0 && o_th + th_bytes <= kMaxLdsBytes;
    static constexpr int MFW = FREEW ? FREEW : kPW;                            // waves sharing the prefix tiles
    static constexpr int TPW = MFP ? (NTT + MFW - 1) / MFW : 0;
    static constexpr size_t o_xs = align16(o_th + (MFP ? th_bytes : 0));       // [PL][V][PP] scaled x
    static constexpr size_t xs_bytes = size_t(PL) * X_PS * 2;
    // The scaled copy of x (the state update's second operand) is kept when
    // it fits; otherwise the scale is applied to that operand's fragments.
    static constexpr bool XS = o_xs + xs_bytes <= kMaxLdsBytes;
    // When some waves own no intra-chunk row block, the rotated C is staged in
    // LDS by all waves (as B is) instead of by the row-block waves into their
    // registers, when it fits; the row-block waves then read their fragments.
    static constexpr size_t o_cl = align16(o_xs + (XS ? xs_bytes : 0));       // [PL][V][NBP] rotated C
    static constexpr size_t cl_bytes = size_t(PL) * BS_PS * 2;
    static constexpr bool CL = FREEW > 0 && o_cl + cl_bytes <= kMaxLdsBytes;
    static constexpr size_t bytes = o_cl + (CL ? cl_bytes : 0);
    static_assert(K * SZ % 16 == 0 && N % 16 == 0 && P % 16 == 0 && K % 8 == 0, "tile sizes");
    static_assert(Q % 16 == 0 && Q <= kQ && V % 32 == 0 && V <= 2 * 16 * kPW, "chunk rows");
    static_assert(FREEW ? NG8 <= FREEW * GPW : NG8 <= kPW, "angle groups per wave");
    static_assert(!BPAD || (BLK && V >= R * N && (NBP - N) * 2 >= 16), "block table in the B row padding");
};

// The wide (conflict-free) layout when it fits with every optional table the
// narrow one has, else the narrow layout.
template <typename IO, int N, int P, int R, int Q, bool BLK>
struct CfgPick {
    typedef CfgW<IO, N, P, R, Q, true, BLK> Wd;
    typedef CfgW<IO, N, P, R, Q, false, BLK> Nw;
    static constexpr bool wide = Wd::bytes <= kMaxLdsBytes && Wd::LWT == Nw::LWT && Wd::MFP == Nw::MFP &&
                                 Wd::XS == Nw::XS && Wd::CL == Nw::CL;
    typedef typename std::conditional<wide, Wd, Nw>::type type;
};
// With the block prologue the layout is the plain one whenever the table fits
// in the staged-B row padding (N <= 64: one 16-byte slot per row), so the
// block variant keeps every optional table of the plain kernel.
template <typename IO, int N, int P, int R, int Q, bool BLK>
struct CfgSel {
    typedef typename CfgPick<IO, N, P, R, Q, false>::type Plain;
    static constexpr bool pad = BLK && N <= Q;
    typedef typename std::conditional<pad, CfgW<IO, N, P, R, Q, Plain::kWide, true, true>,
                                      typename CfgPick<IO, N, P, R, Q, BLK>::type>::type type;
};
template <typename IO, int N, int P, int R, int Q, bool BLK = false>
using Cfg = typename CfgSel<IO, N, P, R, Q, BLK>::type;

// (BLK) entries of the block table at float offset o (a multiple of 4 for
// the float4 read)
template <class C>
__device__ __forceinline__ const float *blk_row(const unsigned char *smem, int o) {
    if constexpr (C::kBpad)
        return reinterpret_cast<const float *>(smem + C::o_bs + size_t(o >> 2) * (C::NBP * 2) + C::N * 2) + (o & 3);
    else
        return reinterpret_cast<const float *>(smem + C::o_blk) + o;
}
template <class C>
__device__ __forceinline__ float4 blk_tbl4(const unsigned char *smem, int o) {
    return *reinterpret_cast<const float4 *>(blk_row<C>(smem, o));
}

// Raw (undecoded) B, x and C of one chunk held in registers.
template <class C>
struct RawChunk {
    uint4 bb[C::UPT_B], xx[C::UPT_X];
    uint4 cc[C::CL ? 1 : C::TBW][C::CL ? 1 : C::NKS][C::CL ? 1 : C::FU]; // C of this wave's row blocks
    uint4 cu[C::CL ? C::UPT_B : 1];                                       // C units, spread as B's (CL)
};

// Raw prologue inputs of one chunk: a group of 8 rotation angles of this
// lane's token (angle waves) or dt, lam of this lane's token (wave 0).
template <class C>
struct RawPro {
    uint4 th[C::MFP ? 1 : C::GPW][C::GU];  // DPP scans: this wave's angle groups of its lane's token
    uint4 thu[C::MFP ? C::UPT_T : 1];      // MFMA prefix: this thread's units of the theta rows
    uint32_t dt, lam, dtn, lamn;           // raw I/O bits of dt, lam (this lane's token, token t0+Q)
};

// Prefix tile m (< TPW) computed by a wave, or -1.  Tile t covers token block
// t % TB and pair block t / TB.  With free waves each takes TPW consecutive
// tiles (the token blocks of one pair block when TPW = TB = 4: one operand
// read serves all four, and every wave gets one chunk-end row).
template <class C>
__device__ __forceinline__ int mfp_tile(int wave, int m) {
    int t;
    if (C::FREEW) t = wave >= C::NTB ? (wave - C::NTB) * C::TPW + m : -1;
    else t = wave + m * kPW;
    return t >= 0 && t < C::NTT ? t : -1;
}

// Angle group m (< GPW) scanned by a wave, or -1.
template <class C>
__device__ __forceinline__ int pro_group(int wave, int m) {
    int grp;
    if (C::FREEW) grp = wave >= C::NTB ? wave - C::NTB + m * C::FREEW : -1;
    else grp = m == 0 ? kPW - 1 - wave : -1;
    return grp >= 0 && grp < C::NG8 ? grp : -1;
}

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
// Sum of squares of a 16-byte unit's elements, read from the raw bits (bf16:
// one v_dot2 per pair, so no unpacked copy of the unit is kept for it).
__device__ __forceinline__ float unit_sumsq(const uint4 &u, bf16) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    float s = 0.f;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf2 v = __builtin_bit_cast(bf2, w[i]);
        s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
    }
    return s;
}
__device__ __forceinline__ float unit_sumsq(const uint4 &u, float) {
    const float a = __uint_as_float(u.x), b = __uint_as_float(u.y);
    const float c = __uint_as_float(u.z), d = __uint_as_float(u.w);
    return a * a + b * b + c * c + d * d;
}

// Virtual-row block i (< TBW) of a wave: blocks w and 2*kPW-1-w, so that the
// causal work of the two blocks balances across waves.
__device__ __forceinline__ int wave_block(int i, int wave) { return i == 0 ? wave : 2 * kPW - 1 - wave; }

// f(integral_constant<J>) for J = J0 .. NJ-1, unrolled at compile time.
template <int J0, int NJ, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (J0 < NJ) {
        f(std::integral_constant<int, J0>{});
        static_for<J0 + 1, NJ>(f);
    }
}

// Loads chunk (b, h, t0 .. t0+Tc-1)'s B, x and C into registers.  Addresses
// are a uniform per-chunk base plus a 32-bit per-thread offset (saddr +
// voffset addressing).  Every load is issued (indices clamped to the last
// unit and the last token): a token past Tc repeats token Tc-1, whose finite
// values meet only zero mask entries, zero state-update scales and outputs
// that are not stored.  With no load under a condition the compiler's wait
// counts stay exact.
// PARTS selects what is loaded: bit 0 B, bit 1 x, bit 2 C; J >= 0 loads only
// unit J of B, x and the spread C units.
template <class C, typename IO, bool OUT, int PARTS = 7, int J = -1>
__device__ __forceinline__ void load_chunk(const PrefillParams &p, int64_t b, int h, int hg, int64_t t0, int Tc,
                                           RawChunk<C> &r) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t tokbase = (b * p.T + t0) * p.H + h;  // token-head index of t0
    const int64_t tokgrp = (b * p.T + t0) * p.G + hg;  // token-group index of t0 (B, C)
    const int H = p.H, G = p.G;
    const IO *Bp = static_cast<const IO *>(p.B) + tokgrp * (C::R * C::N);
    const IO *Xp = static_cast<const IO *>(p.x) + tokbase * (C::R * C::P);
    const IO *Cp = static_cast<const IO *>(p.C) + tokgrp * (C::R * C::N);
#pragma unroll
    for (int j = 0; j < ((PARTS & 1) ? C::UPT_B : 0); ++j) {
        if (J >= 0 && j != J) continue;
        const int u = min(tid + j * kPT, C::UB - 1);
        const int v = u / C::URB, q = u - v * C::URB;
        const int tok = min(v / C::R, Tc - 1), ch = v % C::R;
        r.bb[j] = ld16(Bp + ((tok * G * C::R + ch) * C::N + q * C::EPU));
    }
#pragma unroll
    for (int j = 0; j < ((PARTS & 2) ? C::UPT_X : 0); ++j) {
        if (J >= 0 && j != J) continue;
        const int u = min(tid + j * kPT, C::UX - 1);
        const int v = u / C::URX, q = u - v * C::URX;
        const int tok = min(v / C::R, Tc - 1), ch = v % C::R;
        r.xx[j] = ld16(Xp + ((tok * H * C::R + ch) * C::P + q * C::EPU));
    }
    if constexpr (OUT && (PARTS & 4) && C::CL) {
#pragma unroll
        for (int j = 0; j < C::UPT_B; ++j) {
            if (J >= 0 && j != J) continue;
            const int u = min(tid + j * kPT, C::UB - 1);
            const int v = u / C::URB, q = u - v * C::URB;
            const int tok = min(v / C::R, Tc - 1), ch = v % C::R;
            r.cu[j] = ld16(Cp + ((tok * G * C::R + ch) * C::N + q * C::EPU));
        }
    } else if (OUT && (PARTS & 4)) {
#pragma unroll
        for (int i = 0; i < C::TBW; ++i) {
            // a wave without this row block loads the last block's rows (unused)
            const int tb = min(wave_block(i, wave), C::NTB - 1);
            const int v = 16 * tb + l16;
            const int tok = min(v / C::R, Tc - 1), ch = v % C::R;
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                const int n0 = min(32 * ks + 8 * g, C::N - 8);
#pragma unroll
                for (int f = 0; f < C::FU; ++f)
                    r.cc[i][ks][f] = ld16(Cp + ((tok * G * C::R + ch) * C::N + n0 + f * C::EPU));
            }
        }
    }
}

// Loads the prologue inputs of chunk (b, h, t0 .. t0+Tc-1): the angle groups
// of this wave for its lane's token; wave 0 loads dt and lam of its lane's
// token (and of token t0+64).
template <class C, typename IO>
__device__ __forceinline__ void load_pro(const PrefillParams &p, int64_t b, int h, int64_t t0, int Tc,
                                         RawPro<C> &r) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t tokbase = (b * p.T + t0) * p.H + h;
    const int H = p.H;
    const IO *th = static_cast<const IO *>(p.theta) + tokbase * C::K;
    if constexpr (!C::MFP) {
#pragma unroll
        for (int m = 0; m < C::GPW; ++m) {
            const int grp = pro_group<C>(wave, m);
#pragma unroll
            for (int f = 0; f < C::GU; ++f) {
                r.th[m][f] = make_uint4(0u, 0u, 0u, 0u);
                if (grp >= 0 && lane < Tc)
                    r.th[m][f] = ld16(th + (lane * H * C::K + 8 * grp + f * C::EPU));
            }
        }
    }
    r.dt = r.lam = r.dtn = r.lamn = 0u;
    if (wave == C::CW) {
        // token past Tc: repeats token Tc-1; next chunk's first token: clamped
        // to the last token (its delta is not used when t0 + 64 >= T)
        const IO *dt = static_cast<const IO *>(p.dt) + tokbase;
        const IO *lam = static_cast<const IO *>(p.lam) + tokbase;
        const int lt = min(lane, Tc - 1);
        const int64_t tn = min<int64_t>(C::Q, p.T - 1 - t0);
        r.dt = io<IO>::raw(dt + lt * H);
        r.lam = io<IO>::raw(lam + lt * H);
        r.dtn = io<IO>::raw(dt + tn * H);
        r.lamn = io<IO>::raw(lam + tn * H);
    }
}

// Loads the theta rows of chunk (b, h, t0 .. t0+Tc-1), spread over all
// threads (MFMA prefix only; issued a chunk ahead of their use).
template <class C, typename IO>
__device__ __forceinline__ void load_theta(const PrefillParams &p, int64_t b, int h, int64_t t0, int Tc,
                                           RawPro<C> &r) {
    if constexpr (C::MFP) {
        const IO *th = static_cast<const IO *>(p.theta) + ((b * p.T + t0) * p.H + h) * C::K;
        const int H = p.H;
#pragma unroll
        for (int j = 0; j < C::UPT_T; ++j) {
            const int u = threadIdx.x + j * kPT;
            const int uc = u < C::UT ? u : C::UT - 1;
            const int tr = uc / C::URT, q = uc - tr * C::URT;
            const int tok = tr < Tc ? tr : Tc - 1; // a row past Tc repeats row Tc-1
            r.thu[j] = ld16(th + (tok * H * C::K + q * C::EPU));
        }
    }
}

// Stores the raw theta rows of the next chunk as a row-major bf16 table
// (MFMA prefix only).
template <class C>
__device__ __forceinline__ void write_theta(const RawPro<C> &r, uint16_t *tht) {
    if constexpr (C::MFP) {
#pragma unroll
        for (int j = 0; j < C::UPT_T; ++j) {
            const int u = threadIdx.x + j * kPT;
            const int tok = u / C::URT, q = u - tok * C::URT;
            if (u < C::UT) *reinterpret_cast<uint4 *>(tht + tok * C::THP + q * 8) = r.thu[j];
        }
    }
}

// a1 angles of one chunk: the cos/sin table of the within-chunk angle prefix
// (row = token, (cos, sin) per pair), the chunk rotation (cos, sin of
// Theta_c, the table's row Tc-1) into one half of the double-buffered table,
// and the running fp64 angle.  bf16 I/O: MFMA prefix over the theta table;
// otherwise exact integer scans of fixed-point turns (DPP, lane = token) of
// this wave's angle groups held in registers.  Sin and cos take turns.
template <class C, typename IO>
__device__ __forceinline__ void run_angles(const RawPro<C> &r, int Tc, float *cs, float2 *thc, double *ths,
                                           const uint16_t *tht) {
    constexpr int EPU = C::EPU;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if constexpr (C::MFP) {
        // Phi[t][k] = sum_{s <= t} theta[s][k] as (lower-triangular ones) x theta,
        // one 16x16 tile (16 tokens x 16 pairs) per step; the chunk total is
        // the row of token Tc-1.  Every tile takes both 32-token k-steps (the
        // ones matrix is zero beyond the tile's last token), so a wave issues
        // all its operand reads, then all its products, then the sin/cos.
        typedef typename C::M M;
        const int g = lane >> 4, l16 = lane & 15;
        if (mfp_tile<C>(wave, 0) < 0) return;
        constexpr int KB = C::QTH / 32;
        typename M::frag bf[C::TPW][KB];
        int tbm[C::TPW], pbm[C::TPW];
#pragma unroll
        for (int m = 0; m < C::TPW; ++m) {
            const int tile = mfp_tile<C>(wave, m);
            const int tl = tile < 0 ? 0 : tile;
            tbm[m] = tl % C::TB;
            pbm[m] = tl / C::TB;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                // slots 0-3: tokens 32 kb + 4 g .. +3, slots 4-7: 16 tokens further
                const uint16_t *bp = tht + (32 * kb + 4 * g + (l16 >> 2)) * C::THP + 16 * pbm[m] + 4 * (l16 & 3);
                bf[m][kb] = M::template tr8<0>(bp, bp + 16 * C::THP);
            }
        }
        floatx4 acc[C::TPW];
#pragma unroll
        for (int m = 0; m < C::TPW; ++m) {
            const int trow = 16 * tbm[m] + l16; // A row of this lane
            acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s0 = 32 * kb + (i < 2 ? 4 * g + 2 * i : 16 + 4 * g + 2 * (i - 2)); // token of slot 2 i
                    w[i] = (s0 <= trow ? 0x3F80u : 0u) | (s0 + 1 <= trow ? 0x3F800000u : 0u);
                }
                typename M::frag a;
                a.v[0] = bf16x8_from_words(w[0], w[1], w[2], w[3]);
                acc[m] = M::mma(acc[m], a, bf[m][kb]);
            }
        }
#pragma unroll
        for (int m = 0; m < C::TPW; ++m) {
            if (mfp_tile<C>(wave, m) < 0) continue;
            const int pair = 16 * pbm[m] + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 16 * tbm[m] + 4 * g + v;
                float tf = acc[m][v] * float(1.0 / kTwoPi);
                tf -= rintf(tf);
                const float sn = __builtin_amdgcn_sinf(tf), cn = __builtin_amdgcn_cosf(tf);
                *reinterpret_cast<float2 *>(cs + t * C::CSP + 2 * pair) = make_float2(cn, sn);
            }
        }
        // the chunk total: row Tc-1, held by lane group ge of the tile of
        // token block te (element ve of the lane's four rows)
        const int te = (Tc - 1) >> 4, ge = ((Tc - 1) & 15) >> 2, ve = (Tc - 1) & 3;
#pragma unroll
        for (int m = 0; m < C::TPW; ++m) {
            if (mfp_tile<C>(wave, m) < 0 || tbm[m] != te) continue; // uniform
            if (g == ge) {
                const float a = ve == 0 ? acc[m][0] : ve == 1 ? acc[m][1] : ve == 2 ? acc[m][2] : acc[m][3];
                float tf = a * float(1.0 / kTwoPi);
                tf -= rintf(tf);
                const int pair = 16 * pbm[m] + l16;
                thc[pair] = make_float2(__builtin_amdgcn_cosf(tf), __builtin_amdgcn_sinf(tf));
                ths[pair] += double(a);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < (C::MFP ? 0 : C::GPW); ++m) {
        const int grp = pro_group<C>(wave, m);
        if (grp < 0) continue;
        float th[8];
#pragma unroll
        for (int f = 0; f < C::GU; ++f) unpack_unit(r.th[m][f], th + f * EPU, IO());
        uint32_t u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = wave_scan_dpp(angle_to_turns32(th[j]));
        float cn[8], sn[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float tf = turns32_to_f32(u[j]);
            sn[j] = __builtin_amdgcn_sinf(tf);
            cn[j] = __builtin_amdgcn_cosf(tf);
        }
        float4 *row = reinterpret_cast<float4 *>(cs + lane * C::CSP + 16 * grp);
        if (C::Q == kWave || lane < C::Q) { // the table has a row per token of the chunk
#pragma unroll
            for (int j = 0; j < 4; ++j) row[j] = make_float4(cn[2 * j], sn[2 * j], cn[2 * j + 1], sn[2 * j + 1]);
        }
        if (lane == Tc - 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                thc[8 * grp + j] = make_float2(cn[j], sn[j]);
                ths[8 * grp + j] += turns32_to_rad(u[j]);
            }
        }
    }
}

// a1 coefficients of one chunk (the coefficient wave): the decay prefix ell,
// gam, wgt = gam + delta of the next token, the chunk-end scale exp(g - ell) wgt,
// g_c and delta of the first token, into one half of the double-buffered
// tables.  Wave-local DPP scan; the next token's delta by a DPP wave shift.
template <class C, typename IO>
__device__ __forceinline__ void run_coef(const RawPro<C> &r, int Tc, int64_t t0, int64_t T, float A,
                                         float *coef, float *misc) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (wave == C::CW) {
        const float dtv = io<IO>::value(r.dt), lamv = io<IO>::value(r.lam);
        const float ell = wave_scan_dpp(dtv * A);
        const float gam = lamv * dtv, del = (1.f - lamv) * dtv;
        // delta of the next token: DPP wave shift left by one lane
        float dn = __uint_as_float(dpp_u32<0x130, 0xf, true>(__float_as_uint(del)));
        if (lane == C::Q - 1) dn = (1.f - io<IO>::value(r.lamn)) * io<IO>::value(r.dtn);
        if (t0 + lane + 1 >= T) dn = 0.f;
        const float w = gam + dn;
        const float gc = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ell), Tc - 1));
        coef[lane] = ell;
        coef[kWave + lane] = gam;
        coef[2 * kWave + lane] = w;
        coef[3 * kWave + lane] = lane < Tc ? __expf(gc - ell) * w : 0.f;
        if (lane == 0) {
            misc[0] = gc;
            misc[2] = del;
        }
    }
}

// Block prologue (Mamba-3 review, section 3.4: BC normalisation, B/C biases)
// on NV consecutive channels of one B or C row: e <- e * inv * w + bias, with
// w, bias the row's [N] weight and bias at those channels (block table
// offsets ow, ob) and inv the row's 1 / sqrt(mean_n e^2 + eps) (1 without
// the normalisation).
template <class C, int NV>
__device__ __forceinline__ void block_unit(float *e, float inv, const unsigned char *smem, int ow, int ob) {
#pragma unroll
    for (int i = 0; i < NV; i += 4) {
        const float4 a = blk_tbl4<C>(smem, ow + i);
        const float4 c = blk_tbl4<C>(smem, ob + i);
        e[i] = e[i] * inv * a.x + c.x;
        e[i + 1] = e[i + 1] * inv * a.y + c.y;
        e[i + 2] = e[i + 2] * inv * a.z + c.z;
        e[i + 3] = e[i + 3] * inv * a.w + c.w;
    }
}

// State entering the sequence, as one 16x16 tile of this lane (rows
// n = 16 nt + 4 g + v, column 16 pt + l16), in the state's own frame at the
// sequence start: R(Phi_{-1}) (h~ + delta_0 B~_prev x_prev^T).
template <class C, typename IO>
__device__ __forceinline__ floatx4 fold_init(const PrefillParams &p, int64_t bh, int nt, int pt, float del0) {
    const int lane = threadIdx.x & (kWave - 1), g = lane >> 4, l16 = lane & 15;
    const int pc = 16 * pt + l16;
    const int64_t h0b = bh * int64_t(C::N) * C::P;
    const float *pb = p.prevB0 + bh * int64_t(C::R) * C::N;
    const IO *px = static_cast<const IO *>(p.prevx0) + bh * int64_t(C::R) * C::P;
    float a[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int n = 16 * nt + 4 * g + v;
        float s = p.sbf16 ? bits_to_f32(static_cast<const uint16_t *>(p.h0)[h0b + n * C::P + pc])
                          : static_cast<const float *>(p.h0)[h0b + n * C::P + pc];
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

template <typename IO, int N, int P, int R, int QC, bool OUT, bool BLK>
__global__ __launch_bounds__(kPT) void k_prefill(const PrefillParams p) {
    typedef Cfg<IO, N, P, R, QC, BLK> C;
    typedef typename C::M M;
    typedef typename C::frag frag;
    constexpr int PL = C::PL, K = C::K, V = C::V, NBP = C::NBP, PP = C::PP, EPU = C::EPU;
    constexpr int PT = C::PT, NKS = C::NKS;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, l16 = lane & 15;
    // bf16 I/O with a wave free of intra-chunk rows: that wave scans the next
    // chunk's coefficients in the second phase instead of the first
    constexpr bool CP2 = C::MFP && C::FREEW > 0;
    // the pre-pass has no intra-chunk product, so it stages B~ already scaled
    // by the chunk-end factors (a multiply per value while the row is in
    // registers) and takes x as it is, instead of a scaled copy of x
    constexpr bool BSC = !OUT;

    // workgroup -> (b, h, segment); consecutive indices li land on the same
    // XCD.  Output pass: S segments per sequence, li = bh S + seg (the few
    // segments of a head, and neighbouring heads, share an XCD).  Pre-pass:
    // the first S - 1 segments, each cut into kpre pieces (aggregates indexed
    // by piece), li = piece (b H) + bh, so that the workgroups running at
    // once on an XCD are neighbouring heads at the same tokens: the per-token
    // rows of dt, lam and theta (a few bytes per head) then share cache lines
    // instead of each pulling its own.
    const int nseg = OUT ? p.S : (p.S - 1) * p.kpre;
    const int64_t nbh = p.batch * p.H;
    const int64_t total = nbh * nseg;
    int64_t li = blockIdx.x;
    if (total % 8 == 0) li = int64_t(blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
    const int seg = OUT ? int(li % nseg) : int(li / nbh);
    const int64_t bh = OUT ? li / nseg : li % nbh;
    const int h = int(bh % p.H);
    const int hg = h / p.hpg; // B/C group of the head
    const int64_t b = bh / p.H;
    const int c_begin = seg * p.cps;
    const int c_end = min(p.nC, c_begin + p.cps);

    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *bs = reinterpret_cast<uint16_t *>(smem + C::o_bs);   // rotated B, row-major
    uint16_t *xr = reinterpret_cast<uint16_t *>(smem + C::o_xr);   // x, row-major
    uint16_t *ht = reinterpret_cast<uint16_t *>(smem + C::o_ht);   // state, [p][n]
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem + C::o_xs);   // scaled x, row-major (XS)
    uint16_t *cl = reinterpret_cast<uint16_t *>(smem + C::o_cl);   // rotated C, row-major (CL)
    float *cs_s = reinterpret_cast<float *>(smem + C::o_cs);       // [64][CSP]
    float *coef_s = reinterpret_cast<float *>(smem + C::o_coef);   // [2][4][64]
    float *misc_s = reinterpret_cast<float *>(smem + C::o_misc);   // g_c [2], delta_0 [2]
    float2 *thc_s = reinterpret_cast<float2 *>(smem + C::o_thc);   // [2][K]
    double *ths_s = reinterpret_cast<double *>(smem + C::o_ths);   // [K]
    float *lw_s = reinterpret_cast<float *>(smem + C::o_lw);       // [64][LWP] mask, then e^{ell} [64]
    uint16_t *tht = reinterpret_cast<uint16_t *>(smem + C::o_th);  // theta rows of the next chunk

    // running angle: Phi_{-1} plus the segments before this one (output pass)
    for (int k = tid; k < K; k += kPT) {
        double a = 0.0;
        if (OUT && p.has_init) a = p.S == 1 ? double(p.phi0[bh * K + k]) : p.phi0ws[bh * K + k];
        if (OUT)
            for (int s2 = 0; s2 < seg * p.kpre; ++s2) a += p.segTh[(bh * p.NA + s2) * K + k];
        ths_s[k] = a;
    }

    floatx4 st[C::TW];
#pragma unroll
    for (int j = 0; j < C::TW; ++j) st[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    float gsum = 0.f;
    const float Ah = p.A[h];
    constexpr int Q = C::Q;
    auto tc_of = [&](int c) { return int(min<int64_t>(Q, p.T - int64_t(c) * Q)); };

    // prologue of the first chunk, then its B, x, C and the next prologue inputs
    RawPro<C> rp;
    load_pro<C, IO>(p, b, h, int64_t(c_begin) * Q, tc_of(c_begin), rp);
    load_theta<C, IO>(p, b, h, int64_t(c_begin) * Q, tc_of(c_begin), rp);
    RawChunk<C> raw;
    load_chunk<C, IO, OUT>(p, b, h, hg, int64_t(c_begin) * Q, tc_of(c_begin), raw);
    write_theta<C>(rp, tht);
    run_coef<C, IO>(rp, tc_of(c_begin), int64_t(c_begin) * Q, p.T, Ah, coef_s, misc_s);
    if constexpr (BLK) {
        // this head's block prologue weights and biases (1 and 0 when absent)
        const int64_t hb0 = int64_t(h) * R * N;
        constexpr int F4 = R * N / 4; // float4 entries per array
        for (int f = tid; f < 4 * F4; f += kPT) {
            const int a = f / F4, i = 4 * (f - a * F4);
            const float *src = a == 0 ? p.blk.bw : a == 1 ? p.blk.bb : a == 2 ? p.blk.cw : p.blk.cb;
            const float dflt = (a & 1) ? 0.f : 1.f;
            const float4 v = src ? *reinterpret_cast<const float4 *>(src + hb0 + i) : make_float4(dflt, dflt, dflt, dflt);
            *reinterpret_cast<float4 *>(const_cast<float *>(blk_row<C>(smem, 4 * f))) = v;
        }
    }
    __syncthreads(); // ths_s, theta table, block tables
    run_angles<C, IO>(rp, tc_of(c_begin), cs_s, thc_s, ths_s, tht);
    if (c_begin + 1 < c_end) {
        load_pro<C, IO>(p, b, h, int64_t(c_begin + 1) * Q, tc_of(c_begin + 1), rp);
        load_theta<C, IO>(p, b, h, int64_t(c_begin + 1) * Q, tc_of(c_begin + 1), rp);
    }
    __syncthreads();
    // state at the start of this workgroup's first chunk (before the chunk loop,
    // so that none of its loads is pending inside it)
    {
        const float del0 = misc_s[2];
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
                    for (int s2 = 0; s2 < seg * p.kpre; ++s2) {
                        const int64_t so = bh * p.NA + s2;
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
                const float sv[4] = {st[j][0], st[j][1], st[j][2], st[j][3]};
                st_planes<PL, C::HT_PS, 4>(ht + (16 * pt + l16) * NBP + 16 * nt + 4 * g, sv);
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

    for (int c = c_begin; c < c_end; ++c) {
        const int64_t t0 = int64_t(c) * Q;
        const int Tc = tc_of(c);
        const int buf = (c - c_begin) & 1;
        const float *ell_s = coef_s + buf * (4 * kWave);
        const float *gam_s = ell_s + kWave, *wgt_s = gam_s + kWave, *scl_s = wgt_s + kWave;
        const float2 *thcb = thc_s + buf * K;

        // ---- a2: rotate B and C with the cos/sin table; stage B, x, scaled x.
        // Each unit's register is refilled with the next chunk's unit as soon
        // as it is consumed, so the load issue overlaps the staging work.
        // The next chunk's loads are unconditional: past the last chunk they
        // reload the last one (unused).  A load under a condition would keep
        // the old register value alive beside the new one and cost register
        // copies, and a wait for every load, at the end of each chunk.
        const bool more = c + 1 < c_end;
        const int cn = more ? c + 1 : c, cn2 = min(c + 2, c_end - 1);
        const int64_t tn0 = int64_t(cn) * Q;
        const int Tn = tc_of(cn);
        constexpr int CPART = (OUT && C::CL) ? 4 : 0;
        static_for<0, C::UPT_B>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int u = tid + j * kPT;
            if (C::UB % kPT == 0 || u < C::UB) {
                const int v = u / C::URB, q = u - v * C::URB;
                const float4 *cr = reinterpret_cast<const float4 *>(cs_s + (v / R) * C::CSP + q * EPU);
                float4 csr[EPU / 4];
#pragma unroll
                for (int w4 = 0; w4 < EPU / 4; ++w4) csr[w4] = cr[w4];
                float e[EPU];
                unpack_unit(raw.bb[j], e, IO());
                float ec[EPU];
                if constexpr (OUT && C::CL) unpack_unit(raw.cu[j], ec, IO());
                // the unit's registers are free from here: the next chunk's unit
                // is loaded into them (kept after the unpack, so the loop needs
                // no register copies)
                __builtin_amdgcn_sched_barrier(0);
                load_chunk<C, IO, OUT, 1 | CPART, j>(p, b, h, hg, tn0, Tn, raw);
                if constexpr (BLK) {
                    // block prologue of the row's channels q*EPU..: the row is
                    // held by URB consecutive lanes
                    const int r = v % R;
                    float inv = 1.f, invc = 1.f;
                    if (p.blk.norm) {
                        float ss = 0.f, sc = 0.f;
#pragma unroll
                        for (int i = 0; i < EPU; ++i) ss += e[i] * e[i];
                        if constexpr (OUT && C::CL) {
#pragma unroll
                            for (int i = 0; i < EPU; ++i) sc += ec[i] * ec[i];
                        }
                        ss = row_sum<C::URB>(ss);
                        inv = rsqrtf(ss * (1.f / N) + p.blk.eps);
                        if constexpr (OUT && C::CL) {
                            sc = row_sum<C::URB>(sc);
                            invc = rsqrtf(sc * (1.f / N) + p.blk.eps);
                        }
                    }
                    const int wo = r * N + q * EPU;
                    block_unit<C, EPU>(e, inv, smem, wo, wo + R * N);
                    if constexpr (OUT && C::CL) block_unit<C, EPU>(ec, invc, smem, wo + 2 * R * N, wo + 3 * R * N);
                }
#pragma unroll
                for (int w4 = 0; w4 < EPU / 4; ++w4) {
                    const float4 a = csr[w4];
                    rot_neg(a.x, a.y, e[4 * w4], e[4 * w4 + 1]);
                    rot_neg(a.z, a.w, e[4 * w4 + 2], e[4 * w4 + 3]);
                    if constexpr (OUT && C::CL) {
                        rot_neg(a.x, a.y, ec[4 * w4], ec[4 * w4 + 1]);
                        rot_neg(a.z, a.w, ec[4 * w4 + 2], ec[4 * w4 + 3]);
                    }
                }
                if constexpr (BSC) {
                    const float sc = scl_s[v / R];
#pragma unroll
                    for (int i = 0; i < EPU; ++i) e[i] *= sc;
                }
                st_planes<PL, C::BS_PS, EPU>(bs + v * NBP + q * EPU, e);
                if constexpr (OUT && C::CL) st_planes<PL, C::BS_PS, EPU>(cl + v * NBP + q * EPU, ec);
            } else {
                load_chunk<C, IO, OUT, 1 | CPART, j>(p, b, h, hg, tn0, Tn, raw);
            }
        });
        static_for<0, C::UPT_X>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int u = tid + j * kPT;
            if (C::UX % kPT == 0 || u < C::UX) {
                const int v = u / C::URX, q = u - v * C::URX;
                float e[EPU];
                unpack_unit(raw.xx[j], e, IO());
                if constexpr (PL == 1)
                    *reinterpret_cast<uint4 *>(xr + v * PP + q * EPU) = raw.xx[j];
                else
                    st_planes<PL, C::X_PS, EPU>(xr + v * PP + q * EPU, e);
                __builtin_amdgcn_sched_barrier(0);
                load_chunk<C, IO, OUT, 2, j>(p, b, h, hg, tn0, Tn, raw);
                if constexpr (C::XS && !BSC) {
                    const float sc = scl_s[v / R];
#pragma unroll
                    for (int ee = 0; ee < EPU; ++ee) e[ee] *= sc;
                    st_planes<PL, C::X_PS, EPU>(xs + v * PP + q * EPU, e);
                }
            } else {
                load_chunk<C, IO, OUT, 2, j>(p, b, h, hg, tn0, Tn, raw);
            }
        });
        frag cf[C::TBW][NKS];
        if (OUT && !C::CL) {
#pragma unroll
            for (int i = 0; i < C::TBW; ++i) {
                const int tb = wave_block(i, wave);
                if (C::NTB < C::TBW * kPW && tb >= C::NTB) continue; // uniform: waves without this row block
                const int tok = (16 * tb + l16) / R;
                // (BLK) block prologue of this lane's channels of its row; the
                // row's channels are spread over lanes l16, l16 + 16, +32, +48
                float inv = 1.f;
                if constexpr (BLK) {
                    if (p.blk.norm) {
                        float ss = 0.f;
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) {
                            float sk = 0.f;
#pragma unroll
                            for (int f = 0; f < C::FU; ++f) sk += unit_sumsq(raw.cc[i][ks][f], IO());
                            ss += (N % 32 == 0 || 32 * ks + 8 * g < N) ? sk : 0.f;
                        }
                        ss += __shfl_xor(ss, 16);
                        ss += __shfl_xor(ss, 32);
                        inv = rsqrtf(ss * (1.f / N) + p.blk.eps);
                    }
                }
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int n0 = 32 * ks + 8 * g;
                    float e[8];
#pragma unroll
                    for (int f = 0; f < C::FU; ++f) unpack_unit(raw.cc[i][ks][f], e + f * EPU, IO());
                    if constexpr (BLK) {
                        const int wo = 2 * R * N + ((16 * tb + l16) % R) * N + min(n0, N - 8);
                        block_unit<C, 8>(e, inv, smem, wo, wo + R * N);
                    }
                    if (N % 32 == 0 || n0 < N) {
                        const float4 *cr = reinterpret_cast<const float4 *>(cs_s + tok * C::CSP + n0);
#pragma unroll
                        for (int w4 = 0; w4 < 2; ++w4) {
                            const float4 a = cr[w4];
                            rot_neg(a.x, a.y, e[4 * w4], e[4 * w4 + 1]);
                            rot_neg(a.z, a.w, e[4 * w4 + 2], e[4 * w4 + 3]);
                        }
                    }
                    frag cv = M::pack(e);
                    // (BLK) one fragment at a time, computed here (not next to
                    // its first use): bounds the table reads in flight
                    if constexpr (BLK) {
#pragma unroll
                        for (int k = 0; k < PL; ++k) {
                            u32x4_v t = __builtin_bit_cast(u32x4_v, cv.v[k]);
                            __asm__ volatile("" : "+v"(t));
                            cv.v[k] = __builtin_bit_cast(bf16x8, t);
                        }
                    }
                    cf[i][ks] = cv;
                }
            }
        }
        // Every load issued earlier has now been consumed (or, with bf16 I/O,
        // is consumed right here: the next chunk's theta rows and, without a
        // free coefficient wave, coefficients); only then are the next loads
        // issued, and none of them is touched before the next chunk, so no
        // wait on a load is ever held up by a newer one.
        if (C::MFP && c + 1 < c_end) {
            write_theta<C>(rp, tht);
            if constexpr (!CP2)
                run_coef<C, IO>(rp, tc_of(c + 1), t0 + Q, p.T, Ah, coef_s + (buf ^ 1) * (4 * kWave), misc_s + (buf ^ 1));
        }
        if (OUT && !C::CL) {
            __builtin_amdgcn_sched_barrier(0); // after the C fragments are unpacked
            load_chunk<C, IO, OUT, 4>(p, b, h, hg, tn0, Tn, raw);
        }
        if constexpr (C::MFP) {
            load_theta<C, IO>(p, b, h, int64_t(cn2) * Q, tc_of(cn2), rp);
            if constexpr (!CP2) load_pro<C, IO>(p, b, h, int64_t(cn2) * Q, tc_of(cn2), rp);
        }

        // ---- a3 mask of this chunk: L[t][s] = exp(ell_t - ell_s) wgt_s (s < t),
        // gam_t (s = t), 0 (s > t); row t, ME consecutive s per thread: 8 for
        // 64-token chunks, fewer for small chunks so that more threads share
        // the table (with 8 per thread a 16-token chunk's table would fall on
        // 32 threads of one wave).  With R = 1 and 64-token chunks the rows
        // t < 32 are read for s < 32 only (their source pair), so 384 groups
        // are evaluated, by the first six waves.
        if constexpr (C::LWT) {
            constexpr bool HALF = R == 1 && Q == 64 && kPT == 512;
            constexpr int ME = Q * Q >= 8 * kPT ? 8 : Q * Q >= kPT ? Q * Q / kPT : 1; // entries per thread
            constexpr int GM = Q / ME;                                                // threads per mask row
            const int gi = HALF && tid >= 128 ? tid + 128 : tid; // skip rows < 32 x s >= 32
            const int tt = HALF ? (tid < 128 ? tid >> 2 : gi >> 3) : tid / GM;
            const int s0 = HALF ? (tid < 128 ? (tid & 3) * 8 : (gi & 7) * 8) : (tid % GM) * ME;
            if (OUT && (HALF ? tid < 384 : tid < Q * GM)) {
                float w[ME];
                {
                    // branch-free: every entry is evaluated, then selected
                    const float et = ell_s[tt], gt = gam_s[tt];
                    float el[ME], wg[ME];
                    if constexpr (ME == 8) {
                        const float4 e0 = *reinterpret_cast<const float4 *>(ell_s + s0);
                        const float4 e1 = *reinterpret_cast<const float4 *>(ell_s + s0 + 4);
                        const float4 w0 = *reinterpret_cast<const float4 *>(wgt_s + s0);
                        const float4 w1 = *reinterpret_cast<const float4 *>(wgt_s + s0 + 4);
                        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
                        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            el[j] = ev[j];
                            wg[j] = wv[j];
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < ME; ++j) {
                            el[j] = ell_s[s0 + j];
                            wg[j] = wgt_s[s0 + j];
                        }
                    }
#pragma unroll
                    for (int j = 0; j < ME; ++j) {
                        // exp of a selected argument (0 where masked), then 0/1
                        // weights: no select or branch around the exp
                        const int ts = s0 + j;
                        const float lt = ts < tt ? 1.f : 0.f, eq = ts == tt ? 1.f : 0.f;
                        const float e = __expf(ts < tt ? et - el[j] : 0.f);
                        w[j] = lt * (e * wg[j]) + eq * gt;
                    }
                }
                float *dst = lw_s + tt * C::LWP + s0;
                if constexpr (ME == 8) {
                    reinterpret_cast<float4 *>(dst)[0] = make_float4(w[0], w[1], w[2], w[3]);
                    reinterpret_cast<float4 *>(dst)[1] = make_float4(w[4], w[5], w[6], w[7]);
                } else {
#pragma unroll
                    for (int j = 0; j < ME; ++j) dst[j] = w[j];
                }
            }
            if (OUT && tid < Q) lw_s[Q * C::LWP + tid] = __expf(ell_s[tid]);
        }

        __syncthreads();

        const float gc = misc_s[buf];
        // a1 coefficients of the next chunk on the free coefficient wave, first
        // thing after the barrier: its dt, lam were loaded a chunk earlier and
        // only unconditional loads were issued since
        if constexpr (CP2) {
            if (c + 1 < c_end)
                run_coef<C, IO>(rp, tc_of(c + 1), t0 + Q, p.T, Ah, coef_s + (buf ^ 1) * (4 * kWave), misc_s + (buf ^ 1));
            load_pro<C, IO>(p, b, h, int64_t(cn2) * Q, tc_of(cn2), rp);
        }
        // a1 angles of the next chunk (bf16 I/O: from the theta table written
        // before the barrier), on the waves that own no intra-chunk rows, while
        // the others take the products.  This chunk's staging has read the
        // cos/sin table, and the chunk rotation is double-buffered.
        if constexpr (C::MFP) {
            if (c + 1 < c_end) run_angles<C, IO>(rp, tc_of(c + 1), cs_s, thc_s + (buf ^ 1) * K, ths_s, tht);
        }
        if (OUT) {
            // ---- a3 + a5: y = M x + exp(ell) Chat H for this wave's row blocks,
            // evaluated transposed (y^T = x^T M^T + H^T Chat^T exp(ell)) so that
            // each lane holds consecutive outputs along P
            IO *ybase = static_cast<IO *>(p.y) + ((b * p.T + t0) * p.H + h) * (R * P);
#pragma unroll
            for (int i = 0; i < C::TBW; ++i) {
                const int tb = wave_block(i, wave);
                if (tb >= C::NTB) continue;
                const int t0v = 16 * tb;
                if (t0v / R >= Tc) continue;
                const int tok_last = min((t0v + 15) / R, Tc - 1);
                // (BLK) gate inputs of this lane's outputs, issued here and used
                // at the store; without a gate they are read from x (unused)
                typename io4<IO>::raw zr[BLK ? PT : 1];
                if constexpr (BLK) {
                    const int vr = t0v + l16;
                    const int tz = min(vr / R, Tc - 1), cz = vr % R;
                    const IO *zb = static_cast<const IO *>(p.blk.z ? p.blk.z : p.x) +
                                   ((b * p.T + t0 + tz) * p.H + h) * (R * P) + cz * P + 4 * g;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) zr[pt] = io4<IO>::load(zb + 16 * pt);
                }
                if constexpr (C::CL) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int n0 = 32 * ks + 8 * g;
                        cf[i][ks] = (N % 32 == 0 || n0 < N) ? M::template lds8<C::BS_PS>(cl + (t0v + l16) * NBP + n0) : M::zero();
                    }
                }
                // acci: the inter-chunk term C~ H; acc: the intra-chunk term M x.
                // With rank R > 1 and 64 virtual rows both source pairs are
                // always taken (the mask is zero above the diagonal) and the
                // whole products phase is one straight-line block, so the
                // compiler interleaves the two independent chains (ILP).
                // Otherwise the inter term is scaled in place and the intra
                // term accumulates onto it.
                constexpr bool ILP = R > 1 && V <= 64;
                floatx4 acc[PT], acci[ILP ? PT : 1];
                auto inter = [&](int pt) -> floatx4 & {
                    if constexpr (ILP) return acci[pt];
                    else return acc[pt];
                };
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[pt] = inter(pt) = floatx4{0.f, 0.f, 0.f, 0.f};
                {
                    // C~ H, the state fragments read DEPTH products ahead
                    constexpr int NI = PT * NKS, DEPTH = NI < 4 ? NI : 4;
                    // step it: k-step it / PT, column tile it % PT (consecutive
                    // products go to different accumulators)
                    auto hfrag = [&](int it) {
                        const int pt = it % PT, n0 = 32 * (it / PT) + 8 * g;
                        return (N % 32 == 0 || n0 < N) ? M::template lds8<C::HT_PS>(ht + (16 * pt + l16) * NBP + n0) : M::zero();
                    };
                    if constexpr (!ILP) __builtin_amdgcn_sched_barrier(0);
                    frag hq[DEPTH];
#pragma unroll
                    for (int d = 0; d < DEPTH; ++d) hq[d] = hfrag(d);
#pragma unroll
                    for (int it = 0; it < NI; ++it) {
                        inter(it % PT) = M::mma(inter(it % PT), hq[it % DEPTH], cf[i][it / PT]);
                        if (it + DEPTH < NI) hq[it % DEPTH] = hfrag(it + DEPTH);
                    }
                    if constexpr (N % 32 == 0 && !ILP) sched_pipeline<NI, DEPTH, PL, M::kMfma>();
                    if constexpr (!ILP) __builtin_amdgcn_sched_barrier(0);
                }
                float einter; // e^{ell} of this lane's column token (0 past Tc)
                {
                    // the products are transposed (rows p, column = this lane's
                    // virtual row t0v + l16), so one decay factor per lane
                    const int tok = (t0v + l16) / R;
                    float e;
                    if constexpr (C::LWT) e = lw_s[Q * C::LWP + tok];
                    else e = __expf(ell_s[tok]);
                    if (tok >= Tc) e = 0.f;
                    einter = e;
                    if constexpr (!ILP) {
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) acc[pt] *= e;
                    }
                }
                const int tt = (t0v + l16) / R; // token of this lane's column t
                const float ell_t = ell_s[tt], gam_t = gam_s[tt];
                // mask weight of source token ts for this lane's column token
                // tt (exp argument selected first, so masked entries cannot
                // overflow)
                auto mw = [&](int ts, float ell_ts, float wgt_ts) {
                    const float e = __expf(ts < tt ? ell_t - ell_ts : 0.f) * wgt_ts;
                    return ts < tt ? e : (ts == tt ? gam_t : 0.f);
                };
                // S^T for the 32 source rows s0 .. s0+31 (two 16-row blocks)
                auto s_pair = [&](int s0, floatx4 *sb) {
                    // step it: k-step it / 2, block it % 2, the B~ fragments
                    // read D2 products ahead
                    constexpr int NI2 = 2 * NKS, D2 = NI2 < 4 ? NI2 : 4;
                    auto bfrag = [&](int it) {
                        const int n0 = 32 * (it / 2) + 8 * g;
                        return (N % 32 == 0 || n0 < N) ? M::template lds8<C::BS_PS>(bs + (s0 + 16 * (it % 2) + l16) * NBP + n0) : M::zero();
                    };
                    sb[0] = sb[1] = floatx4{0.f, 0.f, 0.f, 0.f};
                    frag bq[D2];
#pragma unroll
                    for (int d = 0; d < D2; ++d) bq[d] = bfrag(d);
#pragma unroll
                    for (int it = 0; it < NI2; ++it) {
                        sb[it % 2] = M::mma(sb[it % 2], bq[it % D2], cf[i][it / 2]);
                        if (it + D2 < NI2) bq[it % D2] = bfrag(it + D2);
                    }
                    if constexpr (N % 32 == 0 && !ILP) sched_pipeline<NI2, D2, PL, M::kMfma>();
                };
                // x operand of M x: slots 0-3 are rows s0 + 4g .. +3, slots
                // 4-7 rows s0 + 16 + 4g .. +3 (the k order of the M fragment)
                const uint16_t *xq = xr + (4 * g + (l16 >> 2)) * PP + 4 * (l16 & 3);
                const int npairs = ILP ? V / 32 : (R * (tok_last + 1) + 31) / 32;
                // mask weights of this lane's 4 source rows r0 .. r0+3 of block q
                // of the pair at s0, for its column token tt
                auto mask4 = [&](int s0, int q, float *w) {
                    const int r0 = s0 + 16 * q + 4 * g;
                    const float *lr = lw_s + tt * C::LWP; // mask row of this lane's column token
                    if constexpr (C::LWT && R == 1) {
                        const float4 a = *reinterpret_cast<const float4 *>(lr + r0);
                        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                    } else if constexpr (C::LWT && R == 2) {
                        const float2 a = *reinterpret_cast<const float2 *>(lr + r0 / 2);
                        w[0] = w[1] = a.x;
                        w[2] = w[3] = a.y;
                    } else if constexpr (C::LWT && R == 4) {
                        w[0] = w[1] = w[2] = w[3] = lr[r0 / 4];
                    } else if constexpr (C::LWT) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) w[v] = lr[(r0 + v) / R];
                    } else if constexpr (R == 1) {
                        const float4 el = *reinterpret_cast<const float4 *>(ell_s + r0);
                        const float4 wg = *reinterpret_cast<const float4 *>(wgt_s + r0);
                        w[0] = mw(r0, el.x, wg.x);
                        w[1] = mw(r0 + 1, el.y, wg.y);
                        w[2] = mw(r0 + 2, el.z, wg.z);
                        w[3] = mw(r0 + 3, el.w, wg.w);
                    } else if constexpr (R == 2) {
                        const float2 el = *reinterpret_cast<const float2 *>(ell_s + r0 / 2);
                        const float2 wg = *reinterpret_cast<const float2 *>(wgt_s + r0 / 2);
                        w[0] = w[1] = mw(r0 / 2, el.x, wg.x);
                        w[2] = w[3] = mw(r0 / 2 + 1, el.y, wg.y);
                    } else if constexpr (R == 4) {
                        w[0] = w[1] = w[2] = w[3] = mw(r0 / 4, ell_s[r0 / 4], wgt_s[r0 / 4]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int ts = (r0 + v) / R;
                            w[v] = mw(ts, ell_s[ts], wgt_s[ts]);
                        }
                    }
                };
                // the next pair's S and (tabulated) mask weights are fetched
                // while this pair's M x issues
                constexpr bool MPF = C::LWT && R == 1; // mask weights fetched a pair ahead (measured: helps R = 1 only)
                floatx4 sn[2];
                float wn[2][4];
                s_pair(0, sn);
                if constexpr (MPF) {
                    mask4(0, 0, wn[0]);
                    mask4(0, 1, wn[1]);
                }
                for (int mp = 0; mp < (ILP ? V / 32 : npairs); ++mp) {
                    const int s0 = 32 * mp;
                    const floatx4 sb[2] = {sn[0], sn[1]};
                    float wb[2][4];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int v = 0; v < 4; ++v) wb[q][v] = wn[q][v];
                    if (mp + 1 < npairs) {
                        s_pair(s0 + 32, sn);
                        if constexpr (MPF) {
                            mask4(s0 + 32, 0, wn[0]);
                            mask4(s0 + 32, 1, wn[1]);
                        }
                    }
                    if constexpr (!MPF) {
                        mask4(s0, 0, wb[0]);
                        mask4(s0, 1, wb[1]);
                    }
                    float m[8];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int v = 0; v < 4; ++v) m[4 * q + v] = sb[q][v] * wb[q][v];
                    const frag mf = M::pack(m);
                    const uint16_t *xs0 = xq + s0 * PP;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        acc[pt] = M::mma(acc[pt], M::template tr8<C::X_PS>(xs0 + 16 * pt, xs0 + 16 * PP + 16 * pt), mf);
                }
                {
                    // y^T tile: this lane holds outputs p = 16 pt + 4 g .. +3 of
                    // virtual row t0v + l16, four consecutive elements per store
                    const int vr = t0v + l16;
                    const int tok = vr / R, ch = vr - tok * R;
                    if (tok < Tc) {
                        IO *dst = ybase + ((tok * p.H * R + ch) * P + 4 * g);
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) {
                            float o4[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) o4[q] = ILP ? acc[pt][q] + einter * inter(pt)[q] : acc[pt][q];
                            if constexpr (BLK) {
                                if (p.blk.z) {
                                    // output gate: y * silu(z)
                                    float zv[4];
                                    io4<IO>::unpack(zr[pt], zv);
#pragma unroll
                                    for (int q = 0; q < 4; ++q) o4[q] *= silu(zv[q]);
                                }
                            }
                            io<IO>::store4(dst + 16 * pt, o4);
                        }
                    }
                }
            }
        }

        // ---- a4: H <- R(Theta_c) (exp(g_c) H + sum_v Bhat[v] (scaled x)[v]^T)
        {
            const float eg = __expf(gc);
            // slot j of both operands is virtual row 32 ks + 4 g + j (j < 4) or
            // 32 ks + 16 + 4 g + j - 4 (j >= 4)
            const int ra = 4 * g + (l16 >> 2), ca = 4 * (l16 & 3);
            // tile j of this wave: wave + 8 j, i.e. row block nt_j = (wave + 8 j) / PT
            // and the same column block pt = wave % PT for every j (8 is a
            // multiple of PT), so each k-step reads the x operand once
            static_assert(kPW % PT == 0, "state tiles share their column block");
            const int pt = wave % PT;
            floatx4 acc[C::TW];
#pragma unroll
            for (int j = 0; j < C::TW; ++j) acc[j] = st[j] * eg;
            const uint16_t *bp = ((C::XS && !BSC) ? xs : xr) + ra * PP + 16 * pt + ca;
#pragma unroll 2
            for (int ks = 0; ks < V / 32; ++ks) {
                frag bf = M::template tr8<C::X_PS>(bp + 32 * ks * PP, bp + (32 * ks + 16) * PP);
                if constexpr (!C::XS && !BSC) {
                    float f[8];
                    M::unpack(bf, f);
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) f[jj] *= scl_s[(32 * ks + (jj < 4 ? 4 * g + jj : 12 + 4 * g + jj)) / R];
                    bf = M::pack(f);
                }
#pragma unroll
                for (int j = 0; j < C::TW; ++j) {
                    const int tile = wave + kPW * j;
                    if (tile >= C::NTILE) continue;
                    const uint16_t *ap = bs + ra * NBP + 16 * (tile / PT) + ca;
                    const frag af = M::template tr8<C::BS_PS>(ap + 32 * ks * NBP, ap + (32 * ks + 16) * NBP);
                    acc[j] = M::mma(acc[j], af, bf);
                }
            }
#pragma unroll
            for (int j = 0; j < C::TW; ++j) {
                const int tile = wave + kPW * j;
                if (tile >= C::NTILE) continue;
                const int nt = tile / PT;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float2 cs = thcb[8 * nt + 2 * g + q];
                    st[j][2 * q] = cs.x * acc[j][2 * q] - cs.y * acc[j][2 * q + 1];
                    st[j][2 * q + 1] = cs.y * acc[j][2 * q] + cs.x * acc[j][2 * q + 1];
                }
            }
        }
        gsum += gc;

        // ---- a1 of the next chunk, fp32 I/O: angles and coefficients (from
        // the registers loaded a chunk ahead)
        if (c + 1 < c_end) {
            if constexpr (!C::MFP) {
                run_angles<C, IO>(rp, tc_of(c + 1), cs_s, thc_s + (buf ^ 1) * K, ths_s, tht);
                run_coef<C, IO>(rp, tc_of(c + 1), t0 + Q, p.T, Ah, coef_s + (buf ^ 1) * (4 * kWave), misc_s + (buf ^ 1));
                load_pro<C, IO>(p, b, h, int64_t(cn2) * Q, tc_of(cn2), rp);
            }
        }
        __syncthreads();

        if (OUT) {
#pragma unroll
            for (int j = 0; j < C::TW; ++j) {
                const int tile = wave + kPW * j;
                if (tile >= C::NTILE) continue;
                const int nt = tile / PT, pt = tile - nt * PT;
                const float sv[4] = {st[j][0], st[j][1], st[j][2], st[j][3]};
                st_planes<PL, C::HT_PS, 4>(ht + (16 * pt + l16) * NBP + 16 * nt + 4 * g, sv);
            }
        }
    }

    if (!OUT) {
        // segment aggregate: state from zero, summed log decay and angle
        float *U = p.segU + (bh * p.NA + seg) * int64_t(N) * P;
#pragma unroll
        for (int j = 0; j < C::TW; ++j) {
            const int tile = wave + kPW * j;
            if (tile >= C::NTILE) continue;
            const int nt = tile / PT, pt = tile - nt * PT;
#pragma unroll
            for (int v = 0; v < 4; ++v) U[(16 * nt + 4 * g + v) * P + 16 * pt + l16] = st[j][v];
        }
        if (tid == 0) p.segG[bh * p.NA + seg] = gsum;
        for (int k = tid; k < K; k += kPT) p.segTh[(bh * p.NA + seg) * K + k] = ths_s[k];
        return;
    }
    if (seg != p.S - 1 || !p.has_final) return;

    // final carried state in the rotated frame: h~ = R(-Phi_{T-1}) H
    const int64_t hTb = bh * int64_t(N) * P;
    auto put_h = [&](int64_t i, float v) { // final state in its storage type
        if (p.sbf16) static_cast<uint16_t *>(p.hT)[hTb + i] = f32_to_bits(v);
        else static_cast<float *>(p.hT)[hTb + i] = v;
    };
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
            put_h((16 * nt + 4 * g + 2 * q) * P + 16 * pt + l16, u);
            put_h((16 * nt + 4 * g + 2 * q + 1) * P + 16 * pt + l16, v);
        }
    }
    const int64_t tl = (b * p.T + p.T - 1) * p.H + h;   // token-head index of T-1 (x)
    const int64_t tlg = (b * p.T + p.T - 1) * p.G + hg; // token-group index of T-1 (B)
    for (int k = tid; k < K; k += kPT) p.phiT[bh * K + k] = float(wrap_angle(ths_s[k]));
    for (int i = tid; i < R * K; i += kPT) {
        const int r = i / K, k = i - r * K;
        float sn, cs;
        sincos_wrapped(wrap_angle(ths_s[k]), &sn, &cs);
        const IO *Bl = static_cast<const IO *>(p.B) + (tlg * R + r) * N + 2 * k;
        float u = io<IO>::get(Bl), v = io<IO>::get(Bl + 1);
        if constexpr (BLK) {
            // block prologue of the last token's B row r (its RMS over N
            // summed here by this thread)
            float inv = 1.f;
            if (p.blk.norm) {
                const IO *row = Bl - 2 * k;
                float ss = 0.f;
                for (int n = 0; n < N; ++n) {
                    const float t = io<IO>::get(row + n);
                    ss += t * t;
                }
                inv = rsqrtf(ss * (1.f / N) + p.blk.eps);
            }
            const float *wr = blk_row<C>(smem, r * N + 2 * k), *br = blk_row<C>(smem, R * N + r * N + 2 * k);
            u = u * inv * wr[0] + br[0];
            v = v * inv * wr[1] + br[1];
        }
        rot_neg(cs, sn, u, v);
        p.prevBT[(bh * R + r) * N + 2 * k] = u;
        p.prevBT[(bh * R + r) * N + 2 * k + 1] = v;
    }
    const IO *xl = static_cast<const IO *>(p.x) + tl * R * P;
    IO *px = static_cast<IO *>(p.prevxT) + bh * R * P;
    for (int i = tid; i < R * P; i += kPT) px[i] = xl[i];
}

// Host-side launch of one instantiation (pre-pass when OUT is false; the
// block prologue/epilogue kernels when BLK).
template <typename IO, int N, int P, int R, int QC, bool OUT, bool BLK>
hipError_t launch_prefill_inst(const PrefillParams &p, hipStream_t s) {
    typedef Cfg<IO, N, P, R, QC, BLK> C;
    const int nseg = OUT ? p.S : (p.S - 1) * p.kpre;
    if (nseg <= 0) return hipSuccess;
    if (C::bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_prefill<IO, N, P, R, QC, OUT, BLK>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(C::bytes));
        if (e != hipSuccess) return e;
    }
    const dim3 grid(unsigned(p.batch * p.H * nseg)), block(kPT);
    hipLaunchKernelGGL((k_prefill<IO, N, P, R, QC, OUT, BLK>), grid, block, C::bytes, s, p);
    return hipGetLastError();
}

// The instantiation for rank R with chunks of 64 tokens (SMALL false) or of
// small_chunk(R) tokens (SMALL true); combinations whose tiles do not fit in
// the LDS of a CU are not compiled and report hipErrorInvalidValue, as does a
// call whose chunk length p.Q is not this one's.
template <typename IO, int N, int P, int R, bool BLK, bool SMALL>
hipError_t launch_prefill_r(const PrefillParams &p, bool out, hipStream_t s) {
    constexpr int QC = SMALL ? small_chunk(R) : kQ;
    if constexpr ((SMALL && QC == kQ) || Cfg<IO, N, P, R, QC, BLK>::bytes > kMaxLdsBytes) {
        return hipErrorInvalidValue;
    } else {
        if (p.Q != QC) return hipErrorInvalidValue;
        return out ? launch_prefill_inst<IO, N, P, R, QC, true, BLK>(p, s)
                   : launch_prefill_inst<IO, N, P, R, QC, false, BLK>(p, s);
    }
}
template <typename IO, int N, int P, bool BLK, bool SMALL>
hipError_t launch_prefill_pr(const PrefillParams &p, bool out, hipStream_t s) {
    switch (p.R) {
    case 1: return launch_prefill_r<IO, N, P, 1, BLK, SMALL>(p, out, s);
    case 2: return launch_prefill_r<IO, N, P, 2, BLK, SMALL>(p, out, s);
    case 3: return launch_prefill_r<IO, N, P, 3, BLK, SMALL>(p, out, s);
    case 4: return launch_prefill_r<IO, N, P, 4, BLK, SMALL>(p, out, s);
    }
    return hipErrorInvalidValue;
}
// Every (P, R) of one (I/O type, N, block variant, chunk kind).
template <typename IO, int N, bool BLK, bool SMALL>
hipError_t launch_prefill_np(const PrefillParams &p, bool out, hipStream_t s) {
    switch (p.P) {
    case 16: return launch_prefill_pr<IO, N, 16, BLK, SMALL>(p, out, s);
    case 32: return launch_prefill_pr<IO, N, 32, BLK, SMALL>(p, out, s);
    case 64: return launch_prefill_pr<IO, N, 64, BLK, SMALL>(p, out, s);
    }
    return hipErrorInvalidValue;
}

} // namespace m3
