// k_backward.hpp -- gradients of the mixer in chunked form: one workgroup per
// (batch, head), chunks of Q tokens processed last to first, every product
// of a chunk on fp32 MFMA (v_mfma_f32_16x16x4_f32), angles in fp64.
//
// Forward map: the rotated-frame form of the Mamba-3 review, section 3.2.2,
// Prop. 3.2.3, with the coefficients of section 3.1.1, eq. (6), and the
// rank-R products of section 3.3:
//   h~_t = a_t h~_{t-1} + b_t B~_{t-1} x_{t-1}^T + g_t B~_t x_t^T,  y_t = C~_t^T h~_t,
//   B~_t = R(-Phi_t) B_t (same for C), Phi_t = Phi_{t-1} + theta_t,
//   a_t = e^{l_t}, l_t = dt_t A, b_t = d_t a_t, d_t = (1 - lam_t) dt_t, g_t = lam_t dt_t.
// Since b_{s+1} e^{-cum_{s+1}} = d_{s+1} e^{-cum_s}, token s enters h~_t
// (t >= s) with weight e^{cum_t - cum_s} (g_s + [t > s] d_{s+1}): the two taps
// of the trapezoid fold into one decay mask (the review, section 3.1.3,
// eq. (7)), and the chunked SSD form of its section 2.3 applies.
//
// A chunk holds V = Q R rows (token i, rank r -> row i R + r; rows past the
// chunk's tokens are zero).  With ec_i the sum of l over the chunk's tokens
// up to i, dn_j = d of token j + 1, and
//   W(i,j) = [i >= j] e^{ec_i - ec_j} (g_j + [i > j] dn_j),
//   U_j = e^{ec_end - ec_j} (g_j + dn_j),  E_i = e^{ec_i},
//   H_c = h~_{t0-1} + d_{t0} B~_{t0-1} x_{t0-1}^T  (the state entering the chunk),
// the forward is y_v = sum_v' W S(v,v') x_v' + E_i C~_v^T H_c with S = C~ B~^T,
// and H_{c+1} = e^{ec_end} H_c + sum_v' U_j B~_v' x_v'^T.  Given G, the
// gradient of H_{c+1} (zero after the last chunk), and D = gy x^T:
//   dx  = (W.S)^T gy + diag(U) B~ G,     dC~ = (W.D) B~ + diag(E) gy H_c^T,
//   dB~ = (W.D)^T C~ + diag(U) x G^T,    dH_c = e^{ec_end} G + C~^T diag(E) gy,
//   dW(i,j) = sum over the R x R block of S.D,  dU_j = <G, B~_j x_j^T>,
//   dE_i = <C~_i, H_c gy_i>,  d e^{ec_end} = <G, H_c>,
// and the chain rule through W, U and E gives the gradient of each ec_k,
// whose suffix sums over the chunk are the gradients of l.  The rotations give
// dB = R(Phi) dB~ (same for C) and dPhi_t[k] = sum_r (dB~_2k B~_2k+1 -
// dB~_2k+1 B~_2k) + (the same for C); dtheta_t = sum_{s >= t} dPhi_s.  The
// carried state gets dh~_{-1} = dH_0, dB~_{-1} = d_0 dH_0 x_{-1},
// dx_{-1} = d_0 B~_{-1}^T dH_0, dPhi_{-1} = sum_t dPhi_t, and d_0 receives
// <dH_0, B~_{-1} x_{-1}^T>.
//
// Two sweeps per workgroup: forward over the chunks storing H_c and the
// angle at each chunk start (workspace), then backward over the chunks.
// MFMA operand convention: in step (kb, e) of a product, k-slot g of lane l
// stands for contraction index 16 kb + 4 g + e.  An operand in LDS is stored
// with the contraction index contiguous (row pitch 4 x odd, so that 16-byte
// reads of 16 rows hit distinct banks): one 16-byte read gives a lane its
// operand for four steps.  A 16 x 16 accumulator tile (lane l holds rows
// 4 (l / 16) + e of column l % 16) is the B operand of step (kb, e) as it
// stands, which keeps the carried gradient G (in both orientations) and H_c
// in registers.
#pragma once
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

// 8 waves, two per SIMD, in two groups of four: waves 0-3 carry G in one
// orientation (dx and its update), waves 4-7 in the other (dC~, dB~ and its
// update), so that one wave's vector work overlaps the other's MFMAs.
constexpr int kBwdThreads = 512;
constexpr int kBwdWaves = kBwdThreads / 64;

// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][slot l / 16] and
// B[slot l / 16][l % 16]; element e of the result is D[4 (l / 16) + e][l % 16].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ floatx4 lds4(const float *q) { return *reinterpret_cast<const floatx4 *>(q); }

// acc[vb] += A B over k = 0 .. KD-1 for NV row blocks of A: A[i][k] =
// a[(16 vb + i) * PA + k], B[k][j] = bm[j * PBM + k] (both k-contiguous).
// Lane (i, g) reads four consecutive k (16 kb + 4 g ..) of its row and
// column with one 16-byte read each: steps (kb, 0..3).
// The reads of group kb + 1 are issued before the products of group kb (the
// schedule is pinned, so that each group of MFMAs has the next group's
// operands in flight).
// ZV >= 0: the block of A in row block ZV and k block ZK is known to be zero
// (a masked triangle) and its products are skipped.
template <int KD, int PA, int PBM, int NV, int ZV = -1, int ZK = -1>
__device__ __forceinline__ void mm_lds(floatx4 (&acc)[NV], const float *a, const float *bm, int i, int g) {
    constexpr int NK = KD / 16;
    auto live = [](int vb, int kb) { return !(vb == ZV && kb == ZK); };
    floatx4 bv[2], av[2][NV];
    __builtin_amdgcn_sched_barrier(0);
    bv[0] = lds4(bm + i * PBM + 4 * g);
#pragma unroll
    for (int vb = 0; vb < NV; ++vb)
        if (live(vb, 0)) av[0][vb] = lds4(a + (16 * vb + i) * PA + 4 * g);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
        const int cu = kb & 1, nx = cu ^ 1;
        if (kb + 1 < NK) {
            bv[nx] = lds4(bm + i * PBM + 16 * (kb + 1) + 4 * g);
#pragma unroll
            for (int vb = 0; vb < NV; ++vb)
                if (live(vb, kb + 1)) av[nx][vb] = lds4(a + (16 * vb + i) * PA + 16 * (kb + 1) + 4 * g);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int vb = 0; vb < NV; ++vb)
                if (live(vb, kb)) acc[vb] = mfma4(av[cu][vb][e], bv[cu][e], acc[vb]);
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int N, int P, int R>
struct BwdCfg {
    static constexpr int V = kBwdV, Q = V / R, VQ = Q * R, QP = Q + 1;
    static constexpr int K = N / 2, NB = N / 16, PB = P / 16, VB = V / 16, NBW = (NB + 3) / 4;
    // row pitches 4 x odd: 16-byte reads of 16 rows hit distinct banks
    static constexpr int pV = V + 4, pN = N + 4, pP = P + 4, pK = K + 4, pC = K + 1, pQ = QP + 1, SQ = 36;
    static_assert(P <= 2 * V, "the forward sweep's second x^T buffer is the mask area");
    static constexpr int TPS = (Q + 7) / 8; // tokens per segment of the angle scans
    static constexpr int KS = 8 * kBwdWaves, KP = (K + KS - 1) / KS; // pairs per pass, passes of the angle scans
    static constexpr int NBH = (NB + kBwdWaves - 1) / kBwdWaves; // forward sweep: column blocks per wave
    static constexpr int GSN = NB > NBW * PB ? NB : NBW * PB;   // registers of G (either orientation)
    // token scalar tables, SQ floats each
    static constexpr int s_ec = 0, s_E = 1, s_EU = 2, s_U = 3, s_g = 4, s_dn = 5, s_dt = 6, s_lam = 7, s_misc = 8;
    // LDS (floats)
    static constexpr int o_bt = 0;              // B~^T [N][pV]
    static constexpr int o_ct = o_bt + N * pV;  // C~^T [N][pV]
    static constexpr int o_bn = o_ct + N * pV;  // B~ [V][pN]
    static constexpr int o_cn = o_bn + V * pN;  // C~ [V][pN]
    static constexpr int o_t2 = o_cn + V * pN;  // gy^T [P][pV]  (forward sweep: x^T)
    static constexpr int o_xn = o_t2 + P * pV;  // x [V][pP]
    static constexpr int o_gn = o_xn + V * pP;  // gy [V][pP]
    static constexpr int o_ms = o_gn + V * pP;  // (W.S)^T [V][pV]  (row v', column v)
    static constexpr int o_mn = o_ms + V * pV;  // W.D [V][pV]      (row v, column v')
    static constexpr int o_mt = o_mn + V * pV;  // (W.D)^T [V][pV]
    static constexpr int o_sd = o_mt + V * pV;  // S.D [V][pV]
    static constexpr int o_ph = o_sd + V * pV;  // dPhi terms [V][pK]
    static constexpr int o_cs = (o_ph + V * pK + 1) / 2 * 2; // cos, sin of Phi [Q][pC] float2
    static constexpr int o_et = o_cs + 2 * Q * pC; // e^{ec_i - ec_j} [QP][pQ]
    static constexpr int o_dw = o_et + QP * pQ; // per token: row sums, column sums, diagonal [3][pQ]
    static constexpr int o_sc = o_dw + 3 * pQ;  // token scalars [9][SQ]
    static constexpr int o_pu = o_sc + 9 * SQ;  // dU partials [4][V]
    static constexpr int o_pe = o_pu + 4 * V;   // dE partials [4][V]
    static constexpr int o_pz = o_pe + 4 * V;   // per-wave scalars [4][4]
    static constexpr int o_phe = (o_pz + 16 + 1) / 2 * 2; // Phi at the chunk end, fp64 [K]
    // When it fits: the adjoint G handed from the first wave group, which
    // updates it, to the second, which reloads it in its own layout, instead
    // of both groups updating it [N][pG] (row n, column p)
    static constexpr int pG = P + 4;
    static constexpr int o_gx = (o_phe + 2 * K + 3) / 4 * 4;
    static constexpr bool GX = size_t(o_gx + N * pG) * 4 <= kMaxLdsBytes;
    static constexpr int floats = GX ? o_gx + N * pG : o_phe + 2 * K;
    // Otherwise (GA) G goes through areas that are dead from the end of the
    // products to the next chunk's staging: 16-row blocks of G in the run
    // gy^T, x, gy, (W.S)^T (GAN blocks), the rest in S.D.
    static constexpr int GAN = (P * pV + 2 * V * pP + V * pV) / (16 * pG);
    static constexpr bool GA = !GX && GAN + (V * pV) / (16 * pG) >= NB;
    static constexpr size_t bytes = size_t(floats) * 4;
    static_assert(bytes <= kMaxLdsBytes, "backward LDS layout exceeds the workgroup's LDS");
    static_assert(Q * 8 <= kBwdThreads, "one group of 8 threads per token");
    static_assert(PB <= 4, "one column block of dx per wave of the first group");
    // with R dividing 16 no token's rows straddle the two 16-row blocks, so
    // the masks vanish on the block of later rows x earlier columns' transpose
    static constexpr bool TRI = 16 % R == 0 && V == 32;
    static constexpr int ZLO = TRI ? 1 : -1, ZHI = TRI ? 0 : -1; // row block with a zero k block
    // 4-element groups of B / C and of x / gy per chunk, per thread
    static constexpr int NBL = (V * N / 4 + kBwdThreads - 1) / kBwdThreads;
    static constexpr int NXL = (V * P / 4 + kBwdThreads - 1) / kBwdThreads;
};

template <typename IO, int N, int P, int R>
__global__ __launch_bounds__(kBwdThreads) void k_backward(const BwdParams p) {
    typedef BwdCfg<N, P, R> Cf;
    constexpr int V = Cf::V, Q = Cf::Q, VQ = Cf::VQ, QP = Cf::QP, K = Cf::K;
    constexpr int NB = Cf::NB, PB = Cf::PB, VB = Cf::VB, NBW = Cf::NBW, TPS = Cf::TPS, KP = Cf::KP, KS = Cf::KS;
    constexpr int NBH = Cf::NBH, GSN = Cf::GSN, ZLO = Cf::ZLO, ZHI = Cf::ZHI;
    constexpr int pV = Cf::pV, pN = Cf::pN, pP = Cf::pP, pK = Cf::pK, pC = Cf::pC, pQ = Cf::pQ, SQ = Cf::SQ;
    constexpr int NBL = Cf::NBL, NXL = Cf::NXL;
    extern __shared__ __align__(16) float sm[];
    float *BT = sm + Cf::o_bt, *CT = sm + Cf::o_ct, *BN = sm + Cf::o_bn, *CN = sm + Cf::o_cn;
    float *T2 = sm + Cf::o_t2, *XN = sm + Cf::o_xn, *GN = sm + Cf::o_gn;
    float *MS = sm + Cf::o_ms, *MN = sm + Cf::o_mn, *MT = sm + Cf::o_mt, *SD = sm + Cf::o_sd;
    float *PH = sm + Cf::o_ph, *ET = sm + Cf::o_et, *DW = sm + Cf::o_dw;
    float2 *CS = reinterpret_cast<float2 *>(sm + Cf::o_cs);
    float *SC = sm + Cf::o_sc, *PU = sm + Cf::o_pu, *PE = sm + Cf::o_pe, *PZ = sm + Cf::o_pz;
    double *PHE = reinterpret_cast<double *>(sm + Cf::o_phe);
    // row n of the adjoint G handed from the first wave group to the second
    // (GX: its own buffer [N][pG]; GA: 16-row blocks in borrowed areas)
    auto gx_row = [&](int n) -> float * {
        if constexpr (Cf::GX) return sm + Cf::o_gx + n * Cf::pG;
        const int nb = n >> 4;
        return (nb < Cf::GAN ? sm + Cf::o_t2 + nb * 16 * Cf::pG : sm + Cf::o_sd + (nb - Cf::GAN) * 16 * Cf::pG) +
               (n & 15) * Cf::pG;
    };
    auto sc = [&](int s, int i) -> float & { return SC[s * SQ + i]; };

    // lane ids, re-derived through an opaque copy at the top of every chunk so
    // that the per-lane addresses built from them are not hoisted out of the
    // chunk loops (kept live across them, they exceed the register file)
    int tid = threadIdx.x, lane = 0, w = 0, li = 0, lg = 0;
    auto lane_ids = [&]() {
        asm volatile("" : "+v"(tid));
        lane = tid & (kWave - 1);
        w = __builtin_amdgcn_readfirstlane(tid) / kWave;
        li = lane & 15;
        lg = lane >> 4;
    };
    lane_ids();
    // workgroup -> (b, h, segment) and its role: 0 the gradients of the
    // segment, 1 the forward-state aggregate of one piece of a segment, 2 the
    // adjoint aggregate of one piece (a segment's aggregates are cut into KA
    // pieces of cps / KA chunks, so that the aggregate launch fills whole
    // rounds of the CUs)
    const int S = p.S, KA = p.kagg, NPC = S * KA; // pieces per sequence
    int64_t bh;
    int sg, role, pi = 0;
    if (p.mode == 0) {
        bh = blockIdx.x / S;
        sg = int(blockIdx.x % S);
        role = 0;
    } else {
        const int64_t nf = int64_t(S - 1) * KA * p.batch * p.H;
        int64_t idx = blockIdx.x;
        role = idx < nf ? 1 : 2;
        if (role == 2) idx -= nf;
        bh = idx / ((S - 1) * KA);
        pi = int(idx % ((S - 1) * KA)) + (role == 2 ? KA : 0);
        sg = pi / KA;
    }
    const int h = int(bh % p.H);
    const int64_t b = bh / p.H;
    const int64_t T = p.T;
    const int nC = p.nC;
    // this workgroup's chunks: the segment's, or one piece of it (possibly
    // empty past the end of a shorter last segment)
    const int cpp = p.cps / KA;
    const int c0 = role == 0 ? sg * p.cps : min(nC, sg * p.cps + (pi % KA) * cpp);
    const int c1 = role == 0 ? min(nC, c0 + p.cps) : min(nC, c0 + cpp);
    const int64_t bs = bh * S + sg;          // (b, h, segment) index
    const int64_t bp = int64_t(bh) * NPC + pi; // (b, h, piece) index of the aggregates
    const float Ah = p.A[h];
    const IO *xg = static_cast<const IO *>(p.x), *Bg = static_cast<const IO *>(p.B);
    const IO *Cg = static_cast<const IO *>(p.C), *gyg = static_cast<const IO *>(p.gy);
    const IO *thg = static_cast<const IO *>(p.theta), *dtg = static_cast<const IO *>(p.dt);
    const IO *lmg = static_cast<const IO *>(p.lam);
    auto tok = [&](int64_t t) { return (b * T + t) * p.H + h; };
    float *ckh = p.ck_h + bh * int64_t(nC) * N * P;
    double *ckp = p.ck_phi + bh * int64_t(nC) * K;
    // this lane's slot in a chunk's stored state: tile (nb, pb), lane-major
    auto ck_at = [&](int c, int nb, int pb) { return ckh + ((int64_t(c) * NB + nb) * PB + pb) * 256 + lane * 4; };
    auto row_tok = [&](int v) { return min(v / R, Q); }; // token slot of a row (Q: padding)

    // ---- a chunk's inputs are loaded into registers (raw bits) one chunk
    // ahead, during the previous chunk's products, and staged from there.
    // Loads past the chunk's tokens read a valid element and are zeroed when
    // staged.
    typedef typename io4<IO>::raw raw4;
    raw4 qb[NBL], qc[NBL], qx[NXL], qg[NXL];
    uint32_t qth[KP][TPS], qdt = 0, qlm = 0;
    // (addresses: the chunk's first token + a 32-bit offset; token i of the
    // chunk is i * H rows further)
    // (adj: only what the adjoint aggregate reads: C, gy and the scalars)
    auto issue = [&](int64_t t0, int Tc, bool bwd, bool adj) {
        const int64_t tb = tok(t0);
        const int HR = p.H * R;
        const IO *bb = Bg + tb * (R * N), *cb = Cg + tb * (R * N), *xb = xg + tb * (R * P), *gb = gyg + tb * (R * P);
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int gi = tid + j * kBwdThreads;
            const int v = gi % V, n = 4 * (gi / V), i = v / R;
            const bool ok = gi < V * N / 4 && v < VQ && i < Tc;
            const int off = ok ? (i * HR + v - i * R) * N + n : 0;
            if (!adj) qb[j] = io4<IO>::load(bb + off);
            if (bwd) qc[j] = io4<IO>::load(cb + off);
        }
#pragma unroll
        for (int j = 0; j < NXL; ++j) {
            const int gi = tid + j * kBwdThreads;
            const int v = gi % V, pc = 4 * (gi / V), i = v / R;
            const bool ok = gi < V * P / 4 && v < VQ && i < Tc;
            const int off = ok ? (i * HR + v - i * R) * P + pc : 0;
            if (!adj) qx[j] = io4<IO>::load(xb + off);
            if (bwd) qg[j] = io4<IO>::load(gb + off);
        }
        const IO *tbp = thg + tb * K;
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
            const int k = KS * kp + 8 * w + (lane & 7), seg = lane >> 3;
            const int kc = k < K ? k : 0;
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int i = seg * TPS + u;
                qth[kp][u] = io<IO>::raw(tbp + ((i < Tc ? i : 0) * p.H * K + kc));
            }
        }
        if (w == 0) {
            const int i = lane;
            const bool ld = i < Tc || (i == Q && t0 + Q < T);
            qdt = io<IO>::raw(dtg + tb + (ld ? i : 0) * p.H);
            qlm = io<IO>::raw(lmg + tb + (ld ? i : 0) * p.H);
        }
    };

    // ---- staging: token scalars (wave 0, lane = token; lane Q carries the
    // next chunk's first token for its d)
    auto stage_scalars = [&](int64_t t0, int Tc) {
        if (w == 0) {
            const int i = lane;
            const bool real = i < Tc, nxt = i == Q && t0 + Q < T;
            float d = 0.f, l = 0.f;
            if (real || nxt) {
                d = io<IO>::value(qdt);
                l = io<IO>::value(qlm);
            }
            const float ell = real ? d * Ah : 0.f;
            const float gam = real ? l * d : 0.f;
            const float dlt = real || nxt ? (1.f - l) * d : 0.f;
            float dn = __shfl_down(dlt, 1);
            if (i >= Q) dn = 0.f;
            const float ec = wave_scan_dpp(ell);
            const float ecE = __shfl(ec, Q - 1);
            const float E = __expf(ec), EU = __expf(ecE - ec);
            const float U = EU * (gam + dn);
            if (i <= Q) {
                sc(Cf::s_ec, i) = ec; sc(Cf::s_E, i) = E; sc(Cf::s_EU, i) = EU; sc(Cf::s_U, i) = U;
                sc(Cf::s_g, i) = gam; sc(Cf::s_dn, i) = dn; sc(Cf::s_dt, i) = real ? d : 0.f;
                sc(Cf::s_lam, i) = real ? l : 0.f;
            }
            if (i == 0) sc(Cf::s_misc, 0) = __expf(ecE);
        }
    };
    // Phi_t = Phi_start + the sum of theta over the chunk's tokens up to t,
    // fp64: lane = 8 segments x 8 pairs, a segment's prefix in registers, the
    // segment totals scanned over lanes 8 apart.  Writes CS (cos and sin of
    // Phi_t) and PHE (the wrapped angle of the chunk's last token).
    auto stage_angles = [&](int Tc, bool fwd, int c, bool store) {
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
            const int k = KS * kp + 8 * w + (lane & 7), seg = lane >> 3;
            const bool kv = k < K;
            const int kc = kv ? k : 0;
            const double ph0 = fwd ? PHE[kc] : ckp[int64_t(c) * K + kc];
            double lp[TPS];
            double run = 0.0;
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int i = seg * TPS + u;
                const bool ok = kv && i < Tc;
                const float th = io<IO>::value(qth[kp][u]);
                run += ok ? double(th) : 0.0;
                lp[u] = run;
            }
            double x = run;
#pragma unroll
            for (int o = 8; o < kWave; o <<= 1) {
                const double y = __shfl_up(x, o, kWave);
                if (lane >= o) x += y;
            }
            const double ex = x - run;
            if (fwd && store && kv && seg == 0) ckp[int64_t(c) * K + k] = ph0;
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int i = seg * TPS + u;
                if (kv && i < Q) {
                    const double ph = ph0 + ex + lp[u];
                    double tr = ph * (1.0 / kTwoPi);
                    tr -= rint(tr);
                    const float tf = float(tr);
                    CS[i * pC + k] = make_float2(__builtin_amdgcn_cosf(tf), __builtin_amdgcn_sinf(tf));
                    if (i == Tc - 1) PHE[k] = wrap_angle(ph);
                }
            }
        }
    };
    // rotate by -Phi (CS) and store transposed (dT, [n][v]) and row-major (dN, [v][n])
    // (B or C of the chunk, row v = group % V fastest)
    auto rot_store = [&](const raw4 (&qv)[NBL], int Tc, float *dT, float *dN) {
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int gi = tid + j * kBwdThreads;
            if (gi >= V * N / 4) continue;
            const int v = gi % V, n = 4 * (gi / V), i = min(v / R, Q - 1);
            const bool ok = v < VQ && v / R < Tc;
            const float2 c0 = CS[i * pC + n / 2], c1 = CS[i * pC + n / 2 + 1];
            float o[4];
            io4<IO>::unpack(qv[j], o);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = ok ? o[q] : 0.f;
            rot_neg(c0.x, c0.y, o[0], o[1]);
            rot_neg(c1.x, c1.y, o[2], o[3]);
            if (dN) *reinterpret_cast<float4 *>(dN + v * pN + n) = make_float4(o[0], o[1], o[2], o[3]);
            if (dT)
#pragma unroll
                for (int q = 0; q < 4; ++q) dT[(n + q) * pV + v] = o[q];
        }
    };
    // x (and gy) of the chunk into LDS: the forward sweep keeps x transposed
    // (T2); the backward sweep keeps x row-major (XN) and gy both ways (GN, T2)
    auto stage_xg = [&](int Tc, bool fwd, float *xT, bool adj = false) {
#pragma unroll
        for (int j = 0; j < NXL; ++j) {
            const int gi = tid + j * kBwdThreads;
            if (gi >= V * P / 4) continue;
            const int v = gi % V, pc = 4 * (gi / V), i = v / R;
            const bool ok = v < VQ && i < Tc;
            float xv[4] = {0.f, 0.f, 0.f, 0.f}, gv[4];
            if (!adj) io4<IO>::unpack(qx[j], xv);
            if (!fwd) io4<IO>::unpack(qg[j], gv);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[q] = ok ? xv[q] : 0.f;
                gv[q] = ok && !fwd ? gv[q] : 0.f;
            }
            if (fwd) {
#pragma unroll
                for (int q = 0; q < 4; ++q) xT[(pc + q) * pV + v] = xv[q];
            } else {
                if (!adj) *reinterpret_cast<float4 *>(XN + v * pP + pc) = make_float4(xv[0], xv[1], xv[2], xv[3]);
                *reinterpret_cast<float4 *>(GN + v * pP + pc) = make_float4(gv[0], gv[1], gv[2], gv[3]);
#pragma unroll
                for (int q = 0; q < 4; ++q) T2[(pc + q) * pV + v] = gv[q];
            }
        }
    };
    // the factor of row 16 kb + 4 lg + e of this lane's k-slots, per step
    auto row_factor = [&](int s, float (&f)[VB][4]) {
#pragma unroll
        for (int kb = 0; kb < VB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[kb][e] = sc(s, row_tok(kb * 16 + 4 * lg + e));
    };

    // element (n, pc) of R(-phi) M for a [N][P] matrix M (rows 2k, 2k+1 rotated
    // by the angle of pair k)
    auto rot_el = [&](const float *M, int n, int pc, double phi) {
        float sn, cs;
        sincos_wrapped(wrap_angle(phi), &sn, &cs);
        const float u = M[(n & ~1) * P + pc], v = M[(n | 1) * P + pc];
        return (n & 1) ? cs * v - sn * u : cs * u + sn * v;
    };
    // the angle Phi before segment sg's first chunk: Phi_{-1} plus the
    // summed theta of the segments before it
    auto phi_start = [&](int k, int upto) { // upto: pieces
        double a = p.has_init ? double(p.phi0[bh * K + k]) : 0.0;
        for (int s2 = 0; s2 < upto; ++s2) a += p.segTh[(int64_t(bh) * NPC + s2) * K + k];
        return a;
    };

    if (role == 2) {
        // ===================== adjoint aggregate of segment sg: the gradient
        // of the state before its first chunk from the segment's own outputs,
        // with zero gradient after its last chunk, in the frame of its start:
        //   G = sum_c (prod_{c' < c} e^{ec_end(c')}) C~_c^T diag(E_c) gy_c,
        // accumulated in chunk order (G1 layout, second wave group)
        floatx4 Ga[NBW][PB];
#pragma unroll
        for (int q = 0; q < NBW; ++q)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) Ga[q][pb] = zero4();
        float lsum = 0.f;
        if (tid < K) PHE[tid] = 0.0;
        if (c0 < c1) issue(int64_t(c0) * Q, int(min<int64_t>(T - int64_t(c0) * Q, Q)), true, true);
        __syncthreads();
        for (int c = c0; c < c1; ++c) {
            lane_ids();
            const int64_t t0 = int64_t(c) * Q;
            const int Tc = int(min<int64_t>(T - t0, Q));
            stage_scalars(t0, Tc);
            stage_angles(Tc, true, c, false);
            stage_xg(Tc, false, nullptr, true);
            __syncthreads();
            rot_store(qc, Tc, CT, nullptr);
            const float dec = __expf(lsum);
            lsum += sc(Cf::s_ec, Q - 1);
            float ev[VB][4];
            row_factor(Cf::s_E, ev);
            __syncthreads();
            if (c + 1 < c1) issue(t0 + Q, int(min<int64_t>(T - t0 - Q, Q)), true, true);
            if (w >= 4) {
                const int wb = w - 4;
#pragma unroll
                for (int kb = 0; kb < VB; ++kb) {
                    floatx4 bc[NBW], ag[PB];
#pragma unroll
                    for (int q = 0; q < NBW; ++q)
                        if (wb + 4 * q < NB) bc[q] = lds4(CT + ((wb + 4 * q) * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) ag[pb] = lds4(T2 + (pb * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int q = 0; q < NBW; ++q) {
                            if (wb + 4 * q >= NB) continue;
                            const float bq = bc[q][e] * (ev[kb][e] * dec);
#pragma unroll
                            for (int pb = 0; pb < PB; ++pb) Ga[q][pb] = mfma4(ag[pb][e], bq, Ga[q][pb]);
                        }
                }
            }
            __syncthreads();
        }
        if (w >= 4) {
            const int wb = w - 4;
            float *out = p.segGa + bp * int64_t(N) * P;
#pragma unroll
            for (int q = 0; q < NBW; ++q) {
                const int nb = wb + 4 * q;
                if (nb >= NB) continue;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    *reinterpret_cast<floatx4 *>(out + (nb * 16 + li) * P + pb * 16 + 4 * lg) = Ga[q][pb];
            }
        }
        // the last segment's pieces record their sums (the other pieces' come
        // from role 1)
        if (sg == S - 1) {
            if (tid == 0) p.segg[bp] = lsum;
            if (tid < K) p.segTh[bp * K + tid] = PHE[tid];
        }
        return;
    }

    // ===================== forward sweep: H_c and Phi at each chunk start
    // Hf: transposed tiles (pb, nb = w + 8 q) of H_c; element e of lane
    // (li, lg) is H[nb*16 + li][pb*16 + 4 lg + e] (the layout of G in the
    // second wave group below).
    floatx4 Hf[NBH][PB];
    {
        // the state entering the segment: at the sequence start the carried
        // state with its pending term; later, the aggregates of the segments
        // before it folded in, H <- e^{g} H + R(-Phi_start) A (role 1 starts
        // from zero in the frame of its own start)
        const float d0 = io<IO>::get(dtg + tok(0)), l0 = io<IO>::get(lmg + tok(0));
        const float dl0 = (1.f - l0) * d0;
#pragma unroll
        for (int q = 0; q < NBH; ++q)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                Hf[q][pb] = zero4();
                const int nb = w + kBwdWaves * q;
                if (nb >= NB || role != 0) continue;
                const int n = nb * 16 + li, pc = pb * 16 + 4 * lg;
                float hh[4] = {0.f, 0.f, 0.f, 0.f};
                if (p.has_init) {
                    const float4 hv = *reinterpret_cast<const float4 *>(p.h0 + (bh * N + n) * int64_t(P) + pc);
                    hh[0] = hv.x; hh[1] = hv.y; hh[2] = hv.z; hh[3] = hv.w;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float bb = dl0 * p.prevB0[(bh * R + r) * N + n];
                        float xv[4];
                        io<IO>::load4(static_cast<const IO *>(p.prevx0) + (bh * R + r) * P + pc, xv);
#pragma unroll
                        for (int e = 0; e < 4; ++e) hh[e] += bb * xv[e];
                    }
                }
                if (sg > 0) {
                    double ph = p.has_init ? double(p.phi0[bh * K + (n >> 1)]) : 0.0;
                    for (int s2 = 0; s2 < sg * KA; ++s2) {
                        const int64_t o = int64_t(bh) * NPC + s2;
                        const float eg = __expf(p.segg[o]);
                        const float *A = p.segA + o * int64_t(N) * P;
#pragma unroll
                        for (int e = 0; e < 4; ++e) hh[e] = eg * hh[e] + rot_el(A, n, pc + e, ph);
                        ph += p.segTh[o * K + (n >> 1)];
                    }
                }
                Hf[q][pb] = floatx4{hh[0], hh[1], hh[2], hh[3]};
            }
        if (tid < K) PHE[tid] = role == 0 ? phi_start(tid, sg * KA) : 0.0;
    }
    float gsum = 0.f; // role 1: summed log decay of the segment
    if (c0 < c1) issue(int64_t(c0) * Q, int(min<int64_t>(T - int64_t(c0) * Q, Q)), false, false);
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
        lane_ids();
        const int64_t t0 = int64_t(c) * Q;
        const int Tc = int(min<int64_t>(T - t0, Q));
        if (role == 0) {
#pragma unroll
            for (int q = 0; q < NBH; ++q)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    if (w + kBwdWaves * q < NB) *reinterpret_cast<floatx4 *>(ck_at(c, w + kBwdWaves * q, pb)) = Hf[q][pb];
        }
        stage_scalars(t0, Tc);
        stage_angles(Tc, true, c, role == 0);
        // x^T alternates between two buffers (T2 and the mask area, unused in
        // this sweep), so the next chunk's staging needs no barrier after
        // this chunk's update; the token factors are read before the second
        // barrier for the same reason
        float *xT = (c & 1) ? MS : T2;
        stage_xg(Tc, true, xT);
        __syncthreads();
        rot_store(qb, Tc, BT, nullptr);
        const float eE = sc(Cf::s_misc, 0);
        gsum += sc(Cf::s_ec, Q - 1);
        float uv[VB][4];
        row_factor(Cf::s_U, uv);
        __syncthreads();
        if (c + 1 < c1) issue(t0 + Q, int(min<int64_t>(T - t0 - Q, Q)), false, false);
        // H^T[p][n] <- e^{ec_end} H^T + sum_v x[v][p] U_v B~[v][n]
        {
#pragma unroll
            for (int q = 0; q < NBH; ++q)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) Hf[q][pb] *= eE;
#pragma unroll
            for (int kb = 0; kb < VB; ++kb) {
                floatx4 bv[NBH], av[PB];
#pragma unroll
                for (int q = 0; q < NBH; ++q)
                    if (w + kBwdWaves * q < NB) bv[q] = lds4(BT + ((w + kBwdWaves * q) * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) av[pb] = lds4(xT + (pb * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < NBH; ++q) {
                        if (w + kBwdWaves * q >= NB) continue;
                        const float bq = bv[q][e] * uv[kb][e];
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) Hf[q][pb] = mfma4(av[pb][e], bq, Hf[q][pb]);
                    }
            }
        }
    }
    __syncthreads(); // the backward sweep's staging reuses the LDS
    if (role == 1) {
        // forward aggregate of segment sg: its state at the end from zero (frame
        // of its start), summed log decay and summed angle
        float *out = p.segA + bp * int64_t(N) * P;
#pragma unroll
        for (int q = 0; q < NBH; ++q)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int nb = w + kBwdWaves * q;
                if (nb < NB) *reinterpret_cast<floatx4 *>(out + (nb * 16 + li) * P + pb * 16 + 4 * lg) = Hf[q][pb];
            }
        if (tid == 0) p.segg[bp] = gsum;
        if (tid < K) p.segTh[bp * K + tid] = PHE[tid];
        return;
    }

    // ===================== backward sweep
    // G, the gradient of H_{c+1}, in registers GS: waves 0-3 hold G in tiles
    // (nb, pb = w), element e of lane (li, lg) = G[nb*16 + 4 lg + e][w*16 + li]
    // (G2 below); waves 4-7 hold it in Hf's transposed layout, tiles
    // (pb, nb = w - 4 + 4 q) (G1 below).
    floatx4 GS[GSN];
#pragma unroll
    for (int i = 0; i < GSN; ++i) GS[i] = zero4();
#define G2(nb) GS[nb]
#define G1(q, pb) GS[(q) * PB + (pb)]
    // after the last chunk G is the incoming gradient of the final h~ (the
    // last token has no next token, so H after the last chunk is h~_{T-1});
    // after an earlier segment's last chunk it is that gradient carried back
    // through the later segments, folded from their adjoint aggregates:
    // G <- e^{g} G + R(-Phi_start) Ga, last segment first
    if (sg < S - 1) {
        auto gend = [&](int n, int pc) {
            float v = p.ghT ? p.ghT[(bh * N + n) * int64_t(P) + pc] : 0.f;
            double ph = phi_start(n >> 1, NPC - 1);
            for (int s2 = NPC - 1; s2 >= (sg + 1) * KA; --s2) {
                const int64_t o = int64_t(bh) * NPC + s2;
                v = __expf(p.segg[o]) * v + rot_el(p.segGa + o * int64_t(N) * P, n, pc, ph);
                ph -= p.segTh[(o - 1) * K + (n >> 1)];
            }
            return v;
        };
        if (w < 4 && w < PB) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) G2(nb)[e] = gend(nb * 16 + 4 * lg + e, w * 16 + li);
        } else if (w >= 4) {
#pragma unroll
            for (int q = 0; q < NBW; ++q) {
                const int nb = w - 4 + 4 * q;
                if (nb >= NB) continue;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) G1(q, pb)[e] = gend(nb * 16 + li, pb * 16 + 4 * lg + e);
            }
        }
    } else if (p.ghT) {
        const float *gh = p.ghT + bh * int64_t(N) * P;
        if (w < 4 && w < PB) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) G2(nb)[e] = gh[(nb * 16 + 4 * lg + e) * P + w * 16 + li];
        } else if (w >= 4) {
#pragma unroll
            for (int q = 0; q < NBW; ++q) {
                const int nb = w - 4 + 4 * q;
                if (nb >= NB) continue;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    G1(q, pb) = lds4(gh + (nb * 16 + li) * P + pb * 16 + 4 * lg);
            }
        }
    }
    double carry[KP];    // lanes (pair, segment): sum of dPhi over the later chunks
    double carry0[KP];   // its value at the segment's end
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
        // the final Phi_T = Phi_{-1} + sum theta: its incoming gradient adds
        // to every dtheta_t and to dPhi_{-1}.  An earlier segment starts from
        // zero; the later segments' sums are added to its dtheta afterwards.
        const int k = KS * kp + 8 * w + (lane & 7);
        carry[kp] = p.gphiT && k < K && sg == S - 1 ? double(p.gphiT[bh * K + k]) : 0.0;
        carry0[kp] = carry[kp];
    }
    float gA = 0.f;      // wave 0: this lane's share of dA
    bool pend = false;   // wave 0, lane 0: the later chunk's first token awaits its d(delta)
    float pd_g = 0.f, pd_l = 0.f, pd_dt = 0.f, pd_lam = 0.f;
    int64_t pd_tok = 0;
    issue(int64_t(c1 - 1) * Q, int(min<int64_t>(T - int64_t(c1 - 1) * Q, Q)), true, false);
    for (int c = c1 - 1; c >= c0; --c) {
        lane_ids();
        const int64_t t0 = int64_t(c) * Q;
        const int Tc = int(min<int64_t>(T - t0, Q));
        stage_scalars(t0, Tc);
        stage_angles(Tc, false, c, false);
        stage_xg(Tc, false, nullptr);
        // H_c (the second group's tiles), in flight during the staging
        const int wb = w - 4; // wave index in the second group
        floatx4 hq[NBW][PB];
#pragma unroll
        for (int q = 0; q < NBW; ++q)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
                hq[q][pb] = w >= 4 && wb + 4 * q < NB ? *reinterpret_cast<const floatx4 *>(ck_at(c, wb + 4 * q, pb)) : zero4();
        __syncthreads();
        // ---- rotate; the table of e^{ec_i - ec_j}
        for (int idx = tid; idx < QP * QP; idx += kBwdThreads) {
            const int i = idx / QP, j = idx - i * QP;
            ET[i * pQ + j] = i >= j ? __expf(sc(Cf::s_ec, i) - sc(Cf::s_ec, j)) : 0.f;
        }
        rot_store(qb, Tc, BT, BN);
        rot_store(qc, Tc, CT, CN);
        __syncthreads();
        // ---- S = C~ B~^T and D = gy x^T, one 16 x 16 tile per wave of the
        // first group; masks.  The second group meanwhile starts dC~ and dB~
        // with gy H_c^T and x G^T (nothing of this phase needed), their row
        // dots with C~ and B~ (the partial sums of dE and dU) and <G, H_c>.
        floatx4 dcq[NBW][VB], dbq[NBW][VB];
        float pe[VB][4], pu[VB][4];
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
#pragma unroll
            for (int e = 0; e < 4; ++e) pe[vb][e] = pu[vb][e] = 0.f;
        float pz = 0.f;
        if (w >= 4) {
#pragma unroll
            for (int q = 0; q < NBW; ++q) {
                const int nb = wb + 4 * q;
                if (nb >= NB) continue;
                floatx4 (&dc)[VB] = dcq[q], (&db)[VB] = dbq[q];
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) dc[vb] = db[vb] = zero4();
                {
                    floatx4 ag[2][VB], ax[2][VB];
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        ag[0][vb] = lds4(GN + (vb * 16 + li) * pP + 4 * lg);
                        ax[0][vb] = lds4(XN + (vb * 16 + li) * pP + 4 * lg);
                    }
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const int cu = pb & 1, nx = cu ^ 1;
                        if (pb + 1 < PB)
#pragma unroll
                            for (int vb = 0; vb < VB; ++vb) {
                                ag[nx][vb] = lds4(GN + (vb * 16 + li) * pP + (pb + 1) * 16 + 4 * lg);
                                ax[nx][vb] = lds4(XN + (vb * 16 + li) * pP + (pb + 1) * 16 + 4 * lg);
                            }
#pragma unroll
                        for (int e = 0; e < 4; ++e)
#pragma unroll
                            for (int vb = 0; vb < VB; ++vb) {
                                dc[vb] = mfma4(ag[cu][vb][e], hq[q][pb][e], dc[vb]);
                                db[vb] = mfma4(ax[cu][vb][e], G1(q, pb)[e], db[vb]);
                            }
                    }
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * VB, 0);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        if (pb + 1 < PB) __builtin_amdgcn_sched_group_barrier(0x100, 2 * VB, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 8 * VB, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = vb * 16 + 4 * lg + e, n = nb * 16 + li, ti = row_tok(v);
                        pe[vb][e] += dc[vb][e] * CN[v * pN + n];
                        pu[vb][e] += db[vb][e] * BN[v * pN + n];
                        dc[vb][e] *= sc(Cf::s_E, ti);
                        db[vb][e] *= sc(Cf::s_U, ti);
                    }
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) pz += G1(q, pb)[e] * hq[q][pb][e];
            }
        }
        if (w < 4) {
            const int vb = w >> 1, vb2 = w & 1;
            floatx4 S[1] = {zero4()}, D[1] = {zero4()};
            if (!(Cf::TRI && vb == 0 && vb2 == 1)) { // that tile is masked out entirely
                mm_lds<N, pN, pN, 1>(S, CN + vb * 16 * pN, BN + vb2 * 16 * pN, li, lg);
                mm_lds<P, pP, pP, 1>(D, GN + vb * 16 * pP, XN + vb2 * 16 * pP, li, lg);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = vb * 16 + 4 * lg + e, v2 = vb2 * 16 + li;
                const int ti = row_tok(v), tj = row_tok(v2);
                const float wgt =
                    ti >= tj ? ET[ti * pQ + tj] * (sc(Cf::s_g, tj) + (ti > tj ? sc(Cf::s_dn, tj) : 0.f)) : 0.f;
                MS[v2 * pV + v] = wgt * S[0][e];
                MN[v * pV + v2] = wgt * D[0][e];
                MT[v2 * pV + v] = wgt * D[0][e];
                SD[v * pV + v2] = S[0][e] * D[0][e];
            }
        }
        __syncthreads();
        // the previous chunk's inputs, in flight during the products (the first
        // group, whose products are fewer, prefetches now, the second after its
        // products)
        if (c > c0 && w < 4) issue(t0 - Q, Q, true, false);
        // ---- per token j (8 threads each): row sums of dW.W and column sums
        // of dW.e^{ec_i - ec_j} off the diagonal, and dW(j, j); dW(i, j) is
        // the sum of S.D over the R x R block of the token pair
        {
            constexpr int QC = (Q + 7) / 8;
            const int r0 = tid >> 3, ch = tid & 7;
            auto dWf = [&](int i, int j) {
                float s = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int r2 = 0; r2 < R; ++r2) s += SD[(i * R + r) * pV + j * R + r2];
                return s;
            };
            float rw = 0.f, ce = 0.f, dg = 0.f;
            if (r0 < Q)
#pragma unroll
                for (int u = 0; u < QC; ++u) {
                    const int j = ch * QC + u;
                    if (j >= Q) continue;
                    if (j < r0) rw += dWf(r0, j) * ET[r0 * pQ + j] * (sc(Cf::s_g, j) + sc(Cf::s_dn, j));
                    if (j > r0) ce += dWf(j, r0) * ET[j * pQ + r0];
                    if (j == r0) dg = dWf(r0, r0);
                }
            rw = row_sum<8>(rw);
            ce = row_sum<8>(ce);
            dg = row_sum<8>(dg);
            if (ch == 0 && r0 < Q) {
                DW[r0] = rw;
                DW[pQ + r0] = ce;
                DW[2 * pQ + r0] = dg;
            }
        }
        // ---- the six products; the gradient of H_c.  Outputs of token
        // t0 + i, rank r are addressed as the chunk's base + a 32-bit offset.
        const int64_t tb0 = tok(t0);
        const int HR = p.H * R;
        float *gxb = p.gx + tb0 * (R * P), *gBb = p.gB + tb0 * (R * N), *gCb = p.gC + tb0 * (R * N);
        const float eE = sc(Cf::s_misc, 0);
        float ev[VB][4];
        row_factor(Cf::s_E, ev);
        // dx = (W.S)^T gy + diag(U) B~ G   (tiles (vb, pb = w))
        if (w < PB) {
            const int pb = w;
            floatx4 acc[VB];
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) acc[vb] = zero4();
            {
                floatx4 av[2][VB];
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) av[0][vb] = lds4(BN + (vb * 16 + li) * pN + 4 * lg);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int cu = nb & 1, nx = cu ^ 1;
                    if (nb + 1 < NB)
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) av[nx][vb] = lds4(BN + (vb * 16 + li) * pN + (nb + 1) * 16 + 4 * lg);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) acc[vb] = mfma4(av[cu][vb][e], G2(nb)[e], acc[vb]);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, VB, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (nb + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x100, VB, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 4 * VB, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[vb][e] *= sc(Cf::s_U, row_tok(vb * 16 + 4 * lg + e));
            mm_lds<V, pV, pV, VB, ZLO, 0>(acc, MS, T2 + pb * 16 * pV, li, lg);
#pragma unroll
            for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = vb * 16 + 4 * lg + e, i = v / R;
                    // the last token's x is the final state's x_prev
                    float gx = acc[vb][e];
                    if (p.gxpT && t0 + i == T - 1 && v < VQ)
                        gx += p.gxpT[(bh * R + (v - i * R)) * P + pb * 16 + li];
                    if (v < VQ && i < Tc) gxb[(i * HR + v - i * R) * P + pb * 16 + li] = gx;
                }
            // G <- e^{ec_end} G + C~^T diag(E) gy  (this orientation)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) G2(nb) *= eE;
#pragma unroll
            for (int kb = 0; kb < VB; ++kb) {
                const floatx4 bq = lds4(T2 + (pb * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const floatx4 aq = lds4(CT + (nb * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
                    for (int e = 0; e < 4; ++e) G2(nb) = mfma4(aq[e], bq[e] * ev[kb][e], G2(nb));
                }
            }
            if constexpr (Cf::GX) {
                // the updated G for the second group (read after the barrier)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) gx_row(nb * 16 + 4 * lg + e)[w * 16 + li] = G2(nb)[e];
            }
        }
        // dC~ and dB~ (tiles (vb, nb = w + 4 q)) completed, rotated back; dPhi terms
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int nb = wb + 4 * q;
            if (w < 4 || nb >= NB) continue;
            floatx4 (&dc)[VB] = dcq[q], (&db)[VB] = dbq[q];
            mm_lds<V, pV, pV, VB, ZHI, 1>(dc, MN, BT + nb * 16 * pV, li, lg);
            mm_lds<V, pV, pV, VB, ZLO, 0>(db, MT, CT + nb * 16 * pV, li, lg);
            // the last token's B~ is the final state's prev_B
            if (p.gBpT && t0 + Tc == T) {
#pragma unroll
                for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = vb * 16 + 4 * lg + e, i = v / R;
                        if (v < VQ && i == Tc - 1)
                            db[vb][e] += p.gBpT[(bh * R + (v - i * R)) * N + nb * 16 + li];
                    }
            }
#pragma unroll
            for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = vb * 16 + 4 * lg + e, n = nb * 16 + li, i = v / R;
                    // the even lane of each row pair takes its partner's
                    // values and writes both rotated outputs (8 bytes)
                    const float b1 = dpp_f32<0xb1>(db[vb][e]), c1 = dpp_f32<0xb1>(dc[vb][e]); // lane ^ 1
                    if (!(n & 1)) {
                        const float b0 = db[vb][e], c0 = dc[vb][e];
                        const float2 cz = CS[min(i, Q - 1) * pC + (n >> 1)];
                        if (v < VQ && i < Tc) {
                            const int o = (i * HR + v - i * R) * N + n;
                            *reinterpret_cast<float2 *>(gBb + o) = make_float2(cz.x * b0 - cz.y * b1, cz.y * b0 + cz.x * b1);
                            *reinterpret_cast<float2 *>(gCb + o) = make_float2(cz.x * c0 - cz.y * c1, cz.y * c0 + cz.x * c1);
                        }
                        const float2 bt = *reinterpret_cast<const float2 *>(BN + v * pN + n);
                        const float2 ct = *reinterpret_cast<const float2 *>(CN + v * pN + n);
                        PH[v * pK + (n >> 1)] = b0 * bt.y - b1 * bt.x + c0 * ct.y - c1 * ct.x;
                    }
                }
        }
        // G <- e^{ec_end} G + C~^T diag(E) gy  (the transposed orientation;
        // with GX or GA reloaded from the first group's after the barrier)
        if (w >= 4) {
        if constexpr (!Cf::GX && !Cf::GA) {
#pragma unroll
        for (int q = 0; q < NBW; ++q)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) G1(q, pb) *= eE;
#pragma unroll
        for (int kb = 0; kb < VB; ++kb) {
            floatx4 bc[NBW], ag[PB];
#pragma unroll
            for (int q = 0; q < NBW; ++q)
                if (wb + 4 * q < NB) bc[q] = lds4(CT + ((wb + 4 * q) * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) ag[pb] = lds4(T2 + (pb * 16 + li) * pV + 16 * kb + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    if (wb + 4 * q >= NB) continue;
                    const float bq = bc[q][e] * ev[kb][e];
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) G1(q, pb) = mfma4(ag[pb][e], bq, G1(q, pb));
                }
        }
        }
        // per-row partial sums of dE and dU over this wave's columns
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float se = row_sum<16>(pe[vb][e]), su = row_sum<16>(pu[vb][e]);
                if (li == 0) {
                    PE[wb * V + vb * 16 + 4 * lg + e] = se;
                    PU[wb * V + vb * 16 + 4 * lg + e] = su;
                }
            }
        pz = row_sum<16>(pz);
        pz += __shfl_xor(pz, 16);
        pz += __shfl_xor(pz, 32);
        if (lane == 0) PZ[wb * 4] = pz;
        if (c > c0) issue(t0 - Q, Q, true, false);
        }
        __syncthreads();
        if constexpr (Cf::GA) {
            // every read of the areas G borrows is behind this chunk's
            // products; the next writes are the next chunk's staging
            if (w < 4 && w < PB) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) gx_row(nb * 16 + 4 * lg + e)[w * 16 + li] = G2(nb)[e];
            }
            __syncthreads();
        }
        if constexpr (Cf::GX || Cf::GA) {
            // the second group's G tiles (pb, nb = w - 4 + 4 q) from the first
            // group's update; the buffer is next written a chunk later, after
            // further barriers
            if (w >= 4) {
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    const int nb = w - 4 + 4 * q;
                    if (nb >= NB) continue;
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) G1(q, pb) = lds4(gx_row(nb * 16 + li) + pb * 16 + 4 * lg);
                }
            }
        }
        // ---- the scalars (wave 0, lane = token)
        if (w == 0) {
            const int j = lane;
            const bool tj = j < Q;
            const int js = tj ? j : Q;
            float dEj = 0.f, dUj = 0.f;
            if (tj)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) {
                        dEj += PE[ww * V + j * R + r];
                        dUj += PU[ww * V + j * R + r];
                    }
            const float rowW = tj ? DW[j] : 0.f, colE = tj ? DW[pQ + j] : 0.f, dgj = tj ? DW[2 * pQ + j] : 0.f;
            const float Ej = sc(Cf::s_E, js), EUj = sc(Cf::s_EU, js), Uj = sc(Cf::s_U, js);
            const float gd = sc(Cf::s_g, js) + sc(Cf::s_dn, js);
            const float dgam = dgj + colE + dUj * EUj;
            const float ddn = colE + dUj * EUj;
            float dec = rowW - colE * gd + dEj * Ej - dUj * Uj;
            auto last = [](float x) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1)); };
            const float uu = last(wave_scan_dpp(dUj * Uj));
            if (j == Tc - 1) dec += uu + (PZ[0] + PZ[4] + PZ[8] + PZ[12]) * sc(Cf::s_misc, 0);
            const float incl = wave_scan_dpp(dec);
            const float dl = last(incl) - incl + dec;
            const float dd = __shfl_up(ddn, 1);
            const float ddLast = __shfl(ddn, Q - 1);
            const float dtj = sc(Cf::s_dt, js), lmj = sc(Cf::s_lam, js);
            if (j >= 1 && j < Tc) {
                const int64_t o = tok(t0 + j);
                p.gdt[o] = dgam * lmj + dd * (1.f - lmj) + dl * Ah;
                p.glam[o] = (dgam - dd) * dtj;
            }
            if (j < Tc) gA += dl * dtj;
            // the last chunk of an earlier segment: the gradient of the next
            // segment's first delta, added to that token's dt, lam afterwards
            if (j == 0 && c == c1 - 1 && sg < S - 1) p.segdd[bs + 1] = ddLast;
            if (j == 0) {
                if (pend) {
                    p.gdt[pd_tok] = pd_g * pd_lam + ddLast * (1.f - pd_lam) + pd_l * Ah;
                    p.glam[pd_tok] = (pd_g - ddLast) * pd_dt;
                }
                pend = true;
                pd_g = dgam; pd_l = dl; pd_dt = dtj; pd_lam = lmj; pd_tok = tok(t0);
            }
        }
        // ---- dtheta_t = carry + the suffix sum of dPhi over the chunk (every
        // wave: lane = 8 segments x 8 pairs, segment totals scanned over lanes
        // 8 apart, fp64)
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
            const int k = KS * kp + 8 * w + (lane & 7), seg = lane >> 3;
            const bool kv = k < K;
            const int kc = kv ? k : 0;
            double ls[TPS];
            double run = 0.0;
#pragma unroll
            for (int u = TPS - 1; u >= 0; --u) {
                const int i = seg * TPS + u;
                float s = 0.f;
                if (i < Tc)
#pragma unroll
                    for (int r = 0; r < R; ++r) s += PH[(i * R + r) * pK + kc];
                run += double(s);
                ls[u] = run;
            }
            double x = run;
#pragma unroll
            for (int o = 8; o < kWave; o <<= 1) {
                const double y = __shfl_down(x, o, kWave);
                if (lane + o < kWave) x += y;
            }
            const double ex = x - run;
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int i = seg * TPS + u;
                if (kv && i < Tc) p.gtheta[tb0 * K + (i * p.H * K + k)] = float(carry[kp] + ex + ls[u]);
            }
            carry[kp] += __shfl(x, lane & 7, kWave);
        }
        __syncthreads();
    }

    // ===================== the segment's summed dPhi (the later segments'
    // sums are added to an earlier segment's dtheta afterwards)
    lane_ids();
    if (S > 1 && lane < 8)
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
            const int k = KS * kp + 8 * w + lane;
            if (k < K) p.segDphi[bs * K + k] = carry[kp] - carry0[kp];
        }
    // ===================== the carried state (G is now the gradient of H_0)
    float dd0 = 0.f;
    if (p.has_init && sg == 0) {
        const float d0 = io<IO>::get(dtg + tok(0)), l0 = io<IO>::get(lmg + tok(0));
        const float dl0 = (1.f - l0) * d0;
        // from G2 (columns p = w*16 + li): dx_{-1} and the gradient of d_0
        float part = 0.f;
        if (w < PB) {
            const int pc = w * 16 + li;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float xr = io<IO>::get(static_cast<const IO *>(p.prevx0) + (bh * R + r) * P + pc);
                float s = 0.f;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += p.prevB0[(bh * R + r) * N + nb * 16 + 4 * lg + e] * G2(nb)[e];
                s += __shfl_xor(s, 16);
                s += __shfl_xor(s, 32);
                if (lg == 0 && p.gprevx0) p.gprevx0[(bh * R + r) * P + pc] = dl0 * s;
                part += lg == 0 ? s * xr : 0.f;
            }
        }
        part = row_sum<16>(part);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (lane == 0 && w < 4) PZ[w * 4 + 1] = part;
        // from G1 (rows n = nb*16 + li): dh~_{-1} and dB~_{-1}
        const int wb = w - 4;
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int nb = wb + 4 * q;
            if (w < 4 || nb >= NB) continue;
            const int n = nb * 16 + li;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
                if (p.gh0)
                    *reinterpret_cast<float4 *>(p.gh0 + (bh * N + n) * int64_t(P) + pb * 16 + 4 * lg) =
                        make_float4(G1(q, pb)[0], G1(q, pb)[1], G1(q, pb)[2], G1(q, pb)[3]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float s = 0.f;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    float xv[4];
                    io<IO>::load4(static_cast<const IO *>(p.prevx0) + (bh * R + r) * P + pb * 16 + 4 * lg, xv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += G1(q, pb)[e] * xv[e];
                }
                s += __shfl_xor(s, 16);
                s += __shfl_xor(s, 32);
                if (lg == 0 && p.gprevB0) p.gprevB0[(bh * R + r) * N + n] = dl0 * s;
            }
        }
        if (p.gphi0 && S == 1)
#pragma unroll
            for (int kp = 0; kp < KP; ++kp) {
                const int k = KS * kp + 8 * w + lane;
                if (lane < 8 && k < K) p.gphi0[bh * K + k] = float(carry[kp]);
            }
        __syncthreads();
        dd0 = PZ[1] + PZ[5] + PZ[9] + PZ[13];
    }
    if (w == 0) {
        if (lane == 0 && pend) {
            p.gdt[pd_tok] = pd_g * pd_lam + dd0 * (1.f - pd_lam) + pd_l * Ah;
            p.glam[pd_tok] = (pd_g - dd0) * pd_dt;
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) gA += __shfl_xor(gA, o);
        if (lane == 0) p.gA_part[bs] = gA;
    }
#undef G1
#undef G2
}

// Sum of the per-(batch, head, segment) partials of dA over batch and segments.
static __global__ void k_backward_gA(const BwdParams p) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= p.H) return;
    float s = 0.f;
    for (int64_t b = 0; b < p.batch; ++b)
        for (int sg = 0; sg < p.S; ++sg) s += p.gA_part[(b * p.H + h) * p.S + sg];
    p.gA[h] = s;
}

// Split sequences, after the segments' gradients: per (b, h, segment sg),
// kFixParts workgroups each taking a share of the segment's tokens:
//  * dtheta of every token of an earlier segment += dPhi_T's gradient plus
//    the summed dPhi of the later segments (the suffix sums the segment began
//    at zero), the K carries computed once into LDS;
//  * the first token of a later segment: the gradient of its delta from the
//    segment before (delta = (1 - lam) dt) into its dt and lam;
//  * dPhi_{-1} = dPhi_T's gradient plus every segment's sum (segment 0).
constexpr int kFixParts = 8;
template <typename IO>
__global__ __launch_bounds__(256) void k_backward_fix(const BwdParams p) {
    __shared__ float carry[128]; // K <= 64
    const int S = p.S, K = p.K;
    const int part = int(blockIdx.x % kFixParts);
    const int64_t bs = blockIdx.x / kFixParts;
    const int64_t bh = bs / S;
    const int sg = int(bs % S);
    const int h = int(bh % p.H);
    const int64_t b = bh / p.H;
    const int Q = kBwdV / p.R;
    const int64_t t0 = int64_t(sg) * p.cps * Q, t1 = min<int64_t>(p.T, t0 + int64_t(p.cps) * Q);
    auto carry_from = [&](int k, int first) {
        double a = p.gphiT ? double(p.gphiT[bh * K + k]) : 0.0;
        for (int s2 = first; s2 < S; ++s2) a += p.segDphi[(bh * S + s2) * K + k];
        return a;
    };
    if (sg < S - 1) {
        for (int k = threadIdx.x; k < K; k += blockDim.x) carry[k] = float(carry_from(k, sg + 1));
        __syncthreads();
        // this part's tokens; rows of K floats, float4 along k (K % 8 == 0)
        const int64_t nt = t1 - t0, per = (nt + kFixParts - 1) / kFixParts;
        const int64_t ta = t0 + part * per, tb = min(t1, ta + per);
        const int K4 = K / 4;
        for (int64_t i = threadIdx.x; i < (tb - ta) * K4; i += blockDim.x) {
            const int64_t t = ta + i / K4;
            const int k = 4 * int(i % K4);
            float4 *g = reinterpret_cast<float4 *>(p.gtheta + ((b * p.T + t) * p.H + h) * K + k);
            float4 v = *g;
            v.x += carry[k]; v.y += carry[k + 1]; v.z += carry[k + 2]; v.w += carry[k + 3];
            *g = v;
        }
    }
    if (part == 0 && sg > 0 && threadIdx.x == 0) {
        const int64_t o = (b * p.T + t0) * p.H + h;
        const float dd = p.segdd[bh * S + sg];
        const float dtv = io<IO>::get(static_cast<const IO *>(p.dt) + o);
        const float lmv = io<IO>::get(static_cast<const IO *>(p.lam) + o);
        p.gdt[o] += dd * (1.f - lmv);
        p.glam[o] -= dd * dtv;
    }
    if (part == 0 && sg == 0 && p.has_init && p.gphi0)
        for (int k = threadIdx.x; k < K; k += blockDim.x) p.gphi0[bh * K + k] = float(carry_from(k, 0));
}

template <typename IO, int N, int P, int R>
hipError_t launch_backward_inst(const BwdParams &p, hipStream_t s) {
    typedef BwdCfg<N, P, R> Cf;
    if (Cf::bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_backward<IO, N, P, R>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(Cf::bytes));
        if (e != hipSuccess) return e;
    }
    const int64_t nbh = p.batch * p.H;
    hipError_t e;
    if (p.S > 1) {
        // segment aggregates: forward state of segments 0 .. S-2, adjoint of 1 .. S-1
        BwdParams pa = p;
        pa.mode = 1;
        hipLaunchKernelGGL((k_backward<IO, N, P, R>), dim3(unsigned(2 * (p.S - 1) * p.kagg * nbh)), dim3(kBwdThreads), Cf::bytes,
                           s, pa);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    BwdParams pm = p;
    pm.mode = 0;
    hipLaunchKernelGGL((k_backward<IO, N, P, R>), dim3(unsigned(p.S * nbh)), dim3(kBwdThreads), Cf::bytes, s, pm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.S > 1) {
        hipLaunchKernelGGL((k_backward_fix<IO>), dim3(unsigned(p.S * nbh * kFixParts)), dim3(256), 0, s, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
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
