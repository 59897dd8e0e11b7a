// k_chunk_output.hip -- outputs of one chunk: the intra-chunk masked
// contraction plus the contribution of the incoming state (MFMA).
//
// With virtual rows t = (token tt, output channel i) and s = (token ts,
// input channel r) of the chunk (MIMO, Mamba-3 review section 3.3), the
// rotated operands Chat = R(-phi_loc) C, Bhat = R(-phi_loc) B (RoPE form,
// section 3.2.2, Prop. 3.2.3, relative to the chunk start) and the state H
// entering the chunk (in the frame of the chunk start):
//     S[t][s]  = Chat[t] . Bhat[s]                       (C B^T of section 2.3)
//     M[t][s]  = S[t][s] * Lmask(tt, ts)
//     Lmask    = gam_tt                        if ts == tt
//              = exp(ell_tt - ell_ts) wgt_ts   if ts <  tt
//              = 0                             if ts >  tt
//     y[t][p]  = sum_s M[t][s] x[s][p] + exp(ell_tt) sum_n Chat[t][n] H[n][p]
// Lmask is the decay matrix times the 2-band matrix of section 3.1.3,
// eq. (7) (closed form, every factor <= 1), repeated over the R x R channel
// block of each token pair.  This is the chunkwise SSD algorithm (the
// "20.2 Mamba and S6" page, section 2: intra-chunk by matrix products,
// inter-chunk through the passed state).
//
// One workgroup of 256 threads per (b, h, c).  Bhat (row-major), x and H
// (transposed) sit in LDS; Chat rows of the wave's 16-row blocks stay in
// registers, where they serve both as the B operand of S^T = Bhat Chat^T and
// as the A operand of Chat H.  S^T is computed per 16 x 16 block so that its
// accumulator layout (lane = column t, four consecutive s per lane group)
// directly forms the A operand of M x with a matching permutation of the
// s-slots on the x side.  Blocks above the diagonal are skipped.
#include "m3_chunk.hpp"

namespace m3 {

template <typename IO, int N, int P>
struct ChunkOutputLds {
    typedef typename Mma<mode<IO>::f32>::lds_t lds_t;
    static constexpr int K = N / 2, KP = K + 1;
    static constexpr int PADE = 16 / int(sizeof(lds_t));
    static constexpr int NBP = N + PADE; // pitch of Bhat rows and H^T rows
    static __host__ __device__ size_t vp(int R) { return size_t(kQ * R + PADE); }
    static constexpr size_t phi_bytes = size_t(kQ) * KP * sizeof(float);
    static constexpr size_t ht_bytes = size_t(P) * NBP * sizeof(lds_t);
    static constexpr size_t u_bytes = ((phi_bytes > ht_bytes ? phi_bytes : ht_bytes) + 15) / 16 * 16;
    static __host__ __device__ size_t off_u() { return 3 * kQ * sizeof(float); }
    static __host__ __device__ size_t off_bs() { return off_u() + u_bytes; }
    static __host__ __device__ size_t off_xt(int R) { return off_bs() + size_t(kQ * R) * NBP * sizeof(lds_t); }
    static __host__ __device__ size_t bytes(int R) { return off_xt(R) + size_t(P) * vp(R) * sizeof(lds_t); }
};

template <typename IO, int N, int P>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_output(const PrefillParams p) {
    typedef Mma<mode<IO>::f32> M;
    typedef typename M::frag frag;
    typedef typename M::lds_t lds_t;
    typedef ChunkOutputLds<IO, N, P> L;
    constexpr int K = N / 2, KP = K + 1;
    constexpr int NBP = L::NBP;
    constexpr int NKS = N >= 32 ? N / 32 : 1; // K-steps of 32 over the state rows
    constexpr int PT = P / 16;
    const int R = p.R, V = kQ * R;
    const int VP = int(L::vp(R));
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, l16 = lane & 15;
    const ChunkId id = chunk_id(p);

    extern __shared__ __align__(16) unsigned char smem[];
    float *ell_s = reinterpret_cast<float *>(smem);
    float *gam_s = ell_s + kQ;
    float *wgt_s = gam_s + kQ;
    float *phi_s = reinterpret_cast<float *>(smem + L::off_u());
    lds_t *ht = reinterpret_cast<lds_t *>(smem + L::off_u()); // aliases phi_s
    lds_t *bs = reinterpret_cast<lds_t *>(smem + L::off_bs());
    lds_t *xt = reinterpret_cast<lds_t *>(smem + L::off_xt(R));

    if (tid < kQ) {
        float e = 0.f, gm = 0.f, w = 0.f;
        if (tid < id.Tc) {
            const int64_t o = id.bh * p.T + id.t0 + tid;
            e = p.ell[o];
            gm = p.gam[o];
            w = p.wgt[o];
        }
        ell_s[tid] = e;
        gam_s[tid] = gm;
        wgt_s[tid] = w;
    }
    chunk_angles<IO, K>(p, id, phi_s, false); // contains the barriers

    // --- stage Bhat row-major, x transposed; Chat of this wave's blocks to registers
    const IO *Bsrc = static_cast<const IO *>(p.B);
    const IO *Csrc = static_cast<const IO *>(p.C);
    constexpr int NG = N / 8, PG = P / 8;
    for (int it = tid; it < V * NG; it += kThreads) {
        const int v = it / NG, q = it - v * NG;
        float r0[8];
        load_rotated8<IO, K>(p, id, Bsrc, phi_s, v, q, 1.f, r0);
        M::st8(&bs[v * NBP + 8 * q], r0);
    }
    for (int it = tid; it < (V / 2) * PG; it += kThreads) {
        const int vp2 = it / PG, q = it - vp2 * PG;
        const int v0 = 2 * vp2;
        float r0[8], r1[8];
        load_x8<IO>(p, id, v0, q, r0);
        load_x8<IO>(p, id, v0 + 1, q, r1);
#pragma unroll
        for (int j = 0; j < 8; ++j) M::st2(&xt[(8 * q + j) * VP + v0], r0[j], r1[j]);
    }

    // 16-row blocks of virtual rows, dealt to waves so that causal work balances.
    const int NTB = V / 16;
    int tbs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tbs[i] = 4 * i + ((i & 1) ? 3 - wave : wave);
    frag cf[4][NKS];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            cf[i][ks] = M::zero();
            const int n0 = 32 * ks + 8 * g;
            if (tbs[i] < NTB && n0 < N) {
                float r0[8];
                load_rotated8<IO, K>(p, id, Csrc, phi_s, 16 * tbs[i] + l16, n0 / 8, 1.f, r0);
                cf[i][ks] = M::pack(r0);
            }
        }
    }

    // incoming state of this chunk (fp32 [N][P]) -> registers, then H^T to LDS
    const float *Hin = p.ubuf + ((id.bh * p.nC + id.c) * int64_t(N)) * P;
    constexpr int HITEMS = (N / 2) * (P / 4);
    constexpr int HPT = (HITEMS + kThreads - 1) / kThreads;
    float4 hv0[HPT], hv1[HPT];
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        const int it = tid + j * kThreads;
        if (it < HITEMS) {
            const int np = it / (P / 4), p4 = it - np * (P / 4);
            hv0[j] = *reinterpret_cast<const float4 *>(Hin + (2 * np) * P + 4 * p4);
            hv1[j] = *reinterpret_cast<const float4 *>(Hin + (2 * np + 1) * P + 4 * p4);
        }
    }
    __syncthreads(); // phi_s is no longer read: its space becomes H^T
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        const int it = tid + j * kThreads;
        if (it < HITEMS) {
            const int np = it / (P / 4), p4 = it - np * (P / 4);
            const float a[4] = {hv0[j].x, hv0[j].y, hv0[j].z, hv0[j].w};
            const float b[4] = {hv1[j].x, hv1[j].y, hv1[j].z, hv1[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) M::st2(&ht[(4 * p4 + q) * NBP + 2 * np], a[q], b[q]);
        }
    }
    __syncthreads();

    IO *y = static_cast<IO *>(p.y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tb = tbs[i];
        if (tb >= NTB) continue;
        const int t0v = 16 * tb;
        if (t0v / R >= id.Tc) continue; // block holds only padding tokens
        const int tok_last = min((t0v + 15) / R, id.Tc - 1);

        // inter-chunk part: Chat H, rows scaled by exp(ell_t)
        floatx4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int n0 = 32 * ks + 8 * g;
                const frag hb = n0 < N ? M::lds8(&ht[(16 * pt + l16) * NBP + n0]) : M::zero();
                acc[pt] = M::mma(acc[pt], cf[i][ks], hb);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tok = (t0v + 4 * g + v) / R;
            const float e = tok < id.Tc ? expf(ell_s[tok]) : 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt][v] *= e;
        }

        // intra-chunk part over 32-wide column pairs of s, causal blocks only
        const int tt = (t0v + l16) / R; // token of this lane's column t
        const float ell_t = ell_s[tt < kQ ? tt : kQ - 1];
        const float gam_t = gam_s[tt < kQ ? tt : kQ - 1];
        for (int s0 = 0; s0 / R <= tok_last; s0 += 32) {
            floatx4 st[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                st[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int n0 = 32 * ks + 8 * g;
                    const frag ab = n0 < N ? M::lds8(&bs[(s0 + 16 * q + l16) * NBP + n0]) : M::zero();
                    st[q] = M::mma(st[q], ab, cf[i][ks]);
                }
            }
            float m[8];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int ts = (s0 + 16 * q + 4 * g + v) / R;
                    float w = 0.f;
                    if (ts <= tt && tt < id.Tc) w = ts == tt ? gam_t : expf(ell_t - ell_s[ts]) * wgt_s[ts];
                    m[4 * q + v] = st[q][v] * w;
                }
            }
            const frag mf = M::pack(m);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const lds_t *xr = xt + (16 * pt + l16) * VP + s0 + 4 * g;
                acc[pt] = M::mma(acc[pt], mf, M::lds4x2(xr, xr + 16));
            }
        }

        // store rows of valid tokens
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int vr = t0v + 4 * g + v;
            const int tok = vr / R, ch = vr - tok * R;
            if (tok < id.Tc) {
                IO *dst = y + tok_off(p, id, id.t0 + tok, ch, P) + l16;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) io<IO>::put(dst + 16 * pt, acc[pt][v]);
            }
        }
    }
}

#define M3_LAUNCH_CHUNK_OUTPUT(IO, NN, PP)                                                  \
    {                                                                                       \
        const size_t lds = ChunkOutputLds<IO, NN, PP>::bytes(p.R);                          \
        if (lds > 65536) {                                                                  \
            hipError_t e = hipFuncSetAttribute(                                             \
                reinterpret_cast<const void *>(&k_chunk_output<IO, NN, PP>),                \
                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));                      \
            if (e != hipSuccess) return e;                                                  \
        }                                                                                   \
        hipLaunchKernelGGL((k_chunk_output<IO, NN, PP>), grid, block, lds, s, p);           \
        return hipGetLastError();                                                           \
    }

#define M3_LDS_CHUNK_OUTPUT(IO, NN, PP) return ChunkOutputLds<IO, NN, PP>::bytes(R);

size_t chunk_output_lds_bytes(bool is_bf16, int N, int P, int R) {
    if (is_bf16) {
        M3_DISPATCH_NP(::m3::bf16, N, P, M3_LDS_CHUNK_OUTPUT);
    } else {
        M3_DISPATCH_NP(float, N, P, M3_LDS_CHUNK_OUTPUT);
    }
    return 0;
}

hipError_t launch_chunk_output(const PrefillParams &p, bool is_bf16, hipStream_t s) {
    const dim3 grid(unsigned(p.batch * p.H * p.nC)), block(kThreads);
    M3_DISPATCH(is_bf16, p.N, p.P, M3_LAUNCH_CHUNK_OUTPUT);
}

} // namespace m3
