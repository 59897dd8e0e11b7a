// k_chunk_state.hip -- state contributed by one chunk (MFMA).
//
// For chunk c with tokens s in [t0, t0 + Tc) and virtual rows v = s * R + r
// (MIMO: the rank-R update of the Mamba-3 review, section 3.3, is a sum over
// the R columns of B_s and rows of x_s), the chunk's contribution to the state
// at its end, in the frame of the chunk start, is
//     U_c[n][p] = sum_v  exp(g_c - ell_s) * wgt_s * Bhat[v][n] * x[v][p]
// with Bhat = R(-phi_loc[s]) B_s (the RoPE form of section 3.2.2,
// Prop. 3.2.3, relative to the chunk start), g_c = ell at the chunk's last
// token and wgt_s = gamma_s + delta_{s+1}: the weight with which token s
// reaches every later state through the decay matrix times 2-band matrix of
// eq. (7) (for the last token this includes the beta term of the next
// chunk's first token).  The inter-chunk kernel turns U_c into states.
//
// One workgroup of 256 threads per (b, h, c).  B (rotated, scaled) and x are
// staged transposed in LDS (contraction index v contiguous) and contracted
// with v_mfma_f32_16x16x32_bf16; output tiles of 16 x 16 are spread over the
// four waves.  The chunk's angle totals for the inter-chunk kernel are
// written here as a by-product of the angle scan.
#include "m3_chunk.hpp"

namespace m3 {

template <typename IO, int N, int P>
struct ChunkStateLds {
    typedef typename Mma<mode<IO>::f32>::lds_t lds_t;
    static constexpr int K = N / 2, KP = K + 1;
    static constexpr int PADE = 16 / int(sizeof(lds_t));
    static __host__ __device__ size_t vp(int R) { return size_t(kQ * R + PADE); }
    static __host__ __device__ size_t off_phi() { return 2 * kQ * sizeof(float); }
    static __host__ __device__ size_t off_bst() { return off_phi() + size_t(kQ) * KP * sizeof(float); }
    static __host__ __device__ size_t off_xt(int R) { return off_bst() + size_t(N) * vp(R) * sizeof(lds_t); }
    static __host__ __device__ size_t bytes(int R) { return off_xt(R) + size_t(P) * vp(R) * sizeof(lds_t); }
};

template <typename IO, int N, int P>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_state(const PrefillParams p) {
    typedef Mma<mode<IO>::f32> M;
    typedef typename M::lds_t lds_t;
    typedef ChunkStateLds<IO, N, P> L;
    constexpr int K = N / 2;
    const int R = p.R, V = kQ * R;
    const int VP = int(L::vp(R));
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const ChunkId id = chunk_id(p);

    extern __shared__ __align__(16) unsigned char smem[];
    float *ell_s = reinterpret_cast<float *>(smem);
    float *scl_s = ell_s + kQ;
    float *phi_s = reinterpret_cast<float *>(smem + L::off_phi());
    lds_t *bst = reinterpret_cast<lds_t *>(smem + L::off_bst());
    lds_t *xt = reinterpret_cast<lds_t *>(smem + L::off_xt(R));

    if (tid < kQ) {
        float e = 0.f, w = 0.f;
        if (tid < id.Tc) {
            const int64_t o = id.bh * p.T + id.t0 + tid;
            e = p.ell[o];
            w = p.wgt[o];
        }
        ell_s[tid] = e;
        scl_s[tid] = w;
    }
    chunk_angles<IO, K>(p, id, phi_s, true); // contains the barriers
    if (tid < kQ) {
        const float g = ell_s[id.Tc - 1];
        scl_s[tid] = tid < id.Tc ? expf(g - ell_s[tid]) * scl_s[tid] : 0.f;
    }
    __syncthreads();

    // Stage Bhat * scale and x transposed: bst[n][v], xt[p][v]; one item is a
    // pair of adjacent virtual rows and 8 consecutive columns.
    const IO *Bsrc = static_cast<const IO *>(p.B);
    constexpr int NG = N / 8, PG = P / 8;
    for (int it = tid; it < (V / 2) * NG; it += kThreads) {
        const int vp2 = it / NG, q = it - vp2 * NG;
        const int v0 = 2 * vp2;
        float r0[8], r1[8];
        load_rotated8<IO, K>(p, id, Bsrc, phi_s, v0, q, scl_s[v0 / R], r0);
        load_rotated8<IO, K>(p, id, Bsrc, phi_s, v0 + 1, q, scl_s[(v0 + 1) / R], r1);
#pragma unroll
        for (int j = 0; j < 8; ++j) M::st2(&bst[(8 * q + j) * VP + v0], r0[j], r1[j]);
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
    __syncthreads();

    // U[n][p] = sum_v bst[n][v] xt[p][v]: 16 x 16 output tiles over the waves.
    constexpr int NT = N / 16, PT = P / 16;
    const int g = lane >> 4, l16 = lane & 15;
    float *U = p.ubuf + ((id.bh * p.nC + id.c) * int64_t(N)) * P;
    for (int tile = wave; tile < NT * PT; tile += kThreads / kWave) {
        const int nt = tile / PT, pt = tile - nt * PT;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const lds_t *arow = bst + (16 * nt + l16) * VP + 8 * g;
        const lds_t *brow = xt + (16 * pt + l16) * VP + 8 * g;
        for (int ks = 0; ks < V / 32; ++ks)
            acc = M::mma(acc, M::lds8(arow + 32 * ks), M::lds8(brow + 32 * ks));
#pragma unroll
        for (int v = 0; v < 4; ++v) U[(16 * nt + 4 * g + v) * P + 16 * pt + l16] = acc[v];
    }
}

#define M3_LAUNCH_CHUNK_STATE(IO, NN, PP)                                                   \
    {                                                                                       \
        const size_t lds = ChunkStateLds<IO, NN, PP>::bytes(p.R);                           \
        if (lds > 65536) {                                                                  \
            hipError_t e = hipFuncSetAttribute(                                             \
                reinterpret_cast<const void *>(&k_chunk_state<IO, NN, PP>),                 \
                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));                      \
            if (e != hipSuccess) return e;                                                  \
        }                                                                                   \
        hipLaunchKernelGGL((k_chunk_state<IO, NN, PP>), grid, block, lds, s, p);            \
        return hipGetLastError();                                                           \
    }

#define M3_LDS_CHUNK_STATE(IO, NN, PP) return ChunkStateLds<IO, NN, PP>::bytes(R);

size_t chunk_state_lds_bytes(bool is_bf16, int N, int P, int R) {
    if (is_bf16) {
        M3_DISPATCH_NP(::m3::bf16, N, P, M3_LDS_CHUNK_STATE);
    } else {
        M3_DISPATCH_NP(float, N, P, M3_LDS_CHUNK_STATE);
    }
    return 0;
}

hipError_t launch_chunk_state(const PrefillParams &p, bool is_bf16, hipStream_t s) {
    const dim3 grid(unsigned(p.batch * p.H * p.nC)), block(kThreads);
    M3_DISPATCH(is_bf16, p.N, p.P, M3_LAUNCH_CHUNK_STATE);
}

} // namespace m3
