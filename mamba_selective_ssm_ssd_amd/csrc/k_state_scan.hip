// k_state_scan.hip -- inter-chunk state passing.
//
// Chunk c ends with the state (in the frame of its own last token, i.e. the
// start frame of chunk c + 1)
//     Hhat_c = R(Theta_c) ( exp(g_c) Hhat_{c-1} + U_c ),
// where U_c is the chunk's own contribution (k_chunk_state), g_c its summed
// log decay and Theta_c its summed rotary angle: the decay and rotation
// exp(dt A + i theta) of the complex state (Mamba-3 review, section 3.2,
// Props. 3.2.1-3.2.3) compounded over the chunk.  This is the sequential
// passing of end-of-chunk states of the chunkwise algorithm (the
// "20.2 Mamba and S6" page, section 2).  Row pair (2k, 2k+1) at column p is
// the complex number Hhat[2k][p] + i Hhat[2k+1][p].
//
// Each thread owns one complex element (k, p) of one (b, h) and walks the
// chunks in order: a single complex multiply-add per chunk, with the next
// chunks' inputs prefetched, lanes along p so every access is coalesced.
// The chunk buffer is updated in place: slot c receives Hhat_{c-1}, the state
// entering chunk c, which the chunk-output kernel reads.
//
// After the last chunk the state is moved to the caller's rotated frame,
// h~ = R(-Phi_{T-1}) Hhat, with Phi_{T-1} = Phi_{-1} + sum_c Theta_c summed in
// fp64 and wrapped to [-pi, pi).  The same workgroups write the carried
// previous-token terms prev_B = R(-Phi_{T-1}) B_{T-1} and prev_x = x_{T-1}.
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

constexpr int kScanDepth = 8; // chunks prefetched ahead

template <typename IO>
__global__ __launch_bounds__(kThreads) void k_state_scan(const PrefillParams p) {
    const int N = p.N, P = p.P, K = p.K, nC = p.nC;
    const int elems = K * P;
    const int nblk = (elems + kThreads - 1) / kThreads;
    const int64_t bh = blockIdx.x / nblk;
    const int blk = int(blockIdx.x - bh * nblk);
    const int e = blk * kThreads + threadIdx.x;
    if (e >= elems) return;
    const int k = e / P, pc = e - k * P;
    const int64_t b = bh / p.H;
    const int h = int(bh - b * p.H);

    float zr = 0.f, zi = 0.f;
    if (p.has_init) {
        const float *hi = p.hinit + bh * int64_t(N) * P;
        zr = hi[(2 * k) * P + pc];
        zi = hi[(2 * k + 1) * P + pc];
    }
    double thsum = 0.0;
    const int64_t ustride = int64_t(N) * P;
    float *U = p.ubuf + bh * nC * ustride + (2 * k) * P + pc;
    const float *ellh = p.ell + bh * p.T;
    const float2 *cs_h = p.thetaCS + bh * int64_t(nC) * K + k;
    const double *th_h = p.thetaC + bh * int64_t(nC) * K + k;

    for (int c0 = 0; c0 < nC; c0 += kScanDepth) {
        float ur[kScanDepth], ui[kScanDepth], eg[kScanDepth];
        float2 cs[kScanDepth];
#pragma unroll
        for (int j = 0; j < kScanDepth; ++j) {
            const int c = c0 + j;
            if (c < nC) {
                ur[j] = U[c * ustride];
                ui[j] = U[c * ustride + P];
                int64_t last = int64_t(c + 1) * kQ;
                if (last > p.T) last = p.T;
                eg[j] = expf(ellh[last - 1]);
                cs[j] = cs_h[int64_t(c) * K];
                thsum += th_h[int64_t(c) * K];
            }
        }
#pragma unroll
        for (int j = 0; j < kScanDepth; ++j) {
            const int c = c0 + j;
            if (c < nC) {
                U[c * ustride] = zr;
                U[c * ustride + P] = zi;
                const float ar = eg[j] * zr + ur[j];
                const float ai = eg[j] * zi + ui[j];
                zr = cs[j].x * ar - cs[j].y * ai;
                zi = cs[j].y * ar + cs[j].x * ai;
            }
        }
    }

    if (!p.has_final) return;
    const double phi = wrap_angle((p.has_init ? p.phi0ws[bh * K + k] : 0.0) + thsum);
    double sd, cd;
    sincos(phi, &sd, &cd);
    const float cw = float(cd), sw = float(sd);
    float *hT = p.hT + bh * int64_t(N) * P;
    hT[(2 * k) * P + pc] = cw * zr + sw * zi;
    hT[(2 * k + 1) * P + pc] = cw * zi - sw * zr;
    if (pc == 0) p.phiT[bh * K + k] = float(phi);
    const int64_t tl = (b * p.T + p.T - 1) * p.H + h; // token-head index of T-1
    if (pc < p.R) {
        const IO *Bl = static_cast<const IO *>(p.B) + (tl * p.R + pc) * N + 2 * k;
        float u = io<IO>::get(Bl), v = io<IO>::get(Bl + 1);
        rot_neg(cw, sw, u, v);
        float *pb = p.prevBT + (bh * p.R + pc) * N + 2 * k;
        pb[0] = u;
        pb[1] = v;
    }
    if (k == 0) {
        const IO *xl = static_cast<const IO *>(p.x) + tl * p.R * P;
        IO *px = static_cast<IO *>(p.prevxT) + bh * p.R * P;
        for (int r = 0; r < p.R; ++r) px[r * P + pc] = xl[r * P + pc];
    }
}

hipError_t launch_state_scan(const PrefillParams &p, bool is_bf16, hipStream_t s) {
    const int elems = p.K * p.P;
    const int nblk = (elems + kThreads - 1) / kThreads;
    const dim3 grid(unsigned(p.batch * p.H * nblk)), block(kThreads);
    if (is_bf16)
        hipLaunchKernelGGL(k_state_scan<bf16>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(k_state_scan<float>, grid, block, 0, s, p);
    return hipGetLastError();
}

} // namespace m3
