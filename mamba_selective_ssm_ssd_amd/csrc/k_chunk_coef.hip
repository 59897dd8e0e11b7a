// k_chunk_coef.hip -- per-chunk cumulative sum of the log decay and the
// trapezoid weights (one wavefront per (batch, head, chunk), one lane per
// token).
//
// For token t (Mamba-3 review, section 3.1.1, eqs. (5)-(6) and the
// coefficient table):  a_t = dt_t A (log alpha_t),  gamma_t = lam_t dt_t,
// delta_t = (1 - lam_t) dt_t (so beta_t = delta_t alpha_t).  Written out:
//   ell_t = sum_{t0 <= s <= t} a_s        within-chunk inclusive cumsum
//   gam_t = gamma_t
//   wgt_t = gamma_t + delta_{t+1}         (delta_T = 0 at the end of the call)
// In the masked form of section 3.1.3, eq. (7), the product of the decay
// matrix and the 2-band matrix has entries exp(ell_t - ell_s) * wgt_s below
// the diagonal and gam_t on it; wgt_s carries the two taps of token s.
//
// The chunk-0 workgroup of every (b, h) also folds the carried state into the
// state that enters chunk 0, in the state's own frame at the chunk start:
//   hinit = R(Phi_{-1}) (h~ + delta_0 B~_prev x_prev^T),
// the beta term of token 0 taken from the previous token (eq. (6)).
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

template <typename IO>
__global__ __launch_bounds__(kWave) void k_chunk_coef(const PrefillParams p) {
    const int lane = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int c = int(wg % p.nC);
    const int64_t bh = wg / p.nC;
    const int h = int(bh % p.H);
    const int64_t b = bh / p.H;
    const int64_t t = int64_t(c) * kQ + lane;
    const IO *dt = static_cast<const IO *>(p.dt);
    const IO *lam = static_cast<const IO *>(p.lam);

    float d = 0.f, l = 0.f;
    if (t < p.T) {
        d = io<IO>::get(dt + (b * p.T + t) * p.H + h);
        l = io<IO>::get(lam + (b * p.T + t) * p.H + h);
    }
    const float ell = wave_inclusive_sum(d * p.A[h], lane);
    const float gam = l * d;
    const float del = (1.f - l) * d;
    float del_next = __shfl_down(del, 1, kWave);
    if (lane == kWave - 1) {
        del_next = 0.f;
        if (t + 1 < p.T) {
            const float dn = io<IO>::get(dt + (b * p.T + t + 1) * p.H + h);
            const float ln = io<IO>::get(lam + (b * p.T + t + 1) * p.H + h);
            del_next = (1.f - ln) * dn;
        }
    }
    if (t + 1 >= p.T) del_next = 0.f;
    if (t < p.T) {
        const int64_t o = bh * p.T + t;
        p.ell[o] = ell;
        p.gam[o] = gam;
        p.wgt[o] = gam + del_next;
    }

    if (c == 0 && p.has_init) {
        const float del0 = __shfl(del, 0, kWave);
        const int N = p.N, P = p.P, R = p.R, K = p.K;
        const IO *px = static_cast<const IO *>(p.prevx0) + bh * R * P;
        const float *pb = p.prevB0 + bh * R * N;
        const float *h0 = p.h0 + bh * int64_t(N) * P;
        float *hi = p.hinit + bh * int64_t(N) * P;
        for (int e = lane; e < K * P; e += kWave) {
            const int k = e / P, pc = e - k * P;
            float v0 = h0[(2 * k) * P + pc], v1 = h0[(2 * k + 1) * P + pc];
            for (int r = 0; r < R; ++r) {
                const float xr = del0 * io<IO>::get(px + r * P + pc);
                v0 += pb[r * N + 2 * k] * xr;
                v1 += pb[r * N + 2 * k + 1] * xr;
            }
            float sn, cs;
            sincosf(p.phi0[bh * K + k], &sn, &cs);
            hi[(2 * k) * P + pc] = cs * v0 - sn * v1;
            hi[(2 * k + 1) * P + pc] = sn * v0 + cs * v1;
        }
        for (int k = lane; k < K; k += kWave) p.phi0ws[bh * K + k] = double(p.phi0[bh * K + k]);
    }
}

hipError_t launch_chunk_coef(const PrefillParams &p, bool is_bf16, hipStream_t s) {
    const dim3 grid(unsigned(p.batch * p.H * p.nC)), block(kWave);
    if (is_bf16)
        hipLaunchKernelGGL(k_chunk_coef<bf16>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(k_chunk_coef<float>, grid, block, 0, s, p);
    return hipGetLastError();
}

} // namespace m3
