// k_decode.hpp -- one fused decode step for every (batch, head).
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
// head).  Workgroups of 128 or 256 threads walk the (b, h) items grid-stride; each
// thread owns float4 runs along P of the state, so every state access is a
// coalesced 16-byte access, and the state of the workgroup's next item is
// loaded while the current one is computed, so state loads are always in
// flight.  The kernel is instantiated per (I/O type, N, P, R).  The small per-item vectors (B, C, x, x_prev, B~_prev) are read as
// 16-byte units spread over the threads; a thread holding a unit of B or C
// advances Phi for that unit's pairs (fp64 add and wrap, sin/cos of the angle
// in turns) and rotates it.  Values read from the carried state are written
// back only after the workgroup barrier, so no thread overwrites an input
// another thread still reads.
//
// With BLK the Mamba-3 block's prologue and epilogue (review, section 3.4:
// BC normalisation, B/C biases, output gate) run inside the step: a B or C
// unit is scaled by its row's 1 / sqrt(mean_n v^2 + eps) (the row's units sit
// in aligned groups of consecutive lanes, summed by lane shuffles), times the
// per-head weight plus bias, before its rotation; each output is multiplied
// by silu(z) at its store.
#pragma once
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

constexpr int kDecodeCus = 256; // compute units of an MI355X
// Threads per decode workgroup.  An item's step is a chain of phases
// separated by two workgroup barriers, so two-wave workgroups (each thread
// holding twice the state runs) put more items in flight per CU and wait on
// fewer waves at each barrier, where their registers allow it: the plain
// step with N <= 64 and N P <= 4096 (b256 H64 P64 N64 R4: 71.4 vs 74.9 us
// per step with a bf16 state, 103.4 vs 104.2 with fp32).  The block step
// and larger states would spill at that occupancy and keep four waves.
constexpr int decode_threads(int N, int P, bool BLK) { return !BLK && N <= 64 && N * P <= 4096 ? 128 : 256; }
// Resident waves per SIMD: each workgroup holds the state of two items
// (current and prefetched) in registers; a bf16 state takes half the
// registers, so more waves fit (256 threads: 75.0 vs 77.4 us per step of
// the b256 H64 P64 N64 R4 decode at five waves instead of four).  The block
// step's weights, biases and gate inputs take one wave fewer, which keeps
// every instantiation free of register spills.
constexpr int decode_waves_per_simd(int N, int P, bool BLK, bool SB) {
    return N * P > 4096 || (N > 64 && N * P >= 4096) ? 2
         : decode_threads(N, P, BLK) == 128 ? (SB ? 4 : 3)
         : BLK ? (SB ? 4 : 3) : (SB && N <= 64 ? 5 : 4);
}
// Streaming cache hints on the state's read-modify-write (non-temporal
// loads and stores, global_load/store ... nt), chosen per instantiation by
// measurement on the b256 H64 P64 N64 R4 step (us per step, plain / hint):
// the fp32 state reads with the hint (104.2 / 101.2; its stores with it are
// slower, 106.2); the bf16 state and the block step write with it (74.8 /
// 71.0 and 115.4 / 109.8).
constexpr bool decode_nt_load(bool BLK, bool SB) { return !SB; }
// State runs updated together per LDS read of x and x_prev (see the update):
// 4 takes the LDS operand reads of a step from 75 to 27 per wave.  On the b256
// H64 P64 N64 R4 step: bf16 state 69.6 -> 67.0 us, fp32 state and block step
// unchanged (groups of 2: 67.7 us; of 8: register spills, 84 us).
constexpr int DG = 4;
constexpr bool decode_nt_store(bool BLK, bool SB) { return SB || BLK; }
// Resident workgroups per CU (4 SIMDs).
constexpr int decode_wg_per_cu(int N, int P, bool BLK, bool SB) {
    return decode_waves_per_simd(N, P, BLK, SB) * 4 / (decode_threads(N, P, BLK) / kWave);
}

template <int N, int P, int DT>
struct DecodeLds {
    static constexpr int K = N / 2, P4 = P / 4;
    static constexpr int G = DT / P4; // row groups of the state
    // floats: bt, bp, ct [4][N]; x, xp [4][P]; phi' [K]; a 16-byte sink for
    // threads without a unit; red [G][4][P]
    static constexpr int o_bt = 0, o_bp = o_bt + 4 * N, o_ct = o_bp + 4 * N;
    static constexpr int o_x = o_ct + 4 * N, o_xp = o_x + 4 * P, o_ph = o_xp + 4 * P;
    static constexpr int o_sink = o_ph + (K + 3) / 4 * 4, o_red = o_sink + 4;
    static constexpr size_t floats = size_t(o_red) + size_t(G) * 4 * P;
};

// Rotation of one unit of B or C: EPU elements (EPU/2 pairs) by -Phi' with
// Phi' = wrap(Phi + theta) (fp64 add and wrap; sin and cos of the angle in
// turns).  Returns Phi' of the pairs in phn.
template <int NP>
__device__ __forceinline__ void rotate_unit(float *e, const float *ph, const float *th, float *phn) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const double a = wrap_angle(double(ph[j]) + double(th[j]));
        float tf = float(a * (1.0 / kTwoPi));
        tf -= rintf(tf);
        const float sn = __builtin_amdgcn_sinf(tf), cs = __builtin_amdgcn_cosf(tf);
        rot_neg(cs, sn, e[2 * j], e[2 * j + 1]);
        phn[j] = float(a);
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
// theta of EPU/2 pairs held as 8 raw bytes
__device__ __forceinline__ void unpack8(const uint2 &u, float *v, bf16) {
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void unpack8(const uint2 &u, float *v, float) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
}

// The small per-item vectors are cut into 16-byte units, numbered
// B (R*N/EPU units), C (same), x (R*P/EPU), x_prev (same), B~_prev (R*N/4,
// fp32).  A thread owns units tid, tid + 256, ...; the unit's kind, its
// source offset, item stride and LDS destination are fixed for the launch.
enum : int { kUnitB = 0, kUnitC = 1, kUnitX = 2, kUnitXp = 3, kUnitBp = 4, kUnitNone = 5 };

// One run of four consecutive state values (along P) as stored: fp32 (16
// bytes) or, with a bf16 state (SB), four bf16 (8 bytes, rounded to nearest
// even when stored).  Registers hold the stored form until the run is used.
template <bool SB>
struct StateRun;
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));
// One state run moved with or without the non-temporal hint.
template <bool NT>
__device__ __forceinline__ float4 run_load(const float4 *p) {
    if constexpr (!NT) return *p;
    const f32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
template <bool NT>
__device__ __forceinline__ uint2 run_load(const uint2 *p) {
    if constexpr (!NT) return *p;
    const u32x2_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_v *>(p));
    return make_uint2(v.x, v.y);
}
template <bool NT>
__device__ __forceinline__ void run_store(float4 *p, const float4 &a) {
    if constexpr (!NT) { *p = a; return; }
    const f32x4_v v = {a.x, a.y, a.z, a.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_v *>(p));
}
template <bool NT>
__device__ __forceinline__ void run_store(uint2 *p, const uint2 &a) {
    if constexpr (!NT) { *p = a; return; }
    const u32x2_v v = {a.x, a.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_v *>(p));
}
template <>
struct StateRun<false> {
    typedef float4 raw;
    static constexpr int bytes = 16;
    static __device__ __forceinline__ float4 unpack(const raw &r) { return r; }
    static __device__ __forceinline__ raw pack(const float u[4]) { return make_float4(u[0], u[1], u[2], u[3]); }
};
template <>
struct StateRun<true> {
    typedef uint2 raw;
    static constexpr int bytes = 8;
    static __device__ __forceinline__ float4 unpack(const raw &r) {
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
    static __device__ __forceinline__ raw pack(const float u[4]) { return make_uint2(pack2_bf16(u[0], u[1]), pack2_bf16(u[2], u[3])); }
};

template <typename IO, int N, int P, int R, bool BLK, bool SB>
__global__ __launch_bounds__(decode_threads(N, P, BLK)) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd(N, P, BLK, SB)))) void k_decode_step(const DecodeParams p) {
    typedef StateRun<SB> SR;
    typedef typename SR::raw HV;
    constexpr int DT = decode_threads(N, P, BLK);
    typedef DecodeLds<N, P, DT> L;
    constexpr int K = N / 2, P4 = L::P4, G = L::G;
    constexpr int SZ = int(sizeof(IO)), EPU = 16 / SZ, NPU = EPU / 2;
    constexpr int SLOTS = N * P4;                          // float4 runs in the state
    constexpr int SPT = (SLOTS + DT - 1) / DT; // runs per thread
    constexpr int URN = N * SZ / 16, URP = P * SZ / 16;    // 16-byte units per row of B/C and of x
    constexpr int UB = R * URN, UX = R * URP, UPB = R * N / 4, UT = 2 * UB + 2 * UX + UPB;
    constexpr int UPT = (UT + DT - 1) / DT;    // units per thread
    constexpr int64_t sB = int64_t(R) * N * SZ, sX = int64_t(R) * P * SZ, sBp = int64_t(R) * N * 4; // item strides
    static_assert(!BLK || R * P <= 4 * DT, "one gated output quad per thread");
    __shared__ __align__(16) float sm[L::floats];
    float *bt_s = sm + L::o_bt, *bp_s = sm + L::o_bp, *ct_s = sm + L::o_ct;
    float *x_s = sm + L::o_x, *xp_s = sm + L::o_xp, *ph_s = sm + L::o_ph, *red = sm + L::o_red;

    const int tid = threadIdx.x;
    const int64_t BH = p.batch * p.H;
    const int pg = tid % P4, rg = tid / P4;

    // ---- per-thread unit table (launch constant)
    int ukind[UPT], uw[UPT], udst[UPT], uk0[UPT];
    const char *ubase[UPT];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const int u = tid + j * DT;
        int kind, w;
        if (u < UB) kind = kUnitB, w = u;
        else if (u < 2 * UB) kind = kUnitC, w = u - UB;
        else if (u < 2 * UB + UX) kind = kUnitX, w = u - 2 * UB;
        else if (u < 2 * UB + 2 * UX) kind = kUnitXp, w = u - 2 * UB - UX;
        else if (u < UT) kind = kUnitBp, w = u - 2 * UB - 2 * UX;
        else kind = kUnitNone, w = 0;
        const void *b = kind == kUnitC ? p.C : kind == kUnitX ? p.x : kind == kUnitXp ? p.prevx : kind == kUnitBp ? static_cast<const void *>(p.prevB) : p.B;
        ukind[j] = kind;
        uw[j] = w;
        ubase[j] = static_cast<const char *>(b) + int64_t(w) * 16;
        udst[j] = kind == kUnitB ? L::o_bt + w * EPU : kind == kUnitC ? L::o_ct + w * EPU : kind == kUnitX ? L::o_x + w * EPU
                : kind == kUnitXp ? L::o_xp + w * EPU : kind == kUnitBp ? L::o_bp + 4 * w : L::o_sink;
        uk0[j] = kind <= kUnitC ? (w % URN) * NPU : 0;
    }

    // Every global load below is issued unconditionally (indices clamped) and
    // its value is consumed on every path, so no load sinks into a branch and
    // the compiler's wait counts are exact: waiting for an item's small
    // vectors never waits for the state prefetch issued after them.
    // The state of an item is SLOTS consecutive float4 runs; run tid + 256 j
    // is row (tid + 256 j) / P4, columns 4 pg .. 4 pg + 3.
    const int tslot = min(tid, SLOTS - 1);
    auto load_state = [&](int64_t item, HV *hv) {
        const HV *hs = static_cast<const HV *>(p.h) + item * SLOTS;
#pragma unroll
        for (int j = 0; j < SPT; ++j) hv[j] = run_load<decode_nt_load(BLK, SB)>(hs + j * DT + tslot);
    };

    // The small vectors of an item, as loaded (raw bits).  They are loaded one
    // item ahead, with that item's state, so an item's step never waits for
    // a load issued in the same step.
    struct Small {
        uint4 ud[UPT];
        uint2 ut[UPT];
        float ph[UPT][NPU];
        uint32_t dt_raw, lam_raw;
        float Ah;
    };
    // item = (batch, head); gitem = (batch, B/C group of the head)
    auto load_small = [&](const int64_t item, const int64_t gitem, const int h, Small &sv) {
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int64_t st = ukind[j] == kUnitBp ? sBp : (ukind[j] == kUnitX || ukind[j] == kUnitXp) ? sX : sB;
            // B, C units (and threads without a unit, which read B's first
            // unit) are rows of the item's B/C group
            const bool grp = ukind[j] <= kUnitC || ukind[j] == kUnitNone;
            sv.ud[j] = *reinterpret_cast<const uint4 *>(ubase[j] + (grp ? gitem : item) * st);
            sv.ut[j] = *reinterpret_cast<const uint2 *>(static_cast<const IO *>(p.theta) + item * K + uk0[j]);
            if constexpr (NPU == 4) {
                const float4 a = *reinterpret_cast<const float4 *>(p.phi + item * K + uk0[j]);
                sv.ph[j][0] = a.x; sv.ph[j][1] = a.y; sv.ph[j][2] = a.z; sv.ph[j][3] = a.w;
            } else {
                const float2 a = *reinterpret_cast<const float2 *>(p.phi + item * K + uk0[j]);
                sv.ph[j][0] = a.x; sv.ph[j][1] = a.y;
            }
        }
        sv.dt_raw = io<IO>::raw(static_cast<const IO *>(p.dt) + item);
        sv.lam_raw = io<IO>::raw(static_cast<const IO *>(p.lam) + item);
        sv.Ah = p.A[h];
    };

    // one item: cur holds its small vectors and hc its state; the next item's
    // (ni, ngi, nh) small vectors go to nxt and its state to hx
    auto step = [&](const int64_t item, const int h, const Small &cur, Small &nxt, const int64_t ni,
                    const int64_t ngi, const int nh, const HV *hc, HV *hx) {
        const uint4 *ud = cur.ud;
        const uint2 *ut = cur.ut;
        const auto &ph = cur.ph;
        const uint32_t dt_raw = cur.dt_raw, lam_raw = cur.lam_raw;
        const float Ah = cur.Ah;
        // (BLK) weight and bias of each unit's channels and the gate input of
        // this thread's outputs; a missing piece is read from a valid stand-in
        // (the item's state, x) and replaced by its neutral value below
        float4 wq[BLK ? UPT : 1][EPU / 4], bq[BLK ? UPT : 1][EPU / 4];
        typename io4<IO>::raw zr;
        if constexpr (BLK) {
            const float *hs0 = reinterpret_cast<const float *>(static_cast<const char *>(p.h) + item * (N * P / 4 * SR::bytes));
#pragma unroll
            for (int j = 0; j < UPT; ++j) {
                const bool isc = ukind[j] == kUnitC;
                const int off = ukind[j] <= kUnitC ? h * (R * N) + uw[j] * EPU : 0;
                const float *ws = isc ? p.blk.cw : p.blk.bw, *bs = isc ? p.blk.cb : p.blk.bb;
                const float4 *wa = reinterpret_cast<const float4 *>(ws ? ws + off : hs0);
                const float4 *ba = reinterpret_cast<const float4 *>(bs ? bs + off : hs0);
#pragma unroll
                for (int i = 0; i < EPU / 4; ++i) wq[j][i] = wa[i], bq[j][i] = ba[i];
            }
            const IO *zs = static_cast<const IO *>(p.blk.z ? p.blk.z : p.x) + item * (R * P) + min(4 * tid, R * P - 4);
            zr = io4<IO>::load(zs);
        }
        // ---- issue the next item's small vectors and state
        load_small(ni, ngi, nh, nxt);
        load_state(ni, hx);

        // ---- rotate B and C (every unit computes the rotation; only B and C
        // units keep it), stage them and x, x_prev, B~_prev in LDS
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int kind = ukind[j];
            const bool rot = kind <= kUnitC;
            float e[EPU], th[NPU], phn[NPU];
            unpack16(ud[j], e, IO());
            unpack8(ut[j], th, IO());
            float o[EPU];
#pragma unroll
            for (int i = 0; i < EPU; ++i) o[i] = e[i];
            if constexpr (BLK) {
                // block prologue of a B or C unit (its row's lanes all take part)
                float inv = 1.f;
                if (p.blk.norm) {
                    float ss = 0.f;
#pragma unroll
                    for (int i = 0; i < EPU; ++i) ss += e[i] * e[i];
                    inv = rsqrtf(row_sum<URN>(ss) * (1.f / N) + p.blk.eps);
                }
                const bool hw = (ukind[j] == kUnitC ? p.blk.cw : p.blk.bw) != nullptr;
                const bool hb = (ukind[j] == kUnitC ? p.blk.cb : p.blk.bb) != nullptr;
#pragma unroll
                for (int i = 0; i < EPU; ++i) {
                    const float4 a = wq[j][i / 4], c = bq[j][i / 4];
                    const float wv = (&a.x)[i % 4], bv = (&c.x)[i % 4];
                    o[i] = o[i] * inv * (hw ? wv : 1.f) + (hb ? bv : 0.f);
                }
            }
            rotate_unit<NPU>(o, ph[j], th, phn);
#pragma unroll
            for (int i = 0; i < EPU; ++i) o[i] = rot ? o[i] : e[i];
            float4 v0 = make_float4(o[0], o[1], o[2], o[3]);
            if (kind == kUnitBp) v0 = make_float4(__uint_as_float(ud[j].x), __uint_as_float(ud[j].y), __uint_as_float(ud[j].z), __uint_as_float(ud[j].w));
            *reinterpret_cast<float4 *>(sm + udst[j]) = v0;
            if constexpr (EPU == 8)
                if (kind <= kUnitXp) *reinterpret_cast<float4 *>(sm + udst[j] + 4) = make_float4(o[4], o[5], o[6], o[7]);
            if (kind == kUnitB && uw[j] < URN) {
                float *pd = ph_s + uw[j] * NPU;
                if constexpr (NPU == 4) *reinterpret_cast<float4 *>(pd) = make_float4(phn[0], phn[1], phn[2], phn[3]);
                else *reinterpret_cast<float2 *>(pd) = make_float2(phn[0], phn[1]);
            }
            __builtin_amdgcn_sched_barrier(0); // one unit at a time: bounds register use
        }
        __syncthreads();

        // ---- carried small state: B~_prev <- B~, x_prev <- x, Phi <- Phi'
        for (int w = tid; w < UPB; w += DT)
            *reinterpret_cast<float4 *>(p.prevB + item * R * N + 4 * w) = *reinterpret_cast<const float4 *>(bt_s + 4 * w);
        for (int w = tid; w < UX; w += DT) {
            const float *s = x_s + w * EPU;
            IO *d = static_cast<IO *>(p.prevx) + item * R * P + w * EPU;
#pragma unroll
            for (int i = 0; i < EPU; i += 4) io<IO>::store4(d + i, s + i);
        }
        for (int k = tid; k < K; k += DT) p.phi[item * K + k] = ph_s[k];

        // ---- state update and partial outputs
        const float dtv = io<IO>::value(dt_raw), lamv = io<IO>::value(lam_raw);
        const float alpha = __expf(dtv * Ah);
        const float beta = (1.f - lamv) * dtv * alpha;
        const float gamma = lamv * dtv;
        HV *hs = static_cast<HV *>(p.h) + item * SLOTS;
        float yp[R][4];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) yp[i][q] = 0.f;
        // The runs of a thread share their columns (4 pg .. 4 pg + 3), so
        // x and x_prev of those columns are read from LDS once per group of
        // GR runs and rank instead of once per run.
        constexpr int GR = DG < SPT ? DG : SPT;
        static_assert(SPT % GR == 0, "whole groups of state runs");
#pragma unroll
        for (int j0 = 0; j0 < SPT; j0 += GR) {
            float u[GR][4];
#pragma unroll
            for (int jj = 0; jj < GR; ++jj) {
                const float4 hv = SR::unpack(hc[j0 + jj]);
                u[jj][0] = alpha * hv.x; u[jj][1] = alpha * hv.y; u[jj][2] = alpha * hv.z; u[jj][3] = alpha * hv.w;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float4 xp4 = *reinterpret_cast<const float4 *>(xp_s + r * P + 4 * pg);
                const float4 x4 = *reinterpret_cast<const float4 *>(x_s + r * P + 4 * pg);
#pragma unroll
                for (int jj = 0; jj < GR; ++jj) {
                    const int n = min(tid + (j0 + jj) * DT, SLOTS - 1) / P4;
                    const float cb = beta * bp_s[r * N + n], cg = gamma * bt_s[r * N + n];
                    u[jj][0] += cb * xp4.x + cg * x4.x;
                    u[jj][1] += cb * xp4.y + cg * x4.y;
                    u[jj][2] += cb * xp4.z + cg * x4.z;
                    u[jj][3] += cb * xp4.w + cg * x4.w;
                }
            }
#pragma unroll
            for (int jj = 0; jj < GR; ++jj) {
                const int slot = tid + (j0 + jj) * DT;
                if (SLOTS % DT != 0 && slot >= SLOTS) continue;
                const int n = slot / P4;
                run_store<decode_nt_store(BLK, SB)>(hs + slot, SR::pack(u[jj]));
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float cc = ct_s[i * N + n];
#pragma unroll
                    for (int q = 0; q < 4; ++q) yp[i][q] += cc * u[jj][q];
                }
            }
            __builtin_amdgcn_sched_barrier(0); // one group at a time: bounds register use
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
            *reinterpret_cast<float4 *>(red + (rg * 4 + i) * P + 4 * pg) = make_float4(yp[i][0], yp[i][1], yp[i][2], yp[i][3]);
        __syncthreads();

        // y: four consecutive outputs per thread, one 4-element store
        IO *y = static_cast<IO *>(p.y) + item * R * P;
        constexpr int GACT = G < N ? G : N; // row groups that own at least one row
        for (int o = 4 * tid; o < R * P; o += 4 * DT) {
            const int i = o / P, pc = o - i * P;
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int r = 0; r < GACT; ++r) {
                const float4 v = *reinterpret_cast<const float4 *>(red + (r * 4 + i) * P + pc);
                s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
            }
            float sv[4] = {s.x, s.y, s.z, s.w};
            if constexpr (BLK) {
                if (p.blk.z) { // output gate y * silu(z)
                    float zv[4];
                    io4<IO>::unpack(zr, zv);
#pragma unroll
                    for (int q = 0; q < 4; ++q) sv[q] *= silu(zv[q]);
                }
            }
            io<IO>::store4(y + o, sv);
        }
    };

    // Two items per trip, the state registers swapping roles, so the
    // prefetched state is never copied (a copy would wait for it).
    HV ha[SPT], hb[SPT];
    int64_t item = blockIdx.x;       // the grid never exceeds the item count
    int h = int(item % p.H);         // head and batch of the item, advanced
    int64_t bi = item / p.H;         // without a division
    const int hstep = int(gridDim.x % unsigned(p.H));
    const int64_t bstep = gridDim.x / unsigned(p.H);
    auto advance = [&]() {
        item += gridDim.x;
        h += hstep;
        bi += bstep;
        if (h >= p.H) h -= p.H, ++bi;
    };
    auto gitem = [&]() { return bi * p.G + h / p.hpg; };
    // the item after this one (this one again past the last)
    int64_t ni, ngi;
    int nh;
    auto peek = [&]() {
        ni = item + gridDim.x;
        int hh = h + hstep;
        int64_t bb = bi + bstep;
        if (hh >= p.H) hh -= p.H, ++bb;
        if (ni >= BH) ni = item, hh = h, bb = bi;
        nh = hh;
        ngi = bb * p.G + hh / p.hpg;
    };
    Small sa, sb;
    load_small(item, gitem(), h, sa);
    load_state(item, ha);
    for (;;) {
        peek();
        step(item, h, sa, sb, ni, ngi, nh, ha, hb);
        advance();
        if (item >= BH) break;
        peek();
        step(item, h, sb, sa, ni, ngi, nh, hb, ha);
        advance();
        if (item >= BH) break;
    }
}

template <typename IO, int N, int P, int R, bool BLK, bool SB>
hipError_t launch_decode_inst(const DecodeParams &p, hipStream_t s) {
    const int64_t bh = p.batch * p.H;
    const int64_t cap = int64_t(kDecodeCus) * decode_wg_per_cu(N, P, BLK, SB);
    const dim3 grid{static_cast<unsigned>(bh < cap ? bh : cap)}, block{unsigned(decode_threads(N, P, BLK))};
    hipLaunchKernelGGL((k_decode_step<IO, N, P, R, BLK, SB>), grid, block, 0, s, p);
    return hipGetLastError();
}

// Dispatch over (N, P, R) for one I/O type, with or without the block ops,
// fp32 or bf16 state.
template <typename IO, bool BLK, bool SB>
hipError_t launch_decode_io(const DecodeParams &p, hipStream_t s) {
#define M3_DECODE_R(NN, PP)                                                   \
    switch (p.R) {                                                            \
    case 1: return launch_decode_inst<IO, NN, PP, 1, BLK, SB>(p, s);          \
    case 2: return launch_decode_inst<IO, NN, PP, 2, BLK, SB>(p, s);          \
    case 3: return launch_decode_inst<IO, NN, PP, 3, BLK, SB>(p, s);          \
    case 4: return launch_decode_inst<IO, NN, PP, 4, BLK, SB>(p, s);          \
    default: return hipErrorInvalidValue;                                     \
    }
#define M3_DECODE_P(NN)                                                       \
    switch (p.P) {                                                            \
    case 16: M3_DECODE_R(NN, 16)                                              \
    case 32: M3_DECODE_R(NN, 32)                                              \
    case 64: M3_DECODE_R(NN, 64)                                              \
    default: return hipErrorInvalidValue;                                     \
    }
    switch (p.N) {
    case 16: M3_DECODE_P(16)
    case 32: M3_DECODE_P(32)
    case 64: M3_DECODE_P(64)
    case 128: M3_DECODE_P(128)
    default: return hipErrorInvalidValue;
    }
#undef M3_DECODE_P
#undef M3_DECODE_R
}

} // namespace m3
