// m3_device.hpp -- device helpers shared by the gfx950 kernels of the mixer:
// element types, vector loads, the 16x16x32 MFMA fragment abstraction and
// wave-wide scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

constexpr int kQ = 64;        // tokens per chunk
constexpr int kWave = 64;     // CDNA wavefront width
constexpr double kPi = 3.14159265358979323846;
constexpr double kTwoPi = 6.28318530717958647692;

// bf16 as stored in HBM: raw bits.
struct bf16 {
    uint16_t bits;
};

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

__device__ __forceinline__ float bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats -> two bf16 in one word (lo in the low half), one instruction.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float float2_v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

// One 16-byte global load as a plain vector value (not an aggregate copy,
// which can leave its destination in private memory).
__device__ __forceinline__ uint4 ld16(const void *p) {
    const u32x4_v v = *static_cast<const u32x4_v *>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const float2_v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// ---------------------------------------------------------------------------
// I/O element access.  load8 reads 8 consecutive elements (16-byte aligned).
// ---------------------------------------------------------------------------
template <typename IO>
struct io;

template <>
struct io<float> {
    static __device__ __forceinline__ float get(const float *p) { return *p; }
    // Raw bits of one element, and their value: a load kept as raw bits is not
    // waited for until the value is used.
    static __device__ __forceinline__ uint32_t raw(const float *p) { return __float_as_uint(*p); }
    static __device__ __forceinline__ float value(uint32_t r) { return __uint_as_float(r); }
    static __device__ __forceinline__ void put(float *p, float v) { *p = v; }
    static __device__ __forceinline__ void load8(const float *p, float v[8]) {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void load4(const float *p, float v[4]) {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    }
    static __device__ __forceinline__ void store4(float *p, const float v[4]) {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

template <>
struct io<bf16> {
    static __device__ __forceinline__ float get(const bf16 *p) { return bits_to_f32(p->bits); }
    static __device__ __forceinline__ uint32_t raw(const bf16 *p) { return p->bits; }
    static __device__ __forceinline__ float value(uint32_t r) { return __uint_as_float(r << 16); }
    static __device__ __forceinline__ void put(bf16 *p, float v) { p->bits = f32_to_bits(v); }
    static __device__ __forceinline__ void load8(const bf16 *p, float v[8]) {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load4(const bf16 *p, float v[4]) {
        const uint2 a = *reinterpret_cast<const uint2 *>(p);
        v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xffff0000u);
        v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store4(bf16 *p, const float v[4]) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
    }
};

// Four consecutive I/O elements kept as raw bits (8 bytes for bf16, 16 for
// fp32): loaded early, decoded when used.
template <typename IO>
struct io4;
template <>
struct io4<bf16> {
    typedef uint2 raw;
    static __device__ __forceinline__ raw load(const bf16 *p) { return *reinterpret_cast<const uint2 *>(p); }
    static __device__ __forceinline__ void unpack(const raw &r, float v[4]) {
        v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xffff0000u);
        v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xffff0000u);
    }
};
template <>
struct io4<float> {
    typedef uint4 raw;
    static __device__ __forceinline__ raw load(const float *p) { return *reinterpret_cast<const uint4 *>(p); }
    static __device__ __forceinline__ void unpack(const raw &r, float v[4]) {
        v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
    }
};

// ---------------------------------------------------------------------------
// MFMA fragments for v_mfma_f32_16x16x32_bf16 (gfx950).
// Operand A (16 x 32): lane l supplies row (l % 16) and eight k-slots
// (group g = l / 16, j = 0..7).  Operand B (32 x 16): lane l supplies column
// (l % 16) and the same eight k-slots.  The hardware pairs A and B by k-slot,
// so a contraction only needs both operands to use one slot -> k mapping.
// Result D (16 x 16 fp32): lane l holds D[4 g + v][l % 16], v = 0..3.
//
// Staged operands live in LDS as PL planes of bf16 bits, plane 1 a fixed
// number of elements (PS) after plane 0:
//   PL = 1 (bf16 I/O): the value rounded to bf16, one MFMA per step;
//   PL = 2 (fp32 I/O): a = hi + lo, both bf16; a*b is taken as
//          hi*hi + hi*lo + lo*hi (three MFMAs), about 2^-16 relative.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 bf16x8_from_words(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposing LDS load (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 64-bit word addressed by lane
// 4 s + i / 4 of its group, for s = 0..3.  So when lane j of a group
// addresses row r0 + j / 4, elements c0 + 4 (j % 4) .. + 3 of a row-major
// bf16 matrix, lane i receives column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ uint2 lds_tr4(const uint16_t *p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p)));
}

// Scheduling order of a pipelined loop of NI products whose operands are LDS
// reads (RD reads each, MF MFMAs each) issued DEPTH products ahead: DEPTH
// operand reads, then (product, next operand) pairs, then the last DEPTH
// products.  A hint to the scheduler only; it keeps the LDS reads in flight
// instead of waiting for each one in turn.
template <int NI, int DEPTH, int RD, int MF>
__device__ __forceinline__ void sched_pipeline() {
    __builtin_amdgcn_sched_group_barrier(0x100, DEPTH * RD, 0);
#pragma unroll
    for (int i = 0; i < NI - DEPTH; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, DEPTH * MF, 0);
}

template <int PL>
struct Mma {
    static constexpr int kMfma = PL == 2 ? 3 : 1; // MFMA instructions per product
    struct frag {
        bf16x8 v[PL];
    };
    static __device__ __forceinline__ frag zero() {
        frag f;
#pragma unroll
        for (int k = 0; k < PL; ++k) f.v[k] = bf16x8_from_words(0, 0, 0, 0);
        return f;
    }
    // Eight floats into the planes (hi = RNE bf16, lo = bf16 of the rest).
    static __device__ __forceinline__ frag pack(const float a[8]) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hw[i] = pack2_bf16(a[2 * i], a[2 * i + 1]);
            if constexpr (PL == 2)
                lw[i] = pack2_bf16(a[2 * i] - __uint_as_float(hw[i] << 16),
                                   a[2 * i + 1] - __uint_as_float(hw[i] & 0xffff0000u));
        }
        frag f;
        f.v[0] = bf16x8_from_words(hw[0], hw[1], hw[2], hw[3]);
        if constexpr (PL == 2) f.v[1] = bf16x8_from_words(lw[0], lw[1], lw[2], lw[3]);
        return f;
    }
    // The eight values a fragment stands for (sum of its planes).
    static __device__ __forceinline__ void unpack(const frag &f, float a[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = 0.f;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint4 w = __builtin_bit_cast(uint4, f.v[k]);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[2 * i] += __uint_as_float(ws[i] << 16);
                a[2 * i + 1] += __uint_as_float(ws[i] & 0xffff0000u);
            }
        }
    }
    static __device__ __forceinline__ floatx4 mma(floatx4 acc, const frag &a, const frag &b) {
        if constexpr (PL == 2) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[1], b.v[0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[0], b.v[1], acc, 0, 0, 0);
        }
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[0], b.v[0], acc, 0, 0, 0);
    }
    // Eight consecutive elements of each plane (16-byte aligned).
    template <int PS>
    static __device__ __forceinline__ frag lds8(const uint16_t *p) {
        frag f;
#pragma unroll
        for (int k = 0; k < PL; ++k) f.v[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p + k * PS));
        return f;
    }
    // Slots 0-3 from a transposing load at p0, slots 4-7 from one at p1.
    template <int PS>
    static __device__ __forceinline__ frag tr8(const uint16_t *p0, const uint16_t *p1) {
        frag f;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint2 a = lds_tr4(p0 + k * PS), b = lds_tr4(p1 + k * PS);
            f.v[k] = bf16x8_from_words(a.x, a.y, b.x, b.y);
        }
        return f;
    }
};

// Store NV (4 or 8) floats as consecutive elements of each plane at p.
template <int PL, int PS, int NV>
__device__ __forceinline__ void st_planes(uint16_t *p, const float *v) {
    uint32_t hw[NV / 2], lw[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
        hw[i] = pack2_bf16(v[2 * i], v[2 * i + 1]);
        if constexpr (PL == 2)
            lw[i] = pack2_bf16(v[2 * i] - __uint_as_float(hw[i] << 16),
                               v[2 * i + 1] - __uint_as_float(hw[i] & 0xffff0000u));
    }
    if constexpr (NV == 8) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        if constexpr (PL == 2) *reinterpret_cast<uint4 *>(p + PS) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else {
        static_assert(NV == 4, "4 or 8 values");
        *reinterpret_cast<uint2 *>(p) = make_uint2(hw[0], hw[1]);
        if constexpr (PL == 2) *reinterpret_cast<uint2 *>(p + PS) = make_uint2(lw[0], lw[1]);
    }
}

// Compute mode of an I/O type: bf16 I/O -> one bf16 plane; fp32 I/O -> hi/lo planes.
template <typename IO>
struct mode {
    static constexpr bool f32 = false;
};
template <>
struct mode<float> {
    static constexpr bool f32 = true;
};

// ---------------------------------------------------------------------------
// Wave-wide inclusive prefix sums (Kogge-Stone over the 64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_inclusive_sum(float v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

__device__ __forceinline__ double wave_inclusive_sum(double v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

// Wave-wide inclusive prefix sums with DPP lane moves (no LDS): Hillis-Steele
// within each row of 16 lanes (row_shr 1, 2, 4, 8; lanes shifted in from
// outside the row read 0), then row 0's total into row 1 and row 2's into
// row 3 (row_bcast:15), then the total of rows 0-1 into rows 2-3
// (row_bcast:31).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xf, BOUND_ZERO));
}
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __uint_as_float(dpp_u32<CTRL, ROW_MASK, BOUND_ZERO>(__float_as_uint(v)));
}
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ double dpp_add(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK, BOUND_ZERO>(uint32_t(u));
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK, BOUND_ZERO>(uint32_t(u >> 32));
    return v + __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp_add(uint32_t v) {
    return v + dpp_u32<CTRL, ROW_MASK, BOUND_ZERO>(v);
}
template <typename T>
__device__ __forceinline__ T wave_scan_dpp(T v) {
    v = dpp_add<0x111, 0xf, true>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf, true>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf, true>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf, true>(v);  // row_shr:8
    v = dpp_add<0x142, 0xa, false>(v); // row_bcast:15 -> rows 1, 3
    v = dpp_add<0x143, 0xc, false>(v); // row_bcast:31 -> rows 2, 3
    return v;
}

// Angles as 32-bit fixed-point fractions of a turn (2^32 units per 2 pi):
// integer sums of such values are exact modulo one turn, so an angle prefix
// over many tokens needs no floating-point wrap.  Conversion rounds to the
// nearest unit (1.46e-9 rad) in fp64.
__device__ __forceinline__ uint32_t angle_to_turns32(float a) {
    const double t = double(a) * (1.0 / kTwoPi);
    double r = rint((t - rint(t)) * 4294967296.0); // [-2^31, 2^31]
    if (r >= 2147483648.0) r -= 4294967296.0;
    return uint32_t(int32_t(r));
}
// A fixed-point angle as fp32 turns in [-1/2, 1/2).
__device__ __forceinline__ float turns32_to_f32(uint32_t u) { return float(int32_t(u)) * 0x1p-32f; }
// ... and as fp64 radians in [-pi, pi).
__device__ __forceinline__ double turns32_to_rad(uint32_t u) { return double(int32_t(u)) * (kTwoPi / 4294967296.0); }

// Angle wrapped to [-pi, pi), fp64.
__device__ __forceinline__ double wrap_angle(double a) {
    return a - kTwoPi * floor((a + kPi) * (1.0 / kTwoPi));
}

// sin and cos of an angle already wrapped to [-pi, pi], fp64 arithmetic,
// rounded to fp32.  Quadrant reduction x = q pi/2 + r (|r| <= pi/4, exact
// enough in fp64 for |x| <= pi), then the Taylor series of sin r and cos r to
// degree 17 and 18 (truncation below 1e-17 for |r| <= pi/4), and the
// quadrant identities.  Small and branch-free, unlike a general-argument
// library sincos.
__device__ __forceinline__ void sincos_wrapped(double x, float *s_out, float *c_out) {
    const double q = rint(x * (2.0 / kPi));
    const double r = x - q * (kPi / 2.0);
    const double r2 = r * r;
    // sin r = r (1 - r2/3! (1 - r2/(4*5) (1 - r2/(6*7) (...))))
    double sn = 1.0 - r2 * (1.0 / (16.0 * 17.0));
    sn = 1.0 - r2 * (1.0 / (14.0 * 15.0)) * sn;
    sn = 1.0 - r2 * (1.0 / (12.0 * 13.0)) * sn;
    sn = 1.0 - r2 * (1.0 / (10.0 * 11.0)) * sn;
    sn = 1.0 - r2 * (1.0 / (8.0 * 9.0)) * sn;
    sn = 1.0 - r2 * (1.0 / (6.0 * 7.0)) * sn;
    sn = 1.0 - r2 * (1.0 / (4.0 * 5.0)) * sn;
    sn = 1.0 - r2 * (1.0 / (2.0 * 3.0)) * sn;
    sn *= r;
    // cos r = 1 - r2/2! (1 - r2/(3*4) (1 - r2/(5*6) (...)))
    double cs = 1.0 - r2 * (1.0 / (17.0 * 18.0));
    cs = 1.0 - r2 * (1.0 / (15.0 * 16.0)) * cs;
    cs = 1.0 - r2 * (1.0 / (13.0 * 14.0)) * cs;
    cs = 1.0 - r2 * (1.0 / (11.0 * 12.0)) * cs;
    cs = 1.0 - r2 * (1.0 / (9.0 * 10.0)) * cs;
    cs = 1.0 - r2 * (1.0 / (7.0 * 8.0)) * cs;
    cs = 1.0 - r2 * (1.0 / (5.0 * 6.0)) * cs;
    cs = 1.0 - r2 * (1.0 / (3.0 * 4.0)) * cs;
    cs = 1.0 - r2 * 0.5 * cs;
    const int qi = int(q) & 3;
    const double s = qi == 0 ? sn : qi == 1 ? cs : qi == 2 ? -sn : -cs;
    const double c = qi == 0 ? cs : qi == 1 ? -sn : qi == 2 ? -cs : sn;
    *s_out = float(s);
    *c_out = float(c);
}

// Sum of v over the W consecutive lanes that hold one row (W a power of two
// dividing 64, every lane of the row active).  Within a 16-lane DPP row the
// partial sums are exchanged with DPP moves (quad permutations, then the
// half-row and row mirrors), across rows with lane shuffles.
template <int C>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), C, 0xf, 0xf, false));
}
template <int W>
__device__ __forceinline__ float row_sum(float v) {
    if constexpr (W >= 2) v += dpp_f32<0xb1>(v);  // quad_perm [1, 0, 3, 2]
    if constexpr (W >= 4) v += dpp_f32<0x4e>(v);  // quad_perm [2, 3, 0, 1]
    if constexpr (W >= 8) v += dpp_f32<0x141>(v); // row_half_mirror
    if constexpr (W >= 16) v += dpp_f32<0x140>(v); // row_mirror
#pragma unroll
    for (int m = 16; m < W; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Output gate factor silu(z) = z / (1 + e^{-z}) (hardware reciprocal; for
// z -> -inf the exponential overflows to inf and the factor to -0).
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Rotation R(-phi) of a row pair: (u, v) -> (c u + s v, -s u + c v).
__device__ __forceinline__ void rot_neg(float c, float s, float &u, float &v) {
    const float a = u, b = v;
    u = c * a + s * b;
    v = c * b - s * a;
}

} // namespace m3
