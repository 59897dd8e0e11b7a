// m3_ceilings.hip -- the on-chip ceilings of include/m3_ssm_ceilings.h: an
// MFMA-only loop and a float4 stream (copy or in-place read-modify-write).
#include "m3_ssm_ceilings.h"

#include <hip/hip_runtime.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;

// Every wave: iters x 8 MFMAs on 8 independent accumulators (no dependent
// chain shorter than 8 instructions), operands derived from the lane id so
// the compiler cannot fold them.
template <int KIND>
__global__ __launch_bounds__(256) void k_ceiling_mfma(int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    floatx4_t c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
    if constexpr (KIND == 0) {
        bf16x8_t a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(1.0f + 0.001f * float(lane + i));
            b[i] = (__bf16)(1.0f - 0.001f * float(lane - i));
        }
#pragma unroll 2
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
            c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
            c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
            c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
            c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
        }
    } else {
        const float a = 1.0f + 0.001f * float(lane), b = 1.0f - 0.001f * float(lane);
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c3, 0, 0, 0);
            c4 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c4, 0, 0, 0);
            c5 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c5, 0, 0, 0);
            c6 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c6, 0, 0, 0);
            c7 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c7, 0, 0, 0);
        }
    }
    const floatx4_t t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    sink[blockIdx.x * 256 + threadIdx.x] = t[0] + t[1] + t[2] + t[3];
}

// One float4 moved with or without the non-temporal hint.
template <bool NT>
__device__ __forceinline__ floatx4_t ld4(const floatx4_t *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT>
__device__ __forceinline__ void st4(floatx4_t *p, const floatx4_t &v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Each thread moves 8 float4 per trip (all 8 loads issued before the first
// store), so every wave keeps 8 loads in flight.  MODE & 1: in place
// read-modify-write (else copy); MODE & 2: non-temporal hints.
template <int MODE>
__global__ __launch_bounds__(256) void k_ceiling_stream(const floatx4_t *src, floatx4_t *dst, int64_t n) {
    constexpr int U = 8;
    constexpr bool RMW = (MODE & 1) != 0, NT = (MODE & 2) != 0;
    const int64_t stride = int64_t(gridDim.x) * 256 * U;
    for (int64_t i0 = int64_t(blockIdx.x) * 256 * U + threadIdx.x; i0 < n; i0 += stride) {
        floatx4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + int64_t(u) * 256;
            if (i < n) v[u] = ld4<NT>(RMW ? dst + i : src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + int64_t(u) * 256;
            if (i < n) {
                if constexpr (RMW) v[u] = v[u] * 1.0001f + 1e-7f;
                st4<NT>(dst + i, v[u]);
            }
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

} // namespace

extern "C" m3_status_t m3_ceiling_mfma(int32_t kind, int32_t nblocks, int32_t iters, float *sink,
                                       hipStream_t stream) {
    if ((kind != 0 && kind != 1) || nblocks < 1 || iters < 1 || !sink || !aligned16(sink))
        return M3_ERR_INVALID_ARGUMENT;
    if (kind == 0) hipLaunchKernelGGL(k_ceiling_mfma<0>, dim3(nblocks), dim3(256), 0, stream, iters, sink);
    else hipLaunchKernelGGL(k_ceiling_mfma<1>, dim3(nblocks), dim3(256), 0, stream, iters, sink);
    return hipGetLastError() == hipSuccess ? M3_OK : M3_ERR_HIP;
}

extern "C" m3_status_t m3_ceiling_stream(int32_t mode, const void *src, void *dst, int64_t n,
                                         int32_t nblocks, hipStream_t stream) {
    if (mode < 0 || mode > 3 || n < 1 || nblocks < 1 || !dst || !aligned16(dst) ||
        ((mode & 1) == 0 && (!src || !aligned16(src))))
        return M3_ERR_INVALID_ARGUMENT;
    const floatx4_t *s = static_cast<const floatx4_t *>(src);
    floatx4_t *d = static_cast<floatx4_t *>(dst);
    switch (mode) {
    case 0: hipLaunchKernelGGL(k_ceiling_stream<0>, dim3(nblocks), dim3(256), 0, stream, s, d, n); break;
    case 1: hipLaunchKernelGGL(k_ceiling_stream<1>, dim3(nblocks), dim3(256), 0, stream, s, d, n); break;
    case 2: hipLaunchKernelGGL(k_ceiling_stream<2>, dim3(nblocks), dim3(256), 0, stream, s, d, n); break;
    default: hipLaunchKernelGGL(k_ceiling_stream<3>, dim3(nblocks), dim3(256), 0, stream, s, d, n); break;
    }
    return hipGetLastError() == hipSuccess ? M3_OK : M3_ERR_HIP;
}
