// m3_noalloc.hip -- m3_ssm_prefill_noalloc (include/m3_ssm_noalloc.h): the
// prefill with its workspace in a static device array instead of a caller's
// buffer, for callers that cannot allocate.
#include "m3_ssm_noalloc.h"

#include <hip/hip_runtime.h>

#include <mutex>

// The workspace of every m3_ssm_prefill_noalloc call on a device.  In host
// code this name is only a stand-in for the symbol: its device address is
// looked up per device (hipGetSymbolAddress) and only that address is passed
// to the kernels.
static __device__ __align__(256) unsigned char scratch[M3_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of scratch, per device (null: not looked up yet)

// Device address of scratch on the current device, looked up on the first
// call with that device current; null on failure.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

} // namespace

extern "C" m3_status_t m3_ssm_prefill_noalloc(const m3_shape_t *shape, const void *x, const void *dt,
                                              const float *A, const void *lam, const void *theta,
                                              const void *B, const void *C, const m3_state_t *init,
                                              m3_state_t *final_state, void *y, hipStream_t stream) {
    const size_t need = m3_ssm_prefill_workspace_bytes(shape);
    if (need == 0) {
        // invalid or unsupported shape: m3_ssm_prefill reports which
        return m3_ssm_prefill(shape, x, dt, A, lam, theta, B, C, init, final_state, y, nullptr, 0, stream);
    }
    if (need > M3_NOALLOC_SCRATCH_BYTES) return M3_ERR_WORKSPACE;
    void *ws = scratch_ptr();
    if (!ws) return M3_ERR_HIP;
    return m3_ssm_prefill(shape, x, dt, A, lam, theta, B, C, init, final_state, y, ws,
                          M3_NOALLOC_SCRATCH_BYTES, stream);
}
