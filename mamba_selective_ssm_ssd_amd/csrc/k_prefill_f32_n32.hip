// k_prefill_f32_n32.hip -- instantiations of the fused prefill kernel for
// fp32 I/O, N = 32, 64-token chunks.
#include "k_prefill.hpp"

namespace m3 {

hipError_t launch_prefill_f32_n32(const PrefillParams &p, bool out, hipStream_t s) {
    return launch_prefill_np<float, 32, false, false>(p, out, s);
}

} // namespace m3
