// k_prefill_f32_n128.hip -- instantiations of the fused prefill kernel for
// fp32 I/O, N = 128, 64-token chunks.
#include "k_prefill.hpp"

namespace m3 {

hipError_t launch_prefill_f32_n128(const PrefillParams &p, bool out, hipStream_t s) {
    return launch_prefill_np<float, 128, false, false>(p, out, s);
}

} // namespace m3
