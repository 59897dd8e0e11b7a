// k_prefill_f32_n16_blk_qs.hip -- instantiations of the block prologue/epilogue variant of the fused prefill kernel for
// fp32 I/O, N = 16, chunks of 64/R tokens (32 for R = 2, 3; 16 for R = 4).
#include "k_prefill.hpp"

namespace m3 {

hipError_t launch_prefill_f32_n16_blk_qs(const PrefillParams &p, bool out, hipStream_t s) {
    return launch_prefill_np<float, 16, true, true>(p, out, s);
}

} // namespace m3
