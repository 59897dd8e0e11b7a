// k_prefill_bf16_n128_blk_qs.hip -- instantiations of the block prologue/epilogue variant of the fused prefill kernel for
// bf16 I/O, N = 128, chunks of 64/R tokens (32 for R = 2, 3; 16 for R = 4).
#include "k_prefill.hpp"

namespace m3 {

hipError_t launch_prefill_bf16_n128_blk_qs(const PrefillParams &p, bool out, hipStream_t s) {
    return launch_prefill_np<bf16, 128, true, true>(p, out, s);
}

} // namespace m3
