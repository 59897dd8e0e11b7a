// k_prefill_bf16_n32_blk.hip -- instantiations of the block prologue/epilogue variant of the fused prefill kernel for
// bf16 I/O, N = 32, 64-token chunks.
#include "k_prefill.hpp"

namespace m3 {

hipError_t launch_prefill_bf16_n32_blk(const PrefillParams &p, bool out, hipStream_t s) {
    return launch_prefill_np<bf16, 32, true, false>(p, out, s);
}

} // namespace m3
