// k_prefill_bf16_n32_blk.hip -- instantiations of the block prologue/epilogue variant of the fused prefill kernel for bf16 I/O, N = 32.
#include "k_prefill.hpp"

namespace m3 {

template <int P>
static hipError_t by_rank(const PrefillParams &p, bool out, hipStream_t s) {
    switch (p.R) {
    case 1: return out ? launch_prefill_inst<bf16, 32, P, 1, true, true>(p, s) : launch_prefill_inst<bf16, 32, P, 1, false, true>(p, s);
    case 2: return out ? launch_prefill_inst<bf16, 32, P, 2, true, true>(p, s) : launch_prefill_inst<bf16, 32, P, 2, false, true>(p, s);
    case 3: return out ? launch_prefill_inst<bf16, 32, P, 3, true, true>(p, s) : launch_prefill_inst<bf16, 32, P, 3, false, true>(p, s);
    case 4: return out ? launch_prefill_inst<bf16, 32, P, 4, true, true>(p, s) : launch_prefill_inst<bf16, 32, P, 4, false, true>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_n32_blk(const PrefillParams &p, bool out, hipStream_t s) {
    switch (p.P) {
    case 16: return by_rank<16>(p, out, s);
    case 32: return by_rank<32>(p, out, s);
    case 64: return by_rank<64>(p, out, s);
    }
    return hipErrorInvalidValue;
}

} // namespace m3
