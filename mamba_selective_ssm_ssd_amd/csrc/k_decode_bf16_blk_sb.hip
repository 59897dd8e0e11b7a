// k_decode_bf16_blk_sb.hip -- instantiations of the block prologue/epilogue variant of the fused decode step for bf16 I/O with a bf16 carried state.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_bf16_blk_sb(const DecodeParams &p, hipStream_t s) { return launch_decode_io<bf16, true, true>(p, s); }

} // namespace m3
