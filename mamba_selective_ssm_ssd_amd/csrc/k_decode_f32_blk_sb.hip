// k_decode_f32_blk_sb.hip -- instantiations of the block prologue/epilogue variant of the fused decode step for f32 I/O with a bf16 carried state.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_f32_blk_sb(const DecodeParams &p, hipStream_t s) { return launch_decode_io<float, true, true>(p, s); }

} // namespace m3
