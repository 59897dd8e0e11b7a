// k_decode_bf16.hip -- instantiations of the fused decode step for bf16 I/O
// (fp32 state, no block ops), and the dispatch to the other variants.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_bf16(const DecodeParams &p, hipStream_t s) {
    if (p.blk.on) return p.sbf16 ? launch_decode_bf16_blk_sb(p, s) : launch_decode_bf16_blk(p, s);
    if (p.sbf16) return launch_decode_bf16_sb(p, s);
    return launch_decode_io<bf16, false, false>(p, s);
}

} // namespace m3
