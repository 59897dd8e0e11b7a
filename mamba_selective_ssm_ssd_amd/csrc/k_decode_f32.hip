// k_decode_f32.hip -- instantiations of the fused decode step for f32 I/O
// (fp32 state, no block ops), and the dispatch to the other variants.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t s) {
    if (p.blk.on) return p.sbf16 ? launch_decode_f32_blk_sb(p, s) : launch_decode_f32_blk(p, s);
    if (p.sbf16) return launch_decode_f32_sb(p, s);
    return launch_decode_io<float, false, false>(p, s);
}

} // namespace m3
