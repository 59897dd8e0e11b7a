// k_decode_f32.hip -- instantiations of the fused decode step for f32 I/O.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t s) {
    if (p.blk.on) return launch_decode_f32_blk(p, s);
    return launch_decode_io<float, false>(p, s);
}

} // namespace m3
