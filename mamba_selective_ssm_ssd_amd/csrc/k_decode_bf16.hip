// k_decode_bf16.hip -- instantiations of the fused decode step for bf16 I/O.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_bf16(const DecodeParams &p, hipStream_t s) {
    if (p.blk.on) return launch_decode_bf16_blk(p, s);
    return launch_decode_io<bf16, false>(p, s);
}

} // namespace m3
