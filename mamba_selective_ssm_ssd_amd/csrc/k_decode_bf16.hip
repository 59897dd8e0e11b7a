// k_decode_bf16.hip -- instantiations of the fused decode step for bf16 I/O.
#include "k_decode.hpp"

namespace m3 {

hipError_t launch_decode_bf16(const DecodeParams &p, hipStream_t s) { return launch_decode_io<bf16>(p, s); }

} // namespace m3
