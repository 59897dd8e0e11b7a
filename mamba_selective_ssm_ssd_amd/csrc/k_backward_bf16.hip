// k_backward_bf16.hip -- instantiations of the sequential backward kernel for bf16 I/O.
#include "k_backward.hpp"

namespace m3 {

hipError_t launch_backward_bf16(const BwdParams &p, hipStream_t s) { return launch_backward_io<bf16>(p, s); }

} // namespace m3
