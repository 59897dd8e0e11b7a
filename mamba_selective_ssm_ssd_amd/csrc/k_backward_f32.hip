// k_backward_f32.hip -- instantiations of the sequential backward kernel for f32 I/O.
#include "k_backward.hpp"

namespace m3 {

hipError_t launch_backward_f32(const BwdParams &p, hipStream_t s) { return launch_backward_io<float>(p, s); }

} // namespace m3
