// est_affine.hip -- kernel instantiations for the generic affine scan (the
// caller supplies alpha and beta), both directions.
#include "kernels.hpp"

namespace rlca {
rlca_status launch_affine_backward(BackwardParams &p, const LaunchShape &s, hipStream_t stream) {
    return launch_backward_variant<kAffineBackward, false>(p, s, stream);
}
rlca_status launch_affine_forward(ForwardParams &p, const LaunchShape &s, hipStream_t stream) {
    return launch_forward_variant<float, kForwardAffine, false>(p, s, stream);
}
}  // namespace rlca
