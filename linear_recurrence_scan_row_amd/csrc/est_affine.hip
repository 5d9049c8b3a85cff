// est_affine.hip -- kernel instantiations for the generic affine scan (the
// caller supplies alpha and beta), both directions.
#include "kernels.hpp"

namespace rlca {
rlca_status launch_affine_backward(BackwardParams &p, const LaunchShape &s, int storage,
                                   hipStream_t stream) {
    switch (storage) {
        case kStoreBF16:
            return launch_backward_variant<kAffineBackward, false, __bf16>(p, s, stream);
        case kStoreF16:
            return launch_backward_variant<kAffineBackward, false, _Float16>(p, s, stream);
        default: return launch_backward_variant<kAffineBackward, false, float>(p, s, stream);
    }
}
rlca_status launch_affine_forward(ForwardParams &p, const LaunchShape &s, int storage,
                                  hipStream_t stream) {
    return launch_forward_float<kForwardAffine, false>(p, s, storage, stream);
}
}  // namespace rlca
