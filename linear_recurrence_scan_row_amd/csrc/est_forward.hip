// est_forward.hip -- forward-scan kernel instantiations (traces, prefix sums).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_forward_f32(ForwardParams &p, bool after_done, const LaunchShape &s,
                               hipStream_t stream) {
    return after_done ? launch_forward_variant<float, kForwardFlags, true>(p, s, stream)
                      : launch_forward_variant<float, kForwardFlags, false>(p, s, stream);
}
rlca_status launch_forward_u32(ForwardParams &p, bool after_done, const LaunchShape &s,
                               hipStream_t stream) {
    return after_done ? launch_forward_variant<uint32_t, kForwardFlags, true>(p, s, stream)
                      : launch_forward_variant<uint32_t, kForwardFlags, false>(p, s, stream);
}
}  // namespace rlca
