// est_forward.hip -- forward-scan kernel instantiations (traces, prefix sums).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_forward_f32(ForwardParams &p, bool after_done, const LaunchShape &s,
                               hipStream_t stream) {
    return launch_forward<float>(p, after_done, s, stream);
}
rlca_status launch_forward_u32(ForwardParams &p, bool after_done, const LaunchShape &s,
                               hipStream_t stream) {
    return launch_forward<uint32_t>(p, after_done, s, stream);
}
}  // namespace rlca
