// est_forward.hip -- forward-scan kernel instantiations (traces, prefix sums).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_forward_float(ForwardParams &p, bool after_done, const LaunchShape &s,
                                 int storage, hipStream_t stream) {
    return after_done ? launch_forward_float<kForwardFlags, true>(p, s, storage, stream)
                      : launch_forward_float<kForwardFlags, false>(p, s, storage, stream);
}
rlca_status launch_forward_u32(ForwardParams &p, bool after_done, const LaunchShape &s,
                               hipStream_t stream) {
    return after_done
               ? launch_forward_variant<uint32_t, kForwardFlags, true, uint32_t>(p, s, stream)
               : launch_forward_variant<uint32_t, kForwardFlags, false, uint32_t>(p, s, stream);
}
}  // namespace rlca
