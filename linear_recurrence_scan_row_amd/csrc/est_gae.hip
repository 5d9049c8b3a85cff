// est_gae.hip -- kernel instantiations for one estimator (compiled in parallel).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_gae(BackwardParams &p, const LaunchShape &s, int storage,
                       hipStream_t stream) {
    return launch_backward<kGae>(p, s, storage, stream);
}
rlca_status launch_gae_stats(BackwardParams &p, const LaunchShape &s, hipStream_t stream) {
    return p.truncated != nullptr ? launch_backward_variant<kGae, true, float, true>(p, s, stream)
                                  : launch_backward_variant<kGae, false, float, true>(p, s, stream);
}
}  // namespace rlca
