// est_discounted.hip -- kernel instantiations for one estimator (compiled in parallel).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_discounted(BackwardParams &p, const LaunchShape &s, int storage,
                              hipStream_t stream) {
    return launch_backward<kDiscounted>(p, s, storage, stream);
}
}  // namespace rlca
