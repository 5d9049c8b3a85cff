// est_retrace.hip -- kernel instantiations for one estimator (compiled in parallel).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_retrace(BackwardParams &p, const LaunchShape &s, int storage,
                           hipStream_t stream) {
    return launch_backward<kRetrace>(p, s, storage, stream);
}
}  // namespace rlca
