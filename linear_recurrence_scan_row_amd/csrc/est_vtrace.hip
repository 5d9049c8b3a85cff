// est_vtrace.hip -- kernel instantiations for one estimator (compiled in parallel).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_vtrace(BackwardParams &p, const LaunchShape &s, hipStream_t stream) {
    return launch_backward<kVtrace>(p, s, stream);
}
}  // namespace rlca
