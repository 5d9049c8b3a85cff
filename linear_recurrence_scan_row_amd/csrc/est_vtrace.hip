// est_vtrace.hip -- kernel instantiations for one estimator (compiled in parallel).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_vtrace(BackwardParams &p, const LaunchShape &s, int storage,
                          hipStream_t stream) {
    return launch_backward<kVtrace>(p, s, storage, stream);
}
}  // namespace rlca
