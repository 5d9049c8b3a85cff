// est_td_lambda.hip -- kernel instantiations for one estimator (compiled in parallel).
#include "kernels.hpp"

namespace rlca {
rlca_status launch_td_lambda(BackwardParams &p, const LaunchShape &s, int storage,
                             hipStream_t stream) {
    return launch_backward<kTdLambda>(p, s, storage, stream);
}
}  // namespace rlca
