// est_batch.hip -- the grouped kernel: several estimator calls in one launch.
#include "kernels.hpp"

namespace rlca {

__global__ __launch_bounds__(kGroupWaves * kWave) void grouped_scan(GroupedArgs a) {
    // the call whose group range holds this workgroup (uniform per workgroup)
    int c = 0;
    while (c + 1 < a.count && blockIdx.x >= a.first_group[c + 1]) ++c;
    const uint32_t g = blockIdx.x - a.first_group[c];
    const int variant = a.calls[c].variant;
    if (variant < 24) {
        BackwardParams p = a.calls[c].b;
        const uint32_t once = p.geo.num_groups;  // one group per workgroup
        switch (variant) {
#define RLCA_B(EST, TR, WL)                                                                  \
    case grouped_backward_variant(EST, TR, WL):                                             \
        backward_body<EST, TR, true, kGroupWaves, WL, kFull>(p, g, once);                   \
        return;
#define RLCA_B4(EST) RLCA_B(EST, false, false) RLCA_B(EST, false, true) RLCA_B(EST, true, false) \
    RLCA_B(EST, true, true)
            RLCA_B4(kGae)
            RLCA_B4(kTdLambda)
            RLCA_B4(kDiscounted)
            RLCA_B4(kVtrace)
            RLCA_B4(kRetrace)
            RLCA_B(kAffineBackward, false, false)
            RLCA_B(kAffineBackward, false, true)
#undef RLCA_B4
#undef RLCA_B
            default: return;
        }
    }
    ForwardParams p = a.calls[c].f;
    const uint32_t once = p.geo.num_groups;
    switch (variant) {
#define RLCA_F(V, INT, AD, WL)                                                               \
    case grouped_forward_variant(INT, AD, WL):                                              \
        forward_body<V, kForwardFlags, AD, true, kGroupWaves, WL, kFull>(p, g, once);       \
        return;
        RLCA_F(float, false, false, false)
        RLCA_F(float, false, false, true)
        RLCA_F(float, false, true, false)
        RLCA_F(float, false, true, true)
        RLCA_F(uint32_t, true, false, false)
        RLCA_F(uint32_t, true, false, true)
        RLCA_F(uint32_t, true, true, false)
        RLCA_F(uint32_t, true, true, true)
#undef RLCA_F
        case grouped_affine_forward_variant(false):
            forward_body<float, kForwardAffine, false, true, kGroupWaves, false, kFull>(p, g, once);
            return;
        case grouped_affine_forward_variant(true):
            forward_body<float, kForwardAffine, false, true, kGroupWaves, true, kFull>(p, g, once);
            return;
        default: return;
    }
}

rlca_status launch_grouped(const GroupedArgs &args, hipStream_t stream) {
    GroupedArgs a = args;
    void *argv[] = {&a};
    const hipError_t e = hipLaunchKernel((const void *)grouped_scan,
                                         dim3(a.first_group[a.count]),
                                         dim3(kGroupWaves * kWave), argv, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

}  // namespace rlca
