// est_batch.hip -- the grouped kernel: several estimator calls in one launch.
#include "kernels.hpp"

namespace rlca {

static_assert(kMaxGrid < kHeadEndMask, "workgroup indices must stay below the unused-call mark");
// gfx950 preloads at most 14 kernel-argument dwords (user SGPRs 2..15).
static_assert(kMaxGroupedCalls == 14, "the head is 14 preloaded kernel-argument words");

#define RLCA_HEAD_ARGS                                                                         \
    uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3, uint32_t h4, uint32_t h5, uint32_t h6, \
        uint32_t h7, uint32_t h8, uint32_t h9, uint32_t h10, uint32_t h11, uint32_t h12,       \
        uint32_t h13

// S: storage type of every member's real-valued arrays (float also carries
// the int32 prefix sums).
// Eight waves per SIMD must fit: a one-shot step places eight 8-wave
// workgroups' worth of waves on every SIMD, and at seven (the occupancy the
// compiler picks on its own, for its SGPR count) an eighth of them waits
// for a second round.
template <typename S>
__global__ __launch_bounds__(kGroupWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void grouped_scan(RLCA_HEAD_ARGS, GroupedArgs a) {
    const uint32_t head[kMaxGroupedCalls] = {h0, h1, h2,  h3,  h4,  h5,  h6,
                                             h7, h8, h9, h10, h11, h12, h13};
    // The call whose workgroup range holds this workgroup: ends increase, so
    // it follows the last end at or below the workgroup index.
    const uint32_t bid = blockIdx.x;
    uint32_t c = 0, first = 0;
#pragma unroll
    for (int i = 0; i + 1 < kMaxGroupedCalls; ++i) {
        const uint32_t end = head[i] & kHeadEndMask;
        if (bid >= end) c = i + 1, first = end;
    }
    uint32_t variant = 0;
#pragma unroll
    for (int i = 0; i < kMaxGroupedCalls; ++i)
        if (c == (uint32_t)i) variant = head[i] >> kHeadVariantShift;
    const uint32_t wg = bid - first;
    // one-wave calls: wave w of the workgroup runs group 8 * wg + w
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t g1 = wg * kGroupWaves + wave;

    if (variant < 24 || (variant >= 34 && variant < 46)) {
        BackwardParams p = a.calls[c].b;
        const uint32_t once = p.geo.num_groups;  // no group loop: one pass per wave
        switch (variant) {
#define RLCA_B(EST, TR, WL)                                                                  \
    case grouped_backward_variant(EST, TR, WL, false):                                      \
        backward_body<EST, TR, true, kGroupWaves, WL, kFull, S>(p, wg, once);               \
        return;
#define RLCA_B1(EST, TR)                                                                     \
    case grouped_backward_variant(EST, TR, false, true):                                    \
        if (g1 < once) backward_body<EST, TR, true, 1, false, kFull, S>(p, g1, once);       \
        return;
#define RLCA_B_ALL(EST)                                                                      \
    RLCA_B(EST, false, false) RLCA_B(EST, false, true) RLCA_B(EST, true, false)             \
    RLCA_B(EST, true, true) RLCA_B1(EST, false) RLCA_B1(EST, true)
            RLCA_B_ALL(kGae)
            RLCA_B_ALL(kTdLambda)
            RLCA_B_ALL(kDiscounted)
            RLCA_B_ALL(kVtrace)
            RLCA_B_ALL(kRetrace)
            RLCA_B(kAffineBackward, false, false)
            RLCA_B(kAffineBackward, false, true)
            RLCA_B1(kAffineBackward, false)
#undef RLCA_B_ALL
#undef RLCA_B1
#undef RLCA_B
            default: return;
        }
    }
    ForwardParams p = a.calls[c].f;
    const uint32_t once = p.geo.num_groups;
#define RLCA_F(V, ST, INT, AD, WL)                                                           \
    case grouped_forward_variant(INT, AD, WL, false):                                       \
        forward_body<V, kForwardFlags, AD, true, kGroupWaves, WL, kFull, ST>(p, wg, once);  \
        return;
#define RLCA_F1(V, ST, INT, AD)                                                              \
    case grouped_forward_variant(INT, AD, false, true):                                     \
        if (g1 < once)                                                                       \
            forward_body<V, kForwardFlags, AD, true, 1, false, kFull, ST>(p, g1, once);     \
        return;
#define RLCA_F_ALL(V, ST, INT, AD)                                                           \
    RLCA_F(V, ST, INT, AD, false) RLCA_F(V, ST, INT, AD, true) RLCA_F1(V, ST, INT, AD)
    switch (variant) {
        RLCA_F_ALL(float, S, false, false)
        RLCA_F_ALL(float, S, false, true)
        case grouped_affine_forward_variant(false, false):
            forward_body<float, kForwardAffine, false, true, kGroupWaves, false, kFull, S>(
                p, wg, once);
            return;
        case grouped_affine_forward_variant(true, false):
            forward_body<float, kForwardAffine, false, true, kGroupWaves, true, kFull, S>(
                p, wg, once);
            return;
        case grouped_affine_forward_variant(false, true):
            if (g1 < once)
                forward_body<float, kForwardAffine, false, true, 1, false, kFull, S>(p, g1,
                                                                                     once);
            return;
        default: break;
    }
    if constexpr (sizeof(S) == 4) {  // int32 sums only travel in the 4-byte group
        switch (variant) {
            RLCA_F_ALL(uint32_t, uint32_t, true, false)
            RLCA_F_ALL(uint32_t, uint32_t, true, true)
            default: return;
        }
    }
#undef RLCA_F_ALL
#undef RLCA_F1
#undef RLCA_F
}

rlca_status launch_grouped(const GroupedLaunch &launch, int storage, hipStream_t stream) {
    GroupedLaunch l = launch;
    void *argv[kMaxGroupedCalls + 1];
    for (int i = 0; i < kMaxGroupedCalls; ++i) argv[i] = &l.head[i];
    argv[kMaxGroupedCalls] = &l.args;
    const void *kernel = storage == kStoreBF16  ? (const void *)grouped_scan<__bf16>
                         : storage == kStoreF16 ? (const void *)grouped_scan<_Float16>
                                                : (const void *)grouped_scan<float>;
    const hipError_t e = hipLaunchKernel(kernel, dim3(l.workgroups), dim3(kGroupWaves * kWave),
                                         argv, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

}  // namespace rlca
