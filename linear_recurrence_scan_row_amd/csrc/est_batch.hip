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

// Grouped kernels come in five classes (GroupClass): 8-wave calls whose rows
// end at wave boundaries (wave-local), light or importance-weighted; other
// 8-wave calls; one-wave calls; calls over skewed windows.  Each class
// kernel holds only its own bodies, so the light wave-local bodies of
// short-row batches are not held to the register count of the heavier ones.
// S: storage type of every member's real-valued arrays (float also carries
// the int32 prefix sums).
template <typename S, int CLASS>
__global__ __launch_bounds__(kGroupWaves * kWave)
__attribute__((amdgpu_waves_per_eu(kGroupClassWaves[CLASS], 8)))
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
    constexpr bool kWide = sizeof(S) == 4;  // int32 sums only travel in the 4-byte group

    if constexpr (CLASS == kGroupSkew) {
        switch (variant) {
#define RLCA_BS(EST, TR)                                                                     \
    case grouped_skew_backward_variant(EST, TR): {                                           \
        BackwardParams p = a.calls[c].b;                                                     \
        backward_body<EST, TR, kVecSkew, kGroupWaves, false, kFull, S>(p, wg,                \
                                                                      p.geo.num_groups);     \
        return;                                                                              \
    }
#define RLCA_FS(V, ST, INT, AD)                                                              \
    case grouped_skew_forward_variant(INT, AD): {                                            \
        if constexpr (!INT || kWide) {                                                       \
            ForwardParams p = a.calls[c].f;                                                  \
            forward_body<V, kForwardFlags, AD, kVecSkew, kGroupWaves, false, kFull, ST>(     \
                p, wg, p.geo.num_groups);                                                    \
        }                                                                                    \
        return;                                                                              \
    }
            RLCA_BS(kGae, false) RLCA_BS(kGae, true)
            RLCA_BS(kTdLambda, false) RLCA_BS(kTdLambda, true)
            RLCA_BS(kDiscounted, false) RLCA_BS(kDiscounted, true)
            RLCA_BS(kVtrace, false) RLCA_BS(kVtrace, true)
            RLCA_BS(kRetrace, false) RLCA_BS(kRetrace, true)
            RLCA_BS(kAffineBackward, false)
            RLCA_FS(float, S, false, false) RLCA_FS(float, S, false, true)
            RLCA_FS(uint32_t, uint32_t, true, false) RLCA_FS(uint32_t, uint32_t, true, true)
#undef RLCA_FS
#undef RLCA_BS
            case kGroupedSkewAffineForward: {
                ForwardParams p = a.calls[c].f;
                forward_body<float, kForwardAffine, false, kVecSkew, kGroupWaves, false, kFull, S>(
                    p, wg, p.geo.num_groups);
                return;
            }
            default: return;
        }
    } else if constexpr (CLASS == kGroupOneWave) {
        switch (variant) {
#define RLCA_B1(EST, TR)                                                                     \
    case grouped_backward_variant(EST, TR, false, true): {                                  \
        BackwardParams p = a.calls[c].b;                                                     \
        if (g1 < p.geo.num_groups)                                                           \
            backward_body<EST, TR, kVecRows, 1, false, kFull, S>(p, g1, p.geo.num_groups);      \
        return;                                                                              \
    }
#define RLCA_F1(V, ST, INT, AD)                                                              \
    case grouped_forward_variant(INT, AD, false, true): {                                   \
        if constexpr (!INT || kWide) {                                                       \
            ForwardParams p = a.calls[c].f;                                                  \
            if (g1 < p.geo.num_groups)                                                       \
                forward_body<V, kForwardFlags, AD, kVecRows, 1, false, kFull, ST>(              \
                    p, g1, p.geo.num_groups);                                                \
        }                                                                                    \
        return;                                                                              \
    }
            RLCA_B1(kGae, false) RLCA_B1(kGae, true)
            RLCA_B1(kTdLambda, false) RLCA_B1(kTdLambda, true)
            RLCA_B1(kDiscounted, false) RLCA_B1(kDiscounted, true)
            RLCA_B1(kVtrace, false) RLCA_B1(kVtrace, true)
            RLCA_B1(kRetrace, false) RLCA_B1(kRetrace, true)
            RLCA_B1(kAffineBackward, false)
            RLCA_F1(float, S, false, false) RLCA_F1(float, S, false, true)
            RLCA_F1(uint32_t, uint32_t, true, false) RLCA_F1(uint32_t, uint32_t, true, true)
#undef RLCA_F1
#undef RLCA_B1
            case grouped_affine_forward_variant(false, true): {
                ForwardParams p = a.calls[c].f;
                if (g1 < p.geo.num_groups)
                    forward_body<float, kForwardAffine, false, kVecRows, 1, false, kFull, S>(
                        p, g1, p.geo.num_groups);
                return;
            }
            default: return;
        }
    } else {
        constexpr bool WL = CLASS != kGroupWaves8;
        // light and weighted bodies of the wave-local classes
        constexpr bool kLight = CLASS != kGroupWaveLocalWeighted;
        constexpr bool kWeighted = CLASS != kGroupWaveLocal;
        switch (variant) {
#define RLCA_B8(EST, TR)                                                                     \
    case grouped_backward_variant(EST, TR, WL, false): {                                    \
        constexpr bool kHeavy = EST == kVtrace || EST == kRetrace;                           \
        if constexpr (kHeavy ? kWeighted : kLight) {                                         \
            BackwardParams p = a.calls[c].b;                                                 \
            backward_body<EST, TR, kVecRows, kGroupWaves, WL, kFull, S>(p, wg,                  \
                                                                  p.geo.num_groups);        \
        }                                                                                    \
        return;                                                                              \
    }
#define RLCA_F8(V, ST, INT, AD)                                                              \
    case grouped_forward_variant(INT, AD, WL, false): {                                     \
        if constexpr ((!INT || kWide) && kLight) {                                           \
            ForwardParams p = a.calls[c].f;                                                  \
            forward_body<V, kForwardFlags, AD, kVecRows, kGroupWaves, WL, kFull, ST>(           \
                p, wg, p.geo.num_groups);                                                    \
        }                                                                                    \
        return;                                                                              \
    }
            RLCA_B8(kGae, false) RLCA_B8(kGae, true)
            RLCA_B8(kTdLambda, false) RLCA_B8(kTdLambda, true)
            RLCA_B8(kDiscounted, false) RLCA_B8(kDiscounted, true)
            RLCA_B8(kVtrace, false) RLCA_B8(kVtrace, true)
            RLCA_B8(kRetrace, false) RLCA_B8(kRetrace, true)
            RLCA_B8(kAffineBackward, false)
            RLCA_F8(float, S, false, false) RLCA_F8(float, S, false, true)
            RLCA_F8(uint32_t, uint32_t, true, false) RLCA_F8(uint32_t, uint32_t, true, true)
#undef RLCA_F8
#undef RLCA_B8
            case grouped_affine_forward_variant(WL, false): {
                if constexpr (kLight) {
                    ForwardParams p = a.calls[c].f;
                    forward_body<float, kForwardAffine, false, kVecRows, kGroupWaves, WL, kFull, S>(
                        p, wg, p.geo.num_groups);
                }
                return;
            }
            default: return;
        }
    }
}

template <typename S>
static const void *grouped_kernel(int cls) {
    switch (cls) {
        case kGroupWaveLocal: return (const void *)grouped_scan<S, kGroupWaveLocal>;
        case kGroupWaveLocalWeighted:
            return (const void *)grouped_scan<S, kGroupWaveLocalWeighted>;
        case kGroupWaves8: return (const void *)grouped_scan<S, kGroupWaves8>;
        case kGroupSkew: return (const void *)grouped_scan<S, kGroupSkew>;
        default: return (const void *)grouped_scan<S, kGroupOneWave>;
    }
}

rlca_status launch_grouped(const GroupedLaunch &launch, int storage, int cls,
                           hipStream_t stream) {
    GroupedLaunch l = launch;
    void *argv[kMaxGroupedCalls + 1];
    for (int i = 0; i < kMaxGroupedCalls; ++i) argv[i] = &l.head[i];
    argv[kMaxGroupedCalls] = &l.args;
    const void *kernel = storage == kStoreBF16  ? grouped_kernel<__bf16>(cls)
                         : storage == kStoreF16 ? grouped_kernel<_Float16>(cls)
                                                : grouped_kernel<float>(cls);
    const hipError_t e = hipLaunchKernel(kernel, dim3(l.workgroups), dim3(kGroupWaves * kWave),
                                         argv, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

}  // namespace rlca
