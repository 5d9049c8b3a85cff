// est_ppo.hip -- fused consumers of the advantages: the final reduction of
// the statistics the GAE epilogue leaves per workgroup, and the PPO clipped
// surrogate (Schulman et al. 2017), which normalizes the advantages on the fly
// from those statistics and reduces the loss per workgroup.  Every reduction
// runs in a fixed order, so results are reproducible bit for bit.
#include "kernels.hpp"

namespace rlca {

constexpr int kFinishThreads = 4 * kWave;
constexpr int kFinishBatch = 16;  // independent loads in flight per lane
constexpr int kPpoThreads = 256;
constexpr uint32_t kPpoMaxGrid = 2048;

// Sum of `count` (a, b) pairs (b skipped when stride is 1) in fixed order:
// strided per lane in batches of independent loads, then across the
// workgroup.  One workgroup.
__device__ __forceinline__ void sum_pairs(const double *pairs, uint32_t count, int stride,
                                          double &a, double &b) {
    a = 0.0;
    b = 0.0;
    for (uint32_t i0 = threadIdx.x; i0 < count; i0 += kFinishThreads * kFinishBatch) {
        double va[kFinishBatch], vb[kFinishBatch];
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) {
            const uint32_t i = i0 + k * kFinishThreads;
            va[k] = i < count ? pairs[(size_t)i * stride] : 0.0;
            vb[k] = i < count && stride == 2 ? pairs[(size_t)i * 2 + 1] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) {
            a += va[k];
            b += vb[k];
        }
    }
    workgroup_sum2<kFinishThreads / kWave>(a, b);
}

// stats = {mean, sample std (divisor M - 1; 0 when M < 2)} from the (sum,
// sum of squares) partials.
__global__ __launch_bounds__(kFinishThreads) void finish_stats(const double *partials,
                                                               uint32_t count, int64_t M,
                                                               double *stats) {
    double s1, s2;
    sum_pairs(partials, count, 2, s1, s2);
    if (threadIdx.x == 0) {
        const double mean = s1 / (double)M;
        const double var = M > 1 ? fmax(s2 - s1 * mean, 0.0) / (double)(M - 1) : 0.0;
        stats[0] = mean;
        stats[1] = sqrt(var);
    }
}

// loss = -(sum of the per-workgroup surrogate sums) / M.
__global__ __launch_bounds__(kFinishThreads) void finish_loss(const double *partials,
                                                              uint32_t count, int64_t M,
                                                              double *loss) {
    double s, unused;
    sum_pairs(partials, count, 1, s, unused);
    if (threadIdx.x == 0) loss[0] = -s / (double)M;
}

// One step of the clipped surrogate: returns min(rho A, clip(rho) A) and sets
// the gradient of the loss in logp_new (-rho A / M on the unclipped branch,
// ties included; 0 on the clipped one).
__device__ __forceinline__ float ppo_term(float a, float lp_new, float lp_old, float lo, float hi,
                                          float neg_inv_m, float &grad) {
    const float rho = expf(lp_new - lp_old);
    const float unclipped = rho * a;
    const float clipped = clip_to(rho, lo, hi) * a;  // a NaN ratio stays NaN
    const bool take = unclipped <= clipped;
    grad = take ? unclipped * neg_inv_m : 0.f;
    return take ? unclipped : clipped;
}

// NORM: A_hat = (A - mean) * 1/(std + norm_eps) from stats; VEC: four steps
// per load (16-byte aligned arrays), the last M % 4 steps one per lane of
// workgroup 0.  Grid-stride over the steps; each workgroup leaves the sum of
// its surrogate terms in partials.
template <bool NORM, bool GRAD, bool VEC>
__global__ __launch_bounds__(kPpoThreads) void ppo_clip_loss(
    const float *__restrict__ adv, const double *__restrict__ stats,
    const float *__restrict__ logp_new, const float *__restrict__ logp_old, float clip_eps,
    float norm_eps, int64_t M, float *__restrict__ grad, double *__restrict__ partials) {
    const float lo = 1.f - clip_eps, hi = 1.f + clip_eps;
    const float neg_inv_m = (float)(-1.0 / (double)M);
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kPpoThreads;
    float mean = 0.f, scale = 1.f;
    if constexpr (VEC) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const int64_t n4 = M / 4;
        // Each input is read once (non-temporal loads).  A lane's first
        // block goes out before the statistics are read: they come from the
        // previous launch, and waiting for them first would put one more
        // memory round trip ahead of every wave's loads.
        int64_t i = (int64_t)blockIdx.x * kPpoThreads + threadIdx.x;
        f4 a = {}, pn = {}, po = {};
        if (i < n4) {
            a = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(adv) + i);
            pn = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(logp_new) + i);
            po = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(logp_old) + i);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NORM) {
            mean = (float)stats[0];
            scale = (float)(1.0 / (stats[1] + (double)norm_eps));
        }
        while (i < n4) {
            f4 g;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float ah = NORM ? (a[k] - mean) * scale : a[k];
                float gk;
                acc += (double)ppo_term(ah, pn[k], po[k], lo, hi, neg_inv_m, gk);
                g[k] = gk;
            }
            if constexpr (GRAD) __builtin_nontemporal_store(g, reinterpret_cast<f4 *>(grad) + i);
            i += stride;
            if (i < n4) {
                a = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(adv) + i);
                pn = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(logp_new) + i);
                po = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(logp_old) + i);
            }
        }
        const int64_t j = 4 * n4 + threadIdx.x;  // the last M % 4 steps
        if (blockIdx.x == 0 && j < M) {
            const float ah = NORM ? (adv[j] - mean) * scale : adv[j];
            float g;
            acc += (double)ppo_term(ah, logp_new[j], logp_old[j], lo, hi, neg_inv_m, g);
            if constexpr (GRAD) grad[j] = g;
        }
    } else {
        if constexpr (NORM) {
            mean = (float)stats[0];
            scale = (float)(1.0 / (stats[1] + (double)norm_eps));
        }
        for (int64_t i = (int64_t)blockIdx.x * kPpoThreads + threadIdx.x; i < M; i += stride) {
            const float ah = NORM ? (adv[i] - mean) * scale : adv[i];
            float g;
            acc += (double)ppo_term(ah, logp_new[i], logp_old[i], lo, hi, neg_inv_m, g);
            if constexpr (GRAD) grad[i] = g;
        }
    }
    double unused = 0.0;
    workgroup_sum2<kPpoThreads / kWave>(acc, unused);
    if (threadIdx.x == 0) partials[blockIdx.x] = acc;
}

rlca_status launch_finish_stats(const double *partials, uint32_t count, int64_t M,
                                double *stats, hipStream_t stream) {
    void *args[] = {&partials, &count, &M, &stats};
    const hipError_t e = hipLaunchKernel((const void *)finish_stats, dim3(1),
                                         dim3(kFinishThreads), args, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

uint32_t ppo_grid(int64_t M) {
    const int64_t per_group = (int64_t)kPpoThreads * 4;
    const int64_t g = (M + per_group - 1) / per_group;
    return g < 1 ? 1u : g > (int64_t)kPpoMaxGrid ? kPpoMaxGrid : (uint32_t)g;
}

rlca_status launch_ppo_clip_loss(const float *adv, const double *stats, const float *logp_new,
                                 const float *logp_old, float clip_eps, float norm_eps,
                                 int64_t M, bool vec, float *grad, double *partials,
                                 double *loss, hipStream_t stream) {
    const uint32_t grid = ppo_grid(M);
    void *args[] = {&adv, &stats, &logp_new, &logp_old, &clip_eps, &norm_eps,
                    &M,   &grad,  &partials};
    const bool norm = stats != nullptr, with_grad = grad != nullptr;
#define RLCA_PPO(N, G, V) (const void *)ppo_clip_loss<N, G, V>
    const void *kernels[8] = {RLCA_PPO(false, false, false), RLCA_PPO(false, false, true),
                              RLCA_PPO(false, true, false),  RLCA_PPO(false, true, true),
                              RLCA_PPO(true, false, false),  RLCA_PPO(true, false, true),
                              RLCA_PPO(true, true, false),   RLCA_PPO(true, true, true)};
#undef RLCA_PPO
    const void *kernel = kernels[(norm ? 4 : 0) + (with_grad ? 2 : 0) + (vec ? 1 : 0)];
    hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(kPpoThreads), args, 0, stream);
    if (e != hipSuccess) return RLCA_ERR_HIP;
    uint32_t count = grid;
    const double *cp = partials;
    void *fargs[] = {&cp, &count, &M, &loss};
    e = hipLaunchKernel((const void *)finish_loss, dim3(1), dim3(kFinishThreads), fargs, 0,
                        stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

}  // namespace rlca
