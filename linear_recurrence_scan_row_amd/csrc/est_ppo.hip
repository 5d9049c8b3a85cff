// est_ppo.hip -- the PPO clipped surrogate (Schulman et al. 2017), a fused
// consumer of the advantages: it normalizes them on the fly from the
// statistics rlca_gae_stats computes, and reduces the loss in the same
// launch (the last workgroup adds the per-workgroup sums, kernels.hpp).
// Every reduction runs in a fixed order, so results are reproducible bit for
// bit.
#include "kernels.hpp"

namespace rlca {

constexpr int kPpoThreads = 256;
constexpr uint32_t kPpoMaxGrid = 2048;

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
// its surrogate terms in partials, and the last one to finish writes loss.
template <bool NORM, bool GRAD, bool VEC>
__global__ __launch_bounds__(kPpoThreads) void ppo_clip_loss(
    const float *__restrict__ adv, const double *__restrict__ stats,
    const float *__restrict__ logp_new, const float *__restrict__ logp_old, float clip_eps,
    float norm_eps, int64_t M, float *__restrict__ grad, double *__restrict__ partials,
    double *__restrict__ loss) {
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
        if constexpr (NORM) {  // written by an earlier launch: coherent loads
            mean = (float)load_coherent(stats);
            scale = (float)(1.0 / (load_coherent(stats + 1) + (double)norm_eps));
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
        if constexpr (NORM) {  // written by an earlier launch: coherent loads
            mean = (float)load_coherent(stats);
            scale = (float)(1.0 / (load_coherent(stats + 1) + (double)norm_eps));
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
    // loss = -(sum of the per-workgroup surrogate sums) / M
    finish_in_last_workgroup<kPpoThreads, 1>(
        partials, acc, 0.0, [=](double s, double) { loss[0] = -s / (double)M; });
}

uint32_t ppo_grid(int64_t M) {
    const int64_t per_group = (int64_t)kPpoThreads * 4;
    const int64_t g = (M + per_group - 1) / per_group;
    return g < 1 ? 1u : g > (int64_t)kPpoMaxGrid ? kPpoMaxGrid : (uint32_t)g;
}

rlca_status launch_ppo_clip_loss(const float *adv, const double *stats, const float *logp_new,
                                 const float *logp_old, float clip_eps, float norm_eps,
                                 int64_t M, bool vec, float *grad, void *workspace,
                                 double *loss, hipStream_t stream) {
    const uint32_t grid = ppo_grid(M);
    double *partials = reinterpret_cast<double *>(static_cast<char *>(workspace) + kTicketBytes);
    void *args[] = {&adv, &stats, &logp_new, &logp_old, &clip_eps, &norm_eps,
                    &M,   &grad,  &partials, &loss};
    const bool norm = stats != nullptr, with_grad = grad != nullptr;
#define RLCA_PPO(N, G, V) (const void *)ppo_clip_loss<N, G, V>
    const void *kernels[8] = {RLCA_PPO(false, false, false), RLCA_PPO(false, false, true),
                              RLCA_PPO(false, true, false),  RLCA_PPO(false, true, true),
                              RLCA_PPO(true, false, false),  RLCA_PPO(true, false, true),
                              RLCA_PPO(true, true, false),   RLCA_PPO(true, true, true)};
#undef RLCA_PPO
    const void *kernel = kernels[(norm ? 4 : 0) + (with_grad ? 2 : 0) + (vec ? 1 : 0)];
    const hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(kPpoThreads), args, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

}  // namespace rlca
