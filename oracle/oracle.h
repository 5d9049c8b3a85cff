/*
 * oracle.h -- plain sequential fp64 CPU oracle for the seven credit-assignment
 * estimators.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the product path never does.
 * It shares no header, helper or constant with the HIP library.
 *
 * Source of the definitions: "rl-triton: High-Performance Triton GPU Kernels
 * for Reinforcement Learning Credit Assignment" (paperlayer.ai summary):
 *   §1 Introduction          -- the backward recurrence and its forward mirror,
 *   §2.1 Motivation          -- GAE as a strict T-step chain,
 *   §3.2 Episode-boundary    -- termination, truncation, rollout-window edge,
 *   §3.3 Algorithm-specific  -- Retrace uses the next-step importance weight;
 *                               prefix sums are segmented forward scans,
 *   §5 Correctness analysis  -- forward resets use the previous step's done,
 *   §8 Related work          -- V-Trace (Espeholt et al. 2018) and
 *                               Retrace(lambda) (Munos et al. 2016),
 *   §6 Benchmark protocol    -- an independent sequential reference.
 *
 * Layout: every per-step array is dense row-major [num_envs, T], element
 * (n, t) at n*T + t.  fp32 inputs are widened to double exactly; flags are
 * bytes, nonzero = set.  Outputs are double (int32 for the integer prefix sum).
 * Every function walks each row strictly one step at a time.
 */
#ifndef RLCA_ORACLE_H
#define RLCA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Forward-scan reset conventions (§3.3 leaves the boundary convention of the
 * segmented forward scans configurable). */
#define ORACLE_RESET_ON_START 0   /* flag[t] = 1: step t starts a new episode      */
#define ORACLE_RESET_AFTER_DONE 1 /* flag[t-1] = 1: step t-1 ended an episode (§5) */

/* truncated / trunc_values / bootstrap may be NULL (no truncation; zero bootstrap). */
void oracle_gae(const float *rewards, const float *values, const uint8_t *terminated,
                const uint8_t *truncated, const float *trunc_values, const float *bootstrap,
                double gamma, double lam, int64_t num_envs, int64_t T,
                double *advantages, double *returns);

void oracle_td_lambda(const float *rewards, const float *values, const uint8_t *terminated,
                      const uint8_t *truncated, const float *trunc_values,
                      const float *bootstrap, double gamma, double lam, int64_t num_envs,
                      int64_t T, double *returns);

void oracle_discounted_returns(const float *rewards, const uint8_t *terminated,
                               const uint8_t *truncated, const float *trunc_values,
                               const float *bootstrap, double gamma, int64_t num_envs,
                               int64_t T, double *returns);

void oracle_vtrace(const float *rewards, const float *values, const float *behaviour_logp,
                   const float *target_logp, const uint8_t *terminated,
                   const uint8_t *truncated, const float *trunc_values,
                   const float *bootstrap, double gamma, double lam, double rho_bar,
                   double c_bar, int64_t num_envs, int64_t T, double *vs,
                   double *pg_advantages);

void oracle_retrace(const float *rewards, const float *q_values, const float *expected_q,
                    const float *behaviour_logp, const float *target_logp,
                    const uint8_t *terminated, const uint8_t *truncated,
                    const float *trunc_values, const float *bootstrap, double gamma,
                    double lam, double c_bar, int64_t num_envs, int64_t T, double *q_ret);

void oracle_eligibility_traces(const float *increments, const uint8_t *flags, int convention,
                               double gamma, double lam, int64_t num_envs, int64_t T,
                               double *traces);

void oracle_episodic_prefix_sum_f32(const float *x, const uint8_t *flags, int convention,
                                    int64_t num_envs, int64_t T, double *out);

void oracle_episodic_prefix_sum_i32(const int32_t *x, const uint8_t *flags, int convention,
                                    int64_t num_envs, int64_t T, int32_t *out);

/* First-order affine recurrence over caller-built coefficients (summary §4,
 * the generic kernel on precomputed alpha and beta):
 *   backward (direction 0): A_t = alpha_t + beta_t * A_{t+1},  A_T = carry[n]
 *   forward  (direction 1): A_t = alpha_t + beta_t * A_{t-1},  A_{-1} = carry[n]
 * carry may be NULL (zero). */
void oracle_affine_scan(const float *alpha, const float *beta, const float *carry, int direction,
                        int64_t num_envs, int64_t T, double *out);

/* ---- fused consumers of the advantages (summary §9 Discussion and Future
 * Work names fused loss operations; the definitions below are the standard
 * ones the pages leave implicit). */

/* Mean and sample standard deviation (divisor M - 1; 0 when M < 2) of
 * x[0..M), in two passes: the mean, then the squared deviations from it. */
void oracle_mean_std(const double *x, int64_t M, double *mean, double *std);

/* PPO clipped surrogate (Schulman et al. 2017, "Proximal Policy Optimization
 * Algorithms", the L^CLIP objective) over M steps, as a loss to minimize:
 *   A_hat_t = normalize ? (A_t - mean) / (std + norm_eps) : A_t
 *   rho_t   = exp(logp_new_t - logp_old_t)
 *   loss    = -(1/M) sum_t min(rho_t A_hat_t, clip(rho_t, 1-eps, 1+eps) A_hat_t)
 *   grad_t  = d loss / d logp_new_t
 *           = -(1/M) rho_t A_hat_t where the unclipped term is the smaller
 *             of the two (ties included), 0 where the clipped one is.
 * grad may be NULL. */
void oracle_ppo_clip_loss(const float *adv, const float *logp_new, const float *logp_old,
                          int64_t M, int normalize, double mean, double std, double norm_eps,
                          double clip_eps, double *loss, double *grad);

#ifdef __cplusplus
}
#endif

#endif
