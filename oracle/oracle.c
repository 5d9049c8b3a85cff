/*
 * oracle.c -- plain sequential fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Each estimator is its textbook recursion written out one step at a time, in
 * double precision, with the episode-boundary rules of the rl-triton summary
 * (paperlayer.ai page, §3.2 Episode-boundary semantics):
 *   - a terminated step has successor value 0 and cuts the backward chain;
 *   - a truncated step (terminated wins when both are set) takes the
 *     caller-supplied continuation value trunc_values[t] as its successor
 *     value and also cuts the chain, so nothing is counted twice;
 *   - the last step of the window (t = T-1), when not done, takes the row's
 *     bootstrap value as its successor value; a done last step ignores it.
 * The forward scans (eligibility traces, episodic prefix sums) restart their
 * carry at an episode boundary and never bootstrap (§3.2, §5).
 *
 * No scan, no reassociation: the oracle is the sequential reference that the
 * summary's §6 (Correctness validation) describes, not a model of any kernel.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>

/* V-Trace / Retrace clamp of the log importance ratio before exp(). */
#define ORACLE_LOG_RATIO_CLIP 5.0

/* Boundary resolution of step t of one row.
 * Returns 1 when the backward chain continues past t (step t is not done and is
 * not the window's last step); writes the successor value to *next_value when
 * the chain stops (0 / continuation / bootstrap).  When the chain continues the
 * caller uses the next step's own value instead. */
static int resolve_step(const uint8_t *term, const uint8_t *trunc, const float *trunc_values,
                        double bootstrap, int64_t t, int64_t T, double *next_value)
{
    if (term[t]) {
        *next_value = 0.0;
        return 0;
    }
    if (trunc != NULL && trunc[t]) {
        *next_value = (double)trunc_values[t];
        return 0;
    }
    if (t == T - 1) {
        *next_value = bootstrap;
        return 0;
    }
    *next_value = 0.0; /* unused: the successor is step t+1 itself */
    return 1;
}

static double row_bootstrap(const float *bootstrap, int64_t n)
{
    return bootstrap != NULL ? (double)bootstrap[n] : 0.0;
}

static double clipped_ratio(float target_logp, float behaviour_logp)
{
    double l = (double)target_logp - (double)behaviour_logp;
    if (l > ORACLE_LOG_RATIO_CLIP) l = ORACLE_LOG_RATIO_CLIP;
    if (l < -ORACLE_LOG_RATIO_CLIP) l = -ORACLE_LOG_RATIO_CLIP;
    return exp(l);
}

static double min_d(double a, double b) { return a < b ? a : b; }

/* The carried term of a recurrence: coefficient times the value carried from
 * the neighbouring step.  A zero coefficient severs the chain, so the term is
 * 0 whatever the carried value is, NaN or infinite included (summary §5
 * Correctness analysis: a step with beta = 0 composes to (alpha, 0), and
 * nothing beyond it reaches the result).  For finite values this is plain
 * multiplication. */
static double carried(double coef, double value) { return coef == 0.0 ? 0.0 : coef * value; }

/* GAE (Schulman et al. 2016; summary §2.1):
 *   delta_t = r_t + gamma * V(s_{t+1}) - V(s_t)
 *   A_t     = delta_t + gamma * lambda * A_{t+1}   (chain cut at a boundary)
 *   returns = A_t + V(s_t)                                                   */
void oracle_gae(const float *rewards, const float *values, const uint8_t *terminated,
                const uint8_t *truncated, const float *trunc_values, const float *bootstrap,
                double gamma, double lam, int64_t num_envs, int64_t T,
                double *advantages, double *returns)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *r = rewards + n * T, *v = values + n * T;
        const uint8_t *term = terminated + n * T;
        const uint8_t *trunc = truncated ? truncated + n * T : NULL;
        const float *tv = trunc_values ? trunc_values + n * T : NULL;
        double b = row_bootstrap(bootstrap, n);
        double next_adv = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double nv;
            int cont = resolve_step(term, trunc, tv, b, t, T, &nv);
            double delta, adv;
            if (cont) {
                delta = (double)r[t] + gamma * (double)v[t + 1] - (double)v[t];
                adv = delta + carried(gamma * lam, next_adv);
            } else {
                delta = (double)r[t] + gamma * nv - (double)v[t];
                adv = delta;
            }
            advantages[n * T + t] = adv;
            if (returns) returns[n * T + t] = adv + (double)v[t];
            next_adv = adv;
        }
    }
}

/* TD(lambda) return, backward (recursive) form:
 *   G_t = r_t + gamma * ((1 - lambda) * V(s_{t+1}) + lambda * G_{t+1})
 * and at a boundary G_t = r_t + gamma * successor value.                     */
void oracle_td_lambda(const float *rewards, const float *values, const uint8_t *terminated,
                      const uint8_t *truncated, const float *trunc_values,
                      const float *bootstrap, double gamma, double lam, int64_t num_envs,
                      int64_t T, double *returns)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *r = rewards + n * T, *v = values + n * T;
        const uint8_t *term = terminated + n * T;
        const uint8_t *trunc = truncated ? truncated + n * T : NULL;
        const float *tv = trunc_values ? trunc_values + n * T : NULL;
        double b = row_bootstrap(bootstrap, n);
        double next_g = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double nv, g;
            if (resolve_step(term, trunc, tv, b, t, T, &nv))
                g = (double)r[t] + gamma * (1.0 - lam) * (double)v[t + 1] +
                    carried(gamma * lam, next_g);
            else
                g = (double)r[t] + gamma * nv;
            returns[n * T + t] = g;
            next_g = g;
        }
    }
}

/* Discounted return: G_t = r_t + gamma * G_{t+1}; at a boundary
 * G_t = r_t + gamma * successor value (0 / continuation / bootstrap).        */
void oracle_discounted_returns(const float *rewards, const uint8_t *terminated,
                               const uint8_t *truncated, const float *trunc_values,
                               const float *bootstrap, double gamma, int64_t num_envs,
                               int64_t T, double *returns)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *r = rewards + n * T;
        const uint8_t *term = terminated + n * T;
        const uint8_t *trunc = truncated ? truncated + n * T : NULL;
        const float *tv = trunc_values ? trunc_values + n * T : NULL;
        double b = row_bootstrap(bootstrap, n);
        double next_g = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double nv, g;
            if (resolve_step(term, trunc, tv, b, t, T, &nv))
                g = (double)r[t] + carried(gamma, next_g);
            else
                g = (double)r[t] + gamma * nv;
            returns[n * T + t] = g;
            next_g = g;
        }
    }
}

/* V-Trace (Espeholt et al. 2018, summary §8):
 *   rho_t = min(rho_bar, pi/mu), c_t = lambda * min(c_bar, pi/mu)
 *   delta_t = rho_t * (r_t + gamma * V(s_{t+1}) - V(s_t))
 *   vs_t - V(s_t) = delta_t + gamma * c_t * (vs_{t+1} - V(s_{t+1}))
 *   pg_t = rho_t * (r_t + gamma * vs_{t+1} - V(s_t))
 * At a boundary vs_{t+1} is replaced by the successor value.                 */
void oracle_vtrace(const float *rewards, const float *values, const float *behaviour_logp,
                   const float *target_logp, const uint8_t *terminated,
                   const uint8_t *truncated, const float *trunc_values,
                   const float *bootstrap, double gamma, double lam, double rho_bar,
                   double c_bar, int64_t num_envs, int64_t T, double *vs,
                   double *pg_advantages)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *r = rewards + n * T, *v = values + n * T;
        const float *mu = behaviour_logp + n * T, *pi = target_logp + n * T;
        const uint8_t *term = terminated + n * T;
        const uint8_t *trunc = truncated ? truncated + n * T : NULL;
        const float *tv = trunc_values ? trunc_values + n * T : NULL;
        double b = row_bootstrap(bootstrap, n);
        double next_vs = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double ratio = clipped_ratio(pi[t], mu[t]);
            double rho = min_d(rho_bar, ratio);
            double c = lam * min_d(c_bar, ratio);
            double nv, vs_t;
            if (resolve_step(term, trunc, tv, b, t, T, &nv)) {
                double delta = rho * ((double)r[t] + gamma * (double)v[t + 1] - (double)v[t]);
                vs_t = (double)v[t] + delta + carried(gamma * c, next_vs - (double)v[t + 1]);
                /* pg_t = rho (r_t + gamma vs_{t+1} - V_t): its carried term is
                 * rho gamma (vs_{t+1} - V_{t+1}) on top of rho's TD error */
                if (pg_advantages)
                    pg_advantages[n * T + t] =
                        rho * ((double)r[t] + gamma * (double)v[t + 1] - (double)v[t]) +
                        carried(rho * gamma, next_vs - (double)v[t + 1]);
            } else {
                double delta = rho * ((double)r[t] + gamma * nv - (double)v[t]);
                vs_t = (double)v[t] + delta;
                if (pg_advantages) pg_advantages[n * T + t] = delta;
            }
            vs[n * T + t] = vs_t;
            next_vs = vs_t;
        }
    }
}

/* Retrace(lambda) (Munos et al. 2016, summary §3.3 and §8):
 *   Qret_t = r_t + gamma * E_pi Q(s_{t+1}, .)
 *            + gamma * c_{t+1} * (Qret_{t+1} - Q(s_{t+1}, a_{t+1}))
 *   c_t = lambda * min(c_bar, pi/mu)
 * expected_q[t] holds E_pi Q(s_t, .); at a boundary E_pi Q(s_{t+1}, .) is the
 * successor value (0 at termination, trunc_values[t] at truncation, the
 * bootstrap at the window edge) and the correction term is dropped.         */
void oracle_retrace(const float *rewards, const float *q_values, const float *expected_q,
                    const float *behaviour_logp, const float *target_logp,
                    const uint8_t *terminated, const uint8_t *truncated,
                    const float *trunc_values, const float *bootstrap, double gamma,
                    double lam, double c_bar, int64_t num_envs, int64_t T, double *q_ret)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *r = rewards + n * T, *q = q_values + n * T, *eq = expected_q + n * T;
        const float *mu = behaviour_logp + n * T, *pi = target_logp + n * T;
        const uint8_t *term = terminated + n * T;
        const uint8_t *trunc = truncated ? truncated + n * T : NULL;
        const float *tv = trunc_values ? trunc_values + n * T : NULL;
        double b = row_bootstrap(bootstrap, n);
        double next_qret = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double nv, qr;
            if (resolve_step(term, trunc, tv, b, t, T, &nv)) {
                double c_next = lam * min_d(c_bar, clipped_ratio(pi[t + 1], mu[t + 1]));
                qr = (double)r[t] + gamma * (double)eq[t + 1] +
                     carried(gamma * c_next, next_qret - (double)q[t + 1]);
            } else {
                qr = (double)r[t] + gamma * nv;
            }
            q_ret[n * T + t] = qr;
            next_qret = qr;
        }
    }
}

/* Step t starts a fresh episode under the given convention (t = 0 always does:
 * the forward carry starts at zero, summary §3.1 / §5). */
static int starts_episode(const uint8_t *flags, int convention, int64_t t)
{
    if (t == 0) return 1;
    if (convention == ORACLE_RESET_AFTER_DONE) return flags[t - 1] != 0;
    return flags[t] != 0;
}

/* Accumulating eligibility trace: e_t = x_t + gamma * lambda * e_{t-1},
 * restarted (e_{t-1} := 0) at an episode start.                              */
void oracle_eligibility_traces(const float *increments, const uint8_t *flags, int convention,
                               double gamma, double lam, int64_t num_envs, int64_t T,
                               double *traces)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *x = increments + n * T;
        const uint8_t *f = flags + n * T;
        double e = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            if (starts_episode(f, convention, t)) e = 0.0;
            e = (double)x[t] + carried(gamma * lam, e);
            traces[n * T + t] = e;
        }
    }
}

/* Inclusive segmented prefix sum: S_t = x_t + S_{t-1}, restarted at an
 * episode start (summary §3.3).                                              */
void oracle_episodic_prefix_sum_f32(const float *x, const uint8_t *flags, int convention,
                                    int64_t num_envs, int64_t T, double *out)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const uint8_t *f = flags + n * T;
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            if (starts_episode(f, convention, t)) s = 0.0;
            s += (double)x[n * T + t];
            out[n * T + t] = s;
        }
    }
}

/* Integer variant: the running sum is kept in int64 and each output is that
 * sum reduced modulo 2^32 into int32 (two's-complement wrap-around). */
void oracle_episodic_prefix_sum_i32(const int32_t *x, const uint8_t *flags, int convention,
                                    int64_t num_envs, int64_t T, int32_t *out)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const uint8_t *f = flags + n * T;
        int64_t s = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (starts_episode(f, convention, t)) s = 0;
            s += (int64_t)x[n * T + t];
            uint32_t low = (uint32_t)((uint64_t)s & 0xffffffffu);
            out[n * T + t] = (int32_t)(low >= 0x80000000u ? (int64_t)low - 0x100000000LL
                                                          : (int64_t)low);
        }
    }
}

/* One step of the recurrence.  beta = 0 severs the chain: the step's value
 * is alpha whatever the carried value is, NaN or infinite included (summary
 * §5 Correctness analysis: a step with beta = 0 composes to (alpha, 0)). */
static double affine_step(float a, float b, double carried)
{
    return b == 0.0f ? (double)a : (double)a + (double)b * carried;
}

/* The recurrence itself, one step at a time from the carried end. */
void oracle_affine_scan(const float *alpha, const float *beta, const float *carry, int direction,
                        int64_t num_envs, int64_t T, double *out)
{
    for (int64_t n = 0; n < num_envs; ++n) {
        const float *a = alpha + n * T, *b = beta + n * T;
        double A = carry != NULL ? (double)carry[n] : 0.0;
        if (direction == 0) {
            for (int64_t t = T - 1; t >= 0; --t) {
                A = affine_step(a[t], b[t], A);
                out[n * T + t] = A;
            }
        } else {
            for (int64_t t = 0; t < T; ++t) {
                A = affine_step(a[t], b[t], A);
                out[n * T + t] = A;
            }
        }
    }
}

/* Two passes over the data: the mean first, then the sum of squared
 * deviations from it. */
void oracle_mean_std(const double *x, int64_t M, double *mean, double *std)
{
    double s = 0.0;
    for (int64_t i = 0; i < M; ++i) s += x[i];
    const double mu = M > 0 ? s / (double)M : 0.0;
    double ss = 0.0;
    for (int64_t i = 0; i < M; ++i) ss += (x[i] - mu) * (x[i] - mu);
    *mean = mu;
    *std = M > 1 ? sqrt(ss / (double)(M - 1)) : 0.0;
}

/* The clipped surrogate term by term, then its mean. */
void oracle_ppo_clip_loss(const float *adv, const float *logp_new, const float *logp_old,
                          int64_t M, int normalize, double mean, double std, double norm_eps,
                          double clip_eps, double *loss, double *grad)
{
    double total = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        const double a = normalize ? ((double)adv[i] - mean) / (std + norm_eps) : (double)adv[i];
        const double rho = exp((double)logp_new[i] - (double)logp_old[i]);
        double clipped_rho = rho;
        if (clipped_rho < 1.0 - clip_eps) clipped_rho = 1.0 - clip_eps;
        if (clipped_rho > 1.0 + clip_eps) clipped_rho = 1.0 + clip_eps;
        const double unclipped = rho * a, clipped = clipped_rho * a;
        const int take_unclipped = unclipped <= clipped;
        total += take_unclipped ? unclipped : clipped;
        if (grad != NULL) grad[i] = take_unclipped ? -unclipped / (double)M : 0.0;
    }
    *loss = M > 0 ? -total / (double)M : 0.0;
}
