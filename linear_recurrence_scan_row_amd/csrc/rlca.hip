// rlca.hip -- the C ABI of rlca.h: argument checks and launch-shape choice.
//
// The kernels live in kernels.hpp and are instantiated one estimator per
// translation unit (est_*.hip).  Every entry point validates its arguments
// before anything is enqueued, picks a launch shape from (num_envs, T,
// alignment) and enqueues its kernel launch(es) on the caller's stream: one
// launch, or three for a few long rows (the chunk modes).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.hpp"
#include "rlca.h"

namespace rlca {

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

static bool unit_interval(float x) { return x >= 0.f && x <= 1.f; }  // false for NaN
static bool positive_finite(float x) { return x > 0.f && isfinite(x); }

struct Span {
    const void *p;
    size_t bytes;
};

// Size checks common to all entry points.  Sets *elems to num_envs * T.
static rlca_status check_sizes(int64_t num_envs, int64_t T, int64_t *elems) {
    if (num_envs < 0 || T < 0 || T > RLCA_MAX_T || num_envs > RLCA_MAX_ENVS)
        return RLCA_ERR_INVALID_SIZE;
    if (T != 0 && num_envs > INT64_MAX / 8 / T) return RLCA_ERR_INVALID_SIZE;
    *elems = num_envs * T;
    return RLCA_OK;
}

static rlca_status check_aligned4(const void *const *ptrs, int n) {
    for (int i = 0; i < n; ++i)
        if (ptrs[i] != nullptr && ((uintptr_t)ptrs[i] & 3u) != 0) return RLCA_ERR_MISALIGNED;
    return RLCA_OK;
}

// No output may overlap an input or another output.
static rlca_status check_aliasing(const Span *outs, int nout, const Span *ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes)) return RLCA_ERR_ALIASING;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return RLCA_ERR_ALIASING;
    }
    return RLCA_OK;
}

// The vector path loads a lane's K steps with one instruction per stream: it
// needs T % K == 0 and arrays aligned to K elements.
static bool vec_ok(int64_t T, const void *const *f32, int nf, const void *const *u8, int nu) {
    if (T % kK != 0) return false;
    for (int i = 0; i < nf; ++i)
        if (f32[i] != nullptr && ((uintptr_t)f32[i] % (4 * kK)) != 0) return false;
    for (int i = 0; i < nu; ++i)
        if (u8[i] != nullptr && ((uintptr_t)u8[i] % kK) != 0) return false;
    return true;
}

// Launch shape.  Rows that end at wave boundaries (T divides the 256-step
// wave span) need no cross-wave exchange.  The wave count per workgroup was
// chosen by measurement on MI355X with cold HBM-resident operands: such short
// rows run fastest in 8-wave workgroups; rows of 257..1023 steps with one
// wave walking the row tile by tile; longer rows with 8 waves sharing each
// tile through LDS.  Fewer than 64 long rows cannot fill the chip one
// workgroup per row, so they are split into chunks that run in parallel
// (three launches, inputs read twice): 50x faster for one row of 1M steps,
// even at 64 rows, slower from 128 rows on (one workgroup per row then
// sustains 3.4-5 TB/s).
static constexpr int64_t kChunkedMaxRows = 64;

static LaunchShape choose_shape(int64_t num_envs, int64_t T, bool vec) {
    LaunchShape s;
    s.vec = vec;
    s.wave_local = vec && T <= kWave * kK && (kWave * kK) % T == 0;
    s.waves = (T <= kWave * kK || T >= 1024) ? 8 : 1;
    s.chunked = vec && T > 2 * (int64_t)kChunkSteps && num_envs < kChunkedMaxRows;
#ifdef RLCA_FORCE_WAVES
    s.waves = RLCA_FORCE_WAVES;
#endif
#ifdef RLCA_FORCE_CHUNKED
    s.chunked = vec && T > 2 * (int64_t)kChunkSteps && RLCA_FORCE_CHUNKED;
#endif
    return s;
}

static rlca_status run_backward(int est, BackwardParams &p, int64_t T, hipStream_t stream) {
    const void *f32[] = {p.rewards, p.values, p.expected_q, p.behaviour_logp, p.target_logp,
                         p.trunc_values, p.out0, p.out1};
    const void *u8[] = {p.terminated, p.truncated};
    const LaunchShape s = choose_shape(p.geo.num_envs, T, vec_ok(T, f32, 8, u8, 2));
    p.geo.T = (uint32_t)T;
    switch (est) {
        case kGae: return launch_gae(p, s, stream);
        case kTdLambda: return launch_td_lambda(p, s, stream);
        case kDiscounted: return launch_discounted(p, s, stream);
        case kVtrace: return launch_vtrace(p, s, stream);
        case kRetrace: return launch_retrace(p, s, stream);
        default: return launch_affine_backward(p, s, stream);
    }
}

// Checks shared by the five backward estimators.  `ins_f32` lists the
// required fp32 per-step inputs (all non-null).
static rlca_status check_backward(const float *const *req_f32, int nreq, const uint8_t *terminated,
                                  const uint8_t *truncated, const float *trunc_values,
                                  const float *bootstrap, float *const *outs, int nouts,
                                  bool out0_required, int64_t num_envs, int64_t T,
                                  int64_t *elems) {
    rlca_status st = check_sizes(num_envs, T, elems);
    if (st != RLCA_OK) return st;
    if (*elems == 0) return RLCA_OK;
    for (int i = 0; i < nreq; ++i)
        if (req_f32[i] == nullptr) return RLCA_ERR_NULL_POINTER;
    if (terminated == nullptr) return RLCA_ERR_NULL_POINTER;
    if (truncated != nullptr && trunc_values == nullptr) return RLCA_ERR_NULL_POINTER;
    if (out0_required && outs[0] == nullptr) return RLCA_ERR_NULL_POINTER;
    const void *al[16];
    int na = 0;
    for (int i = 0; i < nreq; ++i) al[na++] = req_f32[i];
    al[na++] = truncated ? trunc_values : nullptr;
    al[na++] = bootstrap;
    for (int i = 0; i < nouts; ++i) al[na++] = outs[i];
    st = check_aligned4(al, na);
    if (st != RLCA_OK) return st;
    const size_t fb = (size_t)*elems * 4, ub = (size_t)*elems;
    Span ins[16];
    int ni = 0;
    for (int i = 0; i < nreq; ++i) ins[ni++] = {req_f32[i], fb};
    ins[ni++] = {terminated, ub};
    if (truncated) {
        ins[ni++] = {truncated, ub};
        ins[ni++] = {trunc_values, fb};
    }
    ins[ni++] = {bootstrap, (size_t)num_envs * 4};
    Span os[4];
    for (int i = 0; i < nouts; ++i) os[i] = {outs[i], fb};
    return check_aliasing(os, nouts, ins, ni);
}

static BackwardParams backward_params(int64_t num_envs) {
    BackwardParams p = {};
    p.geo.num_envs = num_envs;
    return p;
}

}  // namespace rlca

using namespace rlca;

extern "C" {

rlca_status rlca_gae(const float *rewards, const float *values, const uint8_t *terminated,
                     const uint8_t *truncated, const float *trunc_values,
                     const float *bootstrap, float gamma, float lambda, int64_t num_envs,
                     int64_t T, float *advantages, float *returns, hipStream_t stream) {
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLCA_ERR_INVALID_VALUE;
    const float *req[] = {rewards, values};
    float *outs[] = {advantages, returns};
    int64_t n;
    rlca_status st = check_backward(req, 2, terminated, truncated, trunc_values, bootstrap, outs,
                                    2, true, num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    BackwardParams p = backward_params(num_envs);
    p.rewards = rewards;
    p.values = values;
    p.terminated = terminated;
    p.truncated = truncated;
    p.trunc_values = truncated ? trunc_values : nullptr;
    p.bootstrap = bootstrap;
    p.out0 = advantages;
    p.out1 = returns;
    p.gamma = gamma;
    p.lambda = lambda;
    return run_backward(kGae, p, T, stream);
}

rlca_status rlca_td_lambda(const float *rewards, const float *values,
                           const uint8_t *terminated, const uint8_t *truncated,
                           const float *trunc_values, const float *bootstrap, float gamma,
                           float lambda, int64_t num_envs, int64_t T, float *returns,
                           hipStream_t stream) {
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLCA_ERR_INVALID_VALUE;
    const float *req[] = {rewards, values};
    float *outs[] = {returns};
    int64_t n;
    rlca_status st = check_backward(req, 2, terminated, truncated, trunc_values, bootstrap, outs,
                                    1, true, num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    BackwardParams p = backward_params(num_envs);
    p.rewards = rewards;
    p.values = values;
    p.terminated = terminated;
    p.truncated = truncated;
    p.trunc_values = truncated ? trunc_values : nullptr;
    p.bootstrap = bootstrap;
    p.out0 = returns;
    p.gamma = gamma;
    p.lambda = lambda;
    return run_backward(kTdLambda, p, T, stream);
}

rlca_status rlca_discounted_returns(const float *rewards, const uint8_t *terminated,
                                    const uint8_t *truncated, const float *trunc_values,
                                    const float *bootstrap, float gamma, int64_t num_envs,
                                    int64_t T, float *returns, hipStream_t stream) {
    if (!unit_interval(gamma)) return RLCA_ERR_INVALID_VALUE;
    const float *req[] = {rewards};
    float *outs[] = {returns};
    int64_t n;
    rlca_status st = check_backward(req, 1, terminated, truncated, trunc_values, bootstrap, outs,
                                    1, true, num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    BackwardParams p = backward_params(num_envs);
    p.rewards = rewards;
    p.terminated = terminated;
    p.truncated = truncated;
    p.trunc_values = truncated ? trunc_values : nullptr;
    p.bootstrap = bootstrap;
    p.out0 = returns;
    p.gamma = gamma;
    return run_backward(kDiscounted, p, T, stream);
}

rlca_status rlca_vtrace(const float *rewards, const float *values, const float *behaviour_logp,
                        const float *target_logp, const uint8_t *terminated,
                        const uint8_t *truncated, const float *trunc_values,
                        const float *bootstrap, float gamma, float lambda, float rho_bar,
                        float c_bar, int64_t num_envs, int64_t T, float *vs,
                        float *pg_advantages, hipStream_t stream) {
    if (!unit_interval(gamma) || !unit_interval(lambda) || !positive_finite(rho_bar) ||
        !positive_finite(c_bar))
        return RLCA_ERR_INVALID_VALUE;
    const float *req[] = {rewards, values, behaviour_logp, target_logp};
    float *outs[] = {vs, pg_advantages};
    int64_t n;
    rlca_status st = check_backward(req, 4, terminated, truncated, trunc_values, bootstrap, outs,
                                    2, true, num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    BackwardParams p = backward_params(num_envs);
    p.rewards = rewards;
    p.values = values;
    p.behaviour_logp = behaviour_logp;
    p.target_logp = target_logp;
    p.terminated = terminated;
    p.truncated = truncated;
    p.trunc_values = truncated ? trunc_values : nullptr;
    p.bootstrap = bootstrap;
    p.out0 = vs;
    p.out1 = pg_advantages;
    p.gamma = gamma;
    p.lambda = lambda;
    p.rho_bar = rho_bar;
    p.c_bar = c_bar;
    return run_backward(kVtrace, p, T, stream);
}

rlca_status rlca_retrace(const float *rewards, const float *q_values, const float *expected_q,
                         const float *behaviour_logp, const float *target_logp,
                         const uint8_t *terminated, const uint8_t *truncated,
                         const float *trunc_values, const float *bootstrap, float gamma,
                         float lambda, float c_bar, int64_t num_envs, int64_t T,
                         float *q_ret, hipStream_t stream) {
    if (!unit_interval(gamma) || !unit_interval(lambda) || !positive_finite(c_bar))
        return RLCA_ERR_INVALID_VALUE;
    const float *req[] = {rewards, q_values, expected_q, behaviour_logp, target_logp};
    float *outs[] = {q_ret};
    int64_t n;
    rlca_status st = check_backward(req, 5, terminated, truncated, trunc_values, bootstrap, outs,
                                    1, true, num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    BackwardParams p = backward_params(num_envs);
    p.rewards = rewards;
    p.values = q_values;
    p.expected_q = expected_q;
    p.behaviour_logp = behaviour_logp;
    p.target_logp = target_logp;
    p.terminated = terminated;
    p.truncated = truncated;
    p.trunc_values = truncated ? trunc_values : nullptr;
    p.bootstrap = bootstrap;
    p.out0 = q_ret;
    p.gamma = gamma;
    p.lambda = lambda;
    p.c_bar = c_bar;
    return run_backward(kRetrace, p, T, stream);
}

static rlca_status run_forward(const void *x, bool is_int, const uint8_t *flags,
                               rlca_reset_convention conv, float decay, int64_t num_envs,
                               int64_t T, void *out, hipStream_t stream) {
    if (conv != RLCA_RESET_ON_START && conv != RLCA_RESET_AFTER_DONE)
        return RLCA_ERR_INVALID_VALUE;
    int64_t n;
    rlca_status st = check_sizes(num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    if (x == nullptr || flags == nullptr || out == nullptr) return RLCA_ERR_NULL_POINTER;
    const void *al[] = {x, out};
    st = check_aligned4(al, 2);
    if (st != RLCA_OK) return st;
    const Span ins[] = {{x, (size_t)n * 4}, {flags, (size_t)n}};
    const Span os[] = {{out, (size_t)n * 4}};
    st = check_aliasing(os, 1, ins, 2);
    if (st != RLCA_OK) return st;
    const void *f32[] = {x, out};
    const void *u8[] = {flags};
    const LaunchShape s = choose_shape(num_envs, T, vec_ok(T, f32, 2, u8, 1));
    ForwardParams p = {};
    p.x = x;
    p.flags = flags;
    p.out = out;
    p.decay = is_int ? __builtin_bit_cast(float, 1u) : decay;
    p.geo.num_envs = num_envs;
    p.geo.T = (uint32_t)T;
    const bool after = conv == RLCA_RESET_AFTER_DONE;
    return is_int ? launch_forward_u32(p, after, s, stream)
                  : launch_forward_f32(p, after, s, stream);
}

rlca_status rlca_eligibility_traces(const float *increments, const uint8_t *flags,
                                    rlca_reset_convention convention, float gamma,
                                    float lambda, int64_t num_envs, int64_t T, float *traces,
                                    hipStream_t stream) {
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLCA_ERR_INVALID_VALUE;
    return run_forward(increments, false, flags, convention, gamma * lambda, num_envs, T,
                       traces, stream);
}

rlca_status rlca_episodic_prefix_sum(const void *x, rlca_dtype dtype, const uint8_t *flags,
                                     rlca_reset_convention convention, int64_t num_envs,
                                     int64_t T, void *out, hipStream_t stream) {
    if (dtype != RLCA_F32 && dtype != RLCA_I32) return RLCA_ERR_INVALID_VALUE;
    return run_forward(x, dtype == RLCA_I32, flags, convention, 1.0f, num_envs, T, out, stream);
}

rlca_status rlca_affine_scan(const float *alpha, const float *beta, const float *carry,
                             rlca_direction direction, int64_t num_envs, int64_t T, float *out,
                             hipStream_t stream) {
    if (direction != RLCA_BACKWARD && direction != RLCA_FORWARD) return RLCA_ERR_INVALID_VALUE;
    int64_t n;
    rlca_status st = check_sizes(num_envs, T, &n);
    if (st != RLCA_OK || n == 0) return st;
    if (alpha == nullptr || beta == nullptr || out == nullptr) return RLCA_ERR_NULL_POINTER;
    const void *al[] = {alpha, beta, carry, out};
    st = check_aligned4(al, 4);
    if (st != RLCA_OK) return st;
    const Span ins[] = {{alpha, (size_t)n * 4}, {beta, (size_t)n * 4}, {carry, (size_t)num_envs * 4}};
    const Span os[] = {{out, (size_t)n * 4}};
    st = check_aliasing(os, 1, ins, 3);
    if (st != RLCA_OK) return st;
    if (direction == RLCA_BACKWARD) {
        BackwardParams p = backward_params(num_envs);
        p.rewards = alpha;
        p.values = beta;
        p.bootstrap = carry;
        p.out0 = out;
        return run_backward(kAffineBackward, p, T, stream);
    }
    const void *f32[] = {alpha, beta, out};
    const LaunchShape s = choose_shape(num_envs, T, vec_ok(T, f32, 3, nullptr, 0));
    ForwardParams p = {};
    p.x = alpha;
    p.beta = beta;
    p.carry = carry;
    p.out = out;
    p.geo.num_envs = num_envs;
    p.geo.T = (uint32_t)T;
    return launch_affine_forward(p, s, stream);
}

const char *rlca_status_string(rlca_status status) {
    switch (status) {
        case RLCA_OK: return "ok";
        case RLCA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case RLCA_ERR_INVALID_SIZE: return "invalid size (negative, too large or overflowing)";
        case RLCA_ERR_INVALID_VALUE: return "invalid parameter value";
        case RLCA_ERR_ALIASING: return "an output overlaps an input or another output";
        case RLCA_ERR_MISALIGNED: return "a 32-bit array is not 4-byte aligned";
        case RLCA_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
