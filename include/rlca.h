/*
 * rlca.h -- C ABI of the MI355X (gfx950) credit-assignment scan library.
 *
 * Seven reinforcement-learning credit-assignment estimators computed as one
 * first-order affine recurrence over [num_envs, T] rollouts:
 *   backward  A_t = alpha_t + beta_t * A_{t+1}   (GAE, TD(lambda), discounted
 *             returns, V-Trace, Retrace(lambda))
 *   forward   A_t = alpha_t + beta_t * A_{t-1}   (eligibility traces, episodic
 *             prefix sums)
 * ("rl-triton: High-Performance Triton GPU Kernels for Reinforcement Learning
 * Credit Assignment", paperlayer.ai summary, §1 Introduction and §3.1 Shared
 * scan formulation).  Each estimator call is one kernel launch that reads
 * its inputs from HBM once and writes each output once -- except for few
 * long rows (fewer than 128 rows of 16384 steps or more; for the forward
 * scans fewer than 160 rows of 32768 steps or more and fewer than 208 from
 * 65536 steps on), where each row is split into chunks that run in
 * parallel: three launches, inputs read twice, and the first
 * output array holds the chunk hand-off values until the last launch
 * overwrites them.  The fused consumers of GAE at the end of this header
 * are one launch each too.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory:  every array argument is a DEVICE pointer (hipMalloc memory or a
 *          torch tensor's data_ptr()) owned by the caller.  The library
 *          allocates nothing, keeps no mutable global state and never
 *          synchronizes: work is enqueued on `stream` and buffers must stay
 *          alive until the stream has passed the call.  With no state
 *          between calls, any entry point may be called from several host
 *          threads at once, on one stream or on several; only calls whose
 *          outputs overlap each other or another call's inputs, with nothing
 *          ordering them, race.
 * Layout:  per-step arrays are dense row-major [num_envs, T]; element (n, t)
 *          is at n*T + t.  `bootstrap` is [num_envs].  Real-valued and int32
 *          data must be aligned to its element size.  Flags are one byte per
 *          step, any nonzero byte meaning "set" (torch.bool and uint8 both
 *          work).  Speed, not results, depends on where arrays start: call
 *          an array's phase its start address's element index mod 4 from a
 *          four-element boundary (16 bytes for fp32, 8 for bf16 / fp16, 4
 *          for flags).  Every per-step array at phase 0 with T % 4 == 0 is
 *          the fastest case; per-step inputs all at one phase take the
 *          vectorised path too (outputs at another phase are then written
 *          element by element); inputs at different phases are read element
 *          by element.  On the vectorised path, except in the fastest case,
 *          the library reads whole aligned four-element blocks: it may read
 *          (never write) up to three elements before the start or past the
 *          end of a per-step input, inside the aligned block that holds its
 *          first or last element.  Such reads cannot fault and their values
 *          are not used.
 * Episode boundaries (summary §3.2 Episode-boundary semantics):
 *          terminated[t]  the episode ends after step t in a terminal state:
 *                         successor value 0, no credit flows back past t.
 *          truncated[t]   the episode is cut after step t (time limit): the
 *                         successor value is trunc_values[t] (the value of the
 *                         state the episode was cut in), no credit flows back
 *                         past t.  Terminated wins when both are set.
 *                         truncated == NULL means no truncation and selects a
 *                         specialised fast path; trunc_values is then ignored.
 *          t = T-1        the rollout window ends: when the last step is not
 *                         done, its successor value is bootstrap[n]
 *                         (bootstrap == NULL means 0).  A done last step
 *                         ignores the bootstrap.
 * Errors:  the return value is the only error channel.  Arguments are checked
 *          before anything is enqueued and a failed call has no side effects.
 *            RLCA_ERR_NULL_POINTER   a required pointer is NULL
 *            RLCA_ERR_INVALID_SIZE   num_envs < 0, T < 0, T > RLCA_MAX_T,
 *                                    num_envs > RLCA_MAX_ENVS, the byte
 *                                    size of an array overflows, or the
 *                                    launch would need more than 2^31 - 1
 *                                    workgroups (only num_envs near
 *                                    RLCA_MAX_ENVS with rows longer than one
 *                                    tile: terabytes of input)
 *            RLCA_ERR_INVALID_VALUE  gamma or lambda outside [0, 1] or not
 *                                    finite, rho_bar <= 0 or not finite,
 *                                    c_bar outside (0, 1], an unknown enum
 *                                    value
 *            RLCA_ERR_ALIASING       an output overlaps an input or another
 *                                    output (in-place is not supported)
 *            RLCA_ERR_MISALIGNED     an array is not aligned to its element size
 *            RLCA_ERR_HIP            a kernel launch failed (its hipError_t)
 *          num_envs * T == 0 is a valid no-op.  Faults inside the kernel
 *          surface at the caller's next synchronisation, as usual in HIP.
 *          Non-finite inputs are not trapped; they propagate inside their
 *          episode segment only.  A chain cut (a terminated or truncated
 *          step, a row end, a forward reset, a coefficient of exactly 0,
 *          e.g. lambda = 0 or gamma = 0) stops them: a NaN or infinity in
 *          one row never reaches another row, and never crosses an episode
 *          boundary within its row.  Inside a segment they also stop where
 *          the product of the coefficients between two steps rounds to 0
 *          (after about 1,700 steps at gamma * lambda = 0.94 in fp32 scans,
 *          far later in fp64 ones).  A NaN log-probability gives a NaN
 *          importance weight (not a clamped one).
 * Numerics: fp32 arithmetic (the summary's §4 requires float32 scans),
 *          with the fp64 scans stated below where fp32 would miss the
 *          summary's tolerance; the scan reassociates the recurrence
 *          (associativity, summary §5), so results match a sequential fp64
 *          evaluation to rounding, not bit for bit.  The int32 prefix sum is exact
 *          (two's-complement wrap).  Arrays may instead be stored as bf16 or
 *          fp16 (rlca_dtype; the summary's §9 defers bfloat16 I/O): they are
 *          widened exactly to fp32 on load and every output is rounded once,
 *          to nearest even, on store.  Every estimator's coefficient is a
 *          contraction, 0 <= beta_t <= 1 (gamma, lambda in [0, 1] and trace
 *          clips c_bar <= 1).  Where a chain that barely decays (beta near 1)
 *          carries a value across the 256-step waves of the scan, fp32
 *          rounding of the beta products and of the carried sums would
 *          build up along the row; such calls (and every generic affine
 *          scan over rows longer than 256 steps) scan in fp64 and round
 *          each output once, so chains that never break (a prefix sum
 *          without resets, gamma = 1 returns) keep their accuracy over the
 *          row, 131072 steps and more.  Affine coefficients beyond +-1 let
 *          products of beta grow, and rounding errors grow with them in
 *          any evaluation order; 16-bit storage may then overflow.
 */
#ifndef RLCA_H
#define RLCA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLCA_MAX_T ((int64_t)1 << 30)
#define RLCA_MAX_ENVS ((int64_t)1 << 31)

/* Clamp applied to log(pi/mu) before exp() in V-Trace and Retrace. */
#define RLCA_LOG_RATIO_CLIP 5.0f

typedef enum {
    RLCA_OK = 0,
    RLCA_ERR_NULL_POINTER = 1,
    RLCA_ERR_INVALID_SIZE = 2,
    RLCA_ERR_INVALID_VALUE = 3,
    RLCA_ERR_ALIASING = 4,
    RLCA_ERR_MISALIGNED = 5,
    RLCA_ERR_HIP = 6
} rlca_status;

/* Forward-scan reset conventions.  The summary's §3.3 leaves the boundary
 * convention of the segmented forward scans configurable; its §5 cuts the
 * forward carry at the step after a done step. */
typedef enum {
    RLCA_RESET_ON_START = 0,  /* flags[t] != 0: step t starts a new episode      */
    RLCA_RESET_AFTER_DONE = 1 /* flags[t-1] != 0: step t-1 ended the episode      */
} rlca_reset_convention;

/* Element type of the data arrays.  RLCA_F32, RLCA_BF16 and RLCA_F16 are
 * storage types of the real-valued arrays (arithmetic is fp32 for all
 * three); RLCA_I32 is the exact integer prefix sum. */
typedef enum { RLCA_F32 = 0, RLCA_I32 = 1, RLCA_BF16 = 2, RLCA_F16 = 3 } rlca_dtype;

typedef enum { RLCA_BACKWARD = 0, RLCA_FORWARD = 1 } rlca_direction;

/* Generalized advantage estimation (Schulman et al. 2016; summary §2.1).
 *   delta_t = r_t + gamma * V(s_{t+1}) - V(s_t),   V(s_{t+1}) per the boundary rules
 *   adv_t   = delta_t + gamma * lambda * adv_{t+1}  (chain cut at done steps and t = T-1)
 *   ret_t   = adv_t + V(s_t)
 * rewards, values [N,T] f32; terminated [N,T] u8 (required); truncated [N,T] u8
 * (nullable); trunc_values [N,T] f32 (required iff truncated); bootstrap [N]
 * f32 (nullable).  Writes advantages [N,T] and, when non-NULL, returns [N,T]. */
rlca_status rlca_gae(const float *rewards, const float *values, const uint8_t *terminated,
                     const uint8_t *truncated, const float *trunc_values,
                     const float *bootstrap, float gamma, float lambda, int64_t num_envs,
                     int64_t T, float *advantages, float *returns, hipStream_t stream);

/* TD(lambda) returns (summary §1, §3.2):
 *   G_t = r_t + gamma * ((1 - lambda) * V(s_{t+1}) + lambda * G_{t+1}),
 *   and G_t = r_t + gamma * successor value at a done step or at t = T-1.
 * Arguments as rlca_gae; writes returns [N,T]. */
rlca_status rlca_td_lambda(const float *rewards, const float *values,
                           const uint8_t *terminated, const uint8_t *truncated,
                           const float *trunc_values, const float *bootstrap, float gamma,
                           float lambda, int64_t num_envs, int64_t T, float *returns,
                           hipStream_t stream);

/* Discounted returns (summary §1, §3.2): G_t = r_t + gamma * G_{t+1}, and
 * G_t = r_t + gamma * successor value at a done step or at t = T-1
 * (bootstrap == NULL gives Monte-Carlo returns).  Writes returns [N,T]. */
rlca_status rlca_discounted_returns(const float *rewards, const uint8_t *terminated,
                                    const uint8_t *truncated, const float *trunc_values,
                                    const float *bootstrap, float gamma, int64_t num_envs,
                                    int64_t T, float *returns, hipStream_t stream);

/* V-Trace (Espeholt et al. 2018; summary §8 Off-policy correction).
 *   ratio_t = exp(clamp(target_logp_t - behaviour_logp_t, -5, 5))
 *   rho_t = min(rho_bar, ratio_t),  c_t = lambda * min(c_bar, ratio_t)
 *   vs_t - V_t = rho_t (r_t + gamma V(s_{t+1}) - V_t) + gamma c_t (vs_{t+1} - V_{t+1})
 *   pg_t = rho_t (r_t + gamma vs_{t+1} - V_t)
 * where at a done step or t = T-1 the successor value replaces V(s_{t+1}) and
 * vs_{t+1}.  lambda = 1 is the IMPALA form.  rho_bar > 0; 0 < c_bar <= 1 (a
 * trace clip above 1 would make the recurrence expansive). 
 * Writes vs [N,T] and, when non-NULL, pg_advantages [N,T]. */
rlca_status rlca_vtrace(const float *rewards, const float *values, const float *behaviour_logp,
                        const float *target_logp, const uint8_t *terminated,
                        const uint8_t *truncated, const float *trunc_values,
                        const float *bootstrap, float gamma, float lambda, float rho_bar,
                        float c_bar, int64_t num_envs, int64_t T, float *vs,
                        float *pg_advantages, hipStream_t stream);

/* Retrace(lambda) (Munos et al. 2016; summary §3.3: the decay uses the
 * next step's importance weight).
 *   c_t = lambda * min(c_bar, exp(clamp(target_logp_t - behaviour_logp_t, -5, 5)))
 *   Qret_t = r_t + gamma E_pi Q(s_{t+1}, .) + gamma c_{t+1} (Qret_{t+1} - Q_{t+1})
 * q_values[t] = Q(s_t, a_t); expected_q[t] = E_pi Q(s_t, .).  At a done step
 * or t = T-1 the successor value (0 / trunc_values[t] = E_pi Q of the cut
 * state / bootstrap[n] = E_pi Q(s_T, .)) replaces E_pi Q(s_{t+1}, .) and the
 * correction term is dropped.  0 < c_bar <= 1 (Munos et al. truncate the
 * trace at 1).  Writes q_ret [N,T]. */
rlca_status rlca_retrace(const float *rewards, const float *q_values, const float *expected_q,
                         const float *behaviour_logp, const float *target_logp,
                         const uint8_t *terminated, const uint8_t *truncated,
                         const float *trunc_values, const float *bootstrap, float gamma,
                         float lambda, float c_bar, int64_t num_envs, int64_t T,
                         float *q_ret, hipStream_t stream);

/* Accumulating eligibility traces, forward in time (summary §1, §3.2):
 *   e_t = x_t + gamma * lambda * e_{t-1},  e_{-1} = 0, and e_{t-1} := 0 where
 *   a new episode starts under `convention`.
 * increments [N,T] f32, flags [N,T] u8 (required).  Writes traces [N,T]. */
rlca_status rlca_eligibility_traces(const float *increments, const uint8_t *flags,
                                    rlca_reset_convention convention, float gamma,
                                    float lambda, int64_t num_envs, int64_t T, float *traces,
                                    hipStream_t stream);

/* Inclusive episodic (segmented) prefix sum, forward in time (summary §3.3):
 *   S_t = x_t + S_{t-1},  S_{-1} = 0, restarted where a new episode starts.
 * x and out are [N,T] of `dtype` (f32, bf16 or f16; or i32 with
 * two's-complement wrap-around, exact); flags [N,T] u8 (required). */
rlca_status rlca_episodic_prefix_sum(const void *x, rlca_dtype dtype, const uint8_t *flags,
                                     rlca_reset_convention convention, int64_t num_envs,
                                     int64_t T, void *out, hipStream_t stream);

/* Generic first-order affine scan over caller-built coefficients (the
 * summary's §4 Scan procedure: the generic kernel that takes precomputed
 * alpha and beta instead of building them from a rollout).
 *   RLCA_BACKWARD: A_t = alpha_t + beta_t * A_{t+1},  A_T = carry[n]
 *   RLCA_FORWARD:  A_t = alpha_t + beta_t * A_{t-1},  A_{-1} = carry[n]
 * alpha, beta, out [N,T] f32; carry [N] f32, nullable (=> 0).  Episode
 * boundaries are the caller's business (beta_t = 0 cuts the chain).  Writes
 * out [N,T]. */
rlca_status rlca_affine_scan(const float *alpha, const float *beta, const float *carry,
                             rlca_direction direction, int64_t num_envs, int64_t T, float *out,
                             hipStream_t stream);

/* ---------------------------------------------------------------- batches
 * Several of the calls above enqueued together.  Each element is validated
 * exactly as its own entry point would validate it (the same status codes,
 * nothing enqueued on any failure), plus: no call may write memory that
 * another call of the batch reads or writes (RLCA_ERR_ALIASING), because the
 * calls run concurrently.  Calls on the vectorised path that need a single
 * launch share grouped launches (one launch for up to 14 calls of one shape
 * class and storage type), which removes the per-launch overhead that
 * dominates small rollouts; the others are enqueued one by one.  Results
 * are bit for bit those of the separate calls (a grouped launch keeps each
 * call's tile geometry).
 * (Launch-overhead reduction for small shapes: the summary's §9
 * Limitations, where launch and wrapper overhead dominate at 16 steps.) */
#define RLCA_MAX_BATCH 64

typedef enum {
    RLCA_OP_GAE = 0,
    RLCA_OP_TD_LAMBDA = 1,
    RLCA_OP_DISCOUNTED_RETURNS = 2,
    RLCA_OP_VTRACE = 3,
    RLCA_OP_RETRACE = 4,
    RLCA_OP_ELIGIBILITY_TRACES = 5,
    RLCA_OP_EPISODIC_PREFIX_SUM = 6,
    RLCA_OP_AFFINE_SCAN = 7
} rlca_op;

/* One call of a batch.  Fields carry the arguments of the op's entry point;
 * fields an op does not take are ignored.
 *   rewards     rewards (GAE, TD, discounted, V-Trace, Retrace); increments
 *               (eligibility traces); x (prefix sum); alpha (affine scan)
 *   values      values (GAE, TD, V-Trace); q_values (Retrace); beta (affine)
 *   terminated  terminated (backward estimators); flags (forward scans)
 *   bootstrap   bootstrap (backward estimators); carry (affine scan)
 *   out0        advantages / returns / vs / q_ret / traces / out
 *   out1        GAE returns or V-Trace pg_advantages; nullable
 *   dtype       element type of every real-valued array of the call, inputs
 *               and outputs alike: RLCA_F32 (0), RLCA_BF16 or RLCA_F16; the
 *               prefix sum also takes RLCA_I32.  This is how the bf16 / fp16
 *               forms of every op are reached (the single-call entry points
 *               above are fp32, except the prefix sum, which takes dtype).
 *   convention, direction: as the forward scans / affine scan take them */
typedef struct {
    rlca_op op;
    int64_t num_envs;
    int64_t T;
    const void *rewards;
    const void *values;
    const void *expected_q;
    const void *behaviour_logp;
    const void *target_logp;
    const uint8_t *terminated;
    const uint8_t *truncated;
    const void *trunc_values;
    const void *bootstrap;
    float gamma;
    float lambda;
    float rho_bar;
    float c_bar;
    int convention;
    int dtype;
    int direction;
    void *out0;
    void *out1;
} rlca_call;

/* Enqueue `count` (0..RLCA_MAX_BATCH) calls on `stream`; `calls` is host
 * memory, read before the function returns. */
rlca_status rlca_run_batch(const rlca_call *calls, int count, hipStream_t stream);

/* ------------------------------------------------- fused consumers of GAE
 * The summary's §9 (Discussion and Future Work) names fused loss operations
 * as the next step for the library; these two calls fuse the usual PPO
 * consumers of the advantages into the scan's epilogue and into one
 * streaming pass.  Each is one launch: every workgroup leaves one partial
 * sum in a caller-owned device workspace and takes a ticket from counters
 * at the workspace's start; the workgroup that takes the last ticket adds
 * the partials in a fixed order (reproducible bit for bit, whichever
 * workgroup is last), writes the result and sets the counters back to
 * zero.  The *_workspace_size call returns the workspace's size (0 for
 * an empty rollout or invalid sizes).  The workspace must be zero-filled
 * before its first use (one hipMemset, or a zero-filled allocation); every
 * call leaves it so, so it can be reused by later calls of either consumer
 * and any size up to its own.  A launch that did not run to completion
 * (a fault) may leave the counter set: zero the workspace again.  The
 * workspace is written like an output: calls that may run at the same time
 * need workspaces of their own.  workspace, stats and loss must be 8-byte
 * aligned; RLCA_ERR_INVALID_SIZE if workspace_bytes is too small;
 * RLCA_ERR_ALIASING if the workspace, stats or loss overlap any other array
 * of the call.  An empty rollout (num_envs * T == 0) writes nothing. */
size_t rlca_gae_stats_workspace_size(int64_t num_envs, int64_t T);

/* rlca_gae (fp32) that also reduces the advantages it computes: stats is
 * double[2] in device memory, {mean, sample standard deviation (divisor
 * N*T - 1; 0 when N*T == 1)} over all N*T steps, accumulated in fp64.  The
 * usual advantage normalization (A - mean) / (std + eps) needs exactly
 * these, without a second pass over the advantages.  advantages and returns
 * are bit for bit those of rlca_gae. */
rlca_status rlca_gae_stats(const float *rewards, const float *values, const uint8_t *terminated,
                           const uint8_t *truncated, const float *trunc_values,
                           const float *bootstrap, float gamma, float lambda, int64_t num_envs,
                           int64_t T, float *advantages, float *returns, double *stats,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* rlca_gae_stats for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same kernels and the same results
 * bit for bit.  The ticket counter and partial sums live instead in a
 * buffer the library owns, RLCA_GAE_STATS_SCRATCH_BYTES of static device
 * memory that each GPU the library runs on holds until the process ends;
 * every size fits in it (the statistics launch never has more workgroups
 * than it has pairs), and a call that would need more returns
 * RLCA_ERR_INVALID_SIZE.  The call allocates nothing: the first call on
 * each device looks up the buffer's address there (hipGetSymbolAddress, no
 * allocation) and enqueues the zeroing of its counters on `stream`, one
 * small kernel (a caller that captures graphs should make that first call
 * before capturing); RLCA_ERR_HIP reports a failed lookup.  Every call on
 * one GPU shares its buffer and leaves its counters at zero: calls on one
 * stream are ordered and safe, but calls that may overlap on one GPU (on
 * different streams, or from threads that do not order them) race and
 * must use rlca_gae_stats with workspaces of their own. */
#define RLCA_GAE_STATS_SCRATCH_BYTES 69760
rlca_status rlca_gae_stats_noalloc(const float *rewards, const float *values,
                                   const uint8_t *terminated, const uint8_t *truncated,
                                   const float *trunc_values, const float *bootstrap, float gamma,
                                   float lambda, int64_t num_envs, int64_t T, float *advantages,
                                   float *returns, double *stats, hipStream_t stream);

size_t rlca_ppo_clip_loss_workspace_size(int64_t num_envs, int64_t T);

/* PPO clipped surrogate (Schulman et al. 2017, L^CLIP) as a loss, over the
 * M = num_envs * T steps of the [num_envs, T] arrays:
 *   A_hat_t = stats ? (A_t - stats[0]) / (stats[1] + norm_eps) : A_t
 *   rho_t   = exp(logp_new_t - logp_old_t)
 *   loss[0] = -(1/M) sum_t min(rho_t A_hat_t, clip(rho_t, 1-clip_eps, 1+clip_eps) A_hat_t)
 *   grad_logp_new[t] = d loss / d logp_new_t: -(1/M) rho_t A_hat_t where the
 *                      unclipped term is the smaller (ties included), else 0.
 * advantages, logp_new, logp_old [N,T] f32; stats double[2] as written by
 * rlca_gae_stats, nullable (no normalization); grad_logp_new [N,T] f32,
 * nullable; loss double[1] (device).  0 <= clip_eps < 1 and norm_eps >= 0,
 * finite, else RLCA_ERR_INVALID_VALUE.  Arithmetic per step is fp32, the
 * sums fp64. */
rlca_status rlca_ppo_clip_loss(const float *advantages, const double *stats,
                               const float *logp_new, const float *logp_old, float clip_eps,
                               float norm_eps, int64_t num_envs, int64_t T, float *grad_logp_new,
                               double *loss, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *rlca_status_string(rlca_status status);

#ifdef __cplusplus
}
#endif

#endif /* RLCA_H */
