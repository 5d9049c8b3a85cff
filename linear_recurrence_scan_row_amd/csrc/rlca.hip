// rlca.hip -- the C ABI of rlca.h: argument checks, launch-shape choice, batching.
//
// The kernels live in kernels.hpp and are instantiated one estimator per
// translation unit (est_*.hip).  Every entry point first turns its arguments
// into a validated Call (nothing is enqueued when a check fails), then
// enqueues it on the caller's stream: one launch, or three for a few long
// rows (the chunk modes).  rlca_run_batch validates a list of calls the same
// way and runs the eligible ones together in grouped launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"
#include "rlca.h"

namespace rlca {

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Enum arguments come from C, where an enum parameter may hold any int; in
// C++ a load of a value outside the enumerators' range is undefined, so the
// entry points read enum arguments by their int representation and check
// them as ints.
template <typename E>
static int enum_code(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized on this ABI");
    int code;
    memcpy(&code, &e, sizeof code);
    return code;
}

static bool unit_interval(float x) { return x >= 0.f && x <= 1.f; }  // false for NaN
static bool positive_finite(float x) { return x > 0.f && isfinite(x); }
// Trace clips: 0 < c_bar <= 1, so every importance-weighted coefficient
// beta_t = gamma * lambda * min(c_bar, ratio_t) stays in [0, 1] (Munos et
// al. truncate the trace at 1; IMPALA's c_bar <= rho_bar, 1 in its runs).
static bool trace_clip(float x) { return x > 0.f && x <= 1.f; }  // false for NaN

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

// Every real-valued or int32 array must be aligned to its element size.
static rlca_status check_aligned(const void *const *ptrs, int n, size_t elem) {
    for (int i = 0; i < n; ++i)
        if (ptrs[i] != nullptr && ((uintptr_t)ptrs[i] % elem) != 0) return RLCA_ERR_MISALIGNED;
    return RLCA_OK;
}

// Storage of real-valued arrays for an rlca_dtype (RLCA_I32 is handled by the
// prefix sum itself); -1 for a dtype that is not a real storage type.
static int storage_of(int dtype) {
    switch (dtype) {
        case RLCA_F32: return kStoreF32;
        case RLCA_BF16: return kStoreBF16;
        case RLCA_F16: return kStoreF16;
    }
    return -1;
}

static size_t storage_bytes(int storage) { return storage == kStoreF32 ? 4 : 2; }

// No output may overlap an input or another output.
static rlca_status check_aliasing(const Span *outs, int nout, const Span *ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes))
                return RLCA_ERR_ALIASING;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return RLCA_ERR_ALIASING;
    }
    return RLCA_OK;
}

// Memory path of a call.  The vector paths read a lane's K steps of each
// per-step input as one aligned block, so every per-step input must sit at
// the same phase: the element index, mod K, at which its K-aligned blocks
// start.  Whole-row lane chunks (kVecRows) further need T % K == 0 and every
// per-step array, outputs included, at phase 0; otherwise windows are
// widened to the inputs' block boundaries (kVecSkew), and outputs at another
// phase are written element by element.  Inputs at different phases take
// the scalar path.  (The [num_envs] arrays are read element by element.)
struct IoChoice {
    int io;
    uint32_t phase, out0_phase;
    bool scatter;
};

static uint32_t phase_of(const void *p, size_t elem) {
    return (uint32_t)(((uintptr_t)p / elem) % kK);
}

static IoChoice io_of(int64_t T, const void *const *ins, int nin, size_t elem,
                      const void *const *u8, int nu, const void *const *outs, int nout) {
    IoChoice c{kScalarIO, 0, 0, false};
    int phase = -1;
    for (int i = 0; i < nin + nu; ++i) {
        const void *p = i < nin ? ins[i] : u8[i - nin];
        if (p == nullptr) continue;
        const int m = (int)phase_of(p, i < nin ? elem : 1);
        if (phase >= 0 && m != phase) return c;
        phase = m;
    }
    c.phase = phase < 0 ? 0u : (uint32_t)phase;
    c.out0_phase = phase_of(outs[0], elem);
    for (int i = 0; i < nout; ++i)
        if (outs[i] != nullptr && phase_of(outs[i], elem) != c.phase) c.scatter = true;
    c.io = T % kK == 0 && c.phase == 0 && !c.scatter ? kVecRows : kVecSkew;
    return c;
}

// Launch shape.  Rows that end at wave boundaries (T divides the 256-step
// wave span) need no cross-wave exchange.  The wave count per workgroup was
// chosen by measurement on MI355X with cold HBM-resident operands: such short
// rows run fastest in 8-wave workgroups; rows of 257..1023 steps with one
// wave walking the row tile by tile when there are at least 4096 rows (with
// fewer, one wave per row leaves most wave slots empty, and 8-wave
// workgroups packing several rows per tile win by 8-19%); longer rows with 8
// waves sharing each tile through LDS.  Few long rows cannot fill the chip one
// workgroup per row (each walks its tiles one after another), so they are
// split into 2048-step chunks that run in parallel: three dependent launches,
// inputs read twice.  Measured on MI355X (GAE with truncation and eligibility
// traces, both paths at every shape, fp32 chunk scans, 16-wave row walks where
// those apply): the three launches cost more than they save below 16384 steps
// (1.2-2.1x slower at 8192, even at 12288); from 16384 steps on, a backward
// scan's chunks win below about 128 rows (1.05x slower at 128, 2-30x faster
// for one row of 2^15..2^19).  A forward scan's row walk moves fewer bytes
// per tile, so its chunks only win from 32768 steps on: below about 160 rows
// there, and below about 208 rows from 65536 steps on.
static constexpr int64_t kChunkedMinSteps = 8 * (int64_t)kChunkSteps;
static constexpr int64_t kChunkedMaxRows = 128;                  // backward, 16384+ steps
static constexpr int64_t kChunkedForwardMinSteps = 2 * kChunkedMinSteps;
static constexpr int64_t kChunkedMaxRowsForward = 160;           // forward, 32768+ steps
static constexpr int64_t kChunkedMaxRowsForwardLong = 208;       // forward, 65536+ steps

static bool take_chunked(int64_t num_envs, int64_t T, bool backward) {
    if (backward) return T >= kChunkedMinSteps && num_envs < kChunkedMaxRows;
    if (T < kChunkedForwardMinSteps) return false;
    return num_envs < (T >= 2 * kChunkedForwardMinSteps ? kChunkedMaxRowsForwardLong
                                                        : kChunkedMaxRowsForward);
}
static constexpr int64_t kOneWaveMinRows = 4096;
// Rows longer than one 2048-step tile walk their tiles one after another, one
// memory round trip per tile.  With at most 512 of them, 16-wave workgroups
// (4096-step tiles, on both vector paths) put twice the bytes in flight per
// row and fill the chip's wave slots: measured on MI355X (GAE with
// truncation, eligibility traces), 10-21% faster than 8-wave ones at 64..512
// rows of 2049..4095 steps and 10-25% at 160..512 rows of 4096..131072, and
// mixed to slower from 1024 rows on, where 8-wave workgroups already fill the
// chip.  Skewed windows (T % 4 != 0) gain 6-28% up to 256 rows and are mixed
// at 512 (GAE 8% slower at 4101..8195 steps).  Results are bit for bit those
// of 8-wave tiles: the carry passes through the same wave totals in the same
// order.  fp64 scans keep 8 waves.
static constexpr int64_t kWideMinSteps = 2 * kChunkSteps + 1;  // longer than one 8-wave tile
static constexpr int64_t kWideMaxRows = 512;
static constexpr int64_t kWideMaxRowsSkewed = 256;
// Rows of T % K != 0 steps (and inputs or outputs off phase 0) are read
// K-wide from windows widened to block boundaries, in 8-wave workgroups for
// every T (one-wave
// workgroups walking rows of 257..1023 steps measured 10-50% slower here:
// a row plus its skew often needs one more 256-step tile).  A row that fits
// one tile but not together with the largest skew its window can have
// (T = 2047) would leave most of a second tile idle: with enough rows,
// windows of K / gcd(T, K) rows, whose starts are all K-aligned, walk their
// tiles instead (25% faster for eligibility traces over 8192 x 2047, 4%
// slower for GAE).  Longer rows keep one row per window (aligned windows of
// 4 rows measured 5-13% slower over 4096 x 4097).
static constexpr int64_t kSkewAlignedMinWindows = 1024;

// Scan precision of a call whose coefficients satisfy |beta_t| <= beta.max.
// Wherever a value crosses the scan's waves (rows longer than one wave),
// two fp32 effects grow along a chain that barely decays: the rounding of
// beta products and carried sums (emulating the fp32 evaluation order: 2e-4
// at beta = 0.999 over 2048 steps, 1.7e-4 at beta = 1 over 131072), and the
// chain's sensitivity to beta itself, which turns the fp32 rounding of a
// product of parameters (gamma * lambda) into an output error of order
// 2^-24 * sqrt(2 / (1 - beta^2)^3).  fp32 keeps the parity bar for beta.max
// <= 0.95; for beta.max <= 0.99 when the fp32 coefficient is the exact
// product of the parameters (beta.exact); and at beta.max = 1 (exact
// products) up to one 2048-step tile.  Other calls scan in fp64 (ScanOf in
// scan_core.hpp), with beta formed in fp64.  Rows that end at wave
// boundaries carry nothing between waves and stay fp32; integer sums are
// exact.
struct BetaBound {
    float max;   // largest beta_t, as the fp32 kernels form it
    bool exact;  // that fp32 value is the exact product of the parameters
};

static BetaBound product_bound(float a, float b) {
    const float p = a * b;
    return {p, (double)p == (double)a * (double)b};
}

// The importance-weighted estimators: beta_t = gamma * (lambda * min(c_bar,
// ratio_t)), largest where the ratio is clipped at c_bar.
static BetaBound weighted_bound(float gamma, float lambda, float c_bar) {
    const BetaBound c = product_bound(lambda, c_bar);
    const BetaBound b = product_bound(gamma, c.max);
    return {b.max, c.exact && b.exact};
}

static void set_precision(LaunchShape &s, int64_t T, BetaBound beta, bool is_int) {
    const bool fp32_ok = beta.max <= 0.95f || (beta.exact && beta.max <= 0.99f) ||
                         (beta.exact && beta.max == 1.f && T <= (int64_t)kChunkSteps);
    s.f64 = !is_int && !s.wave_local && T > kWave * kK && !fp32_ok;
    // the fp64 scans' registers allow one 16-wave workgroup per CU only
    if (s.f64 && s.waves == 16) s.waves = 8;
}

static LaunchShape choose_shape(int64_t num_envs, int64_t T, const IoChoice &io,
                                bool backward) {
    LaunchShape s;
    s.vec = io.io != kScalarIO;
    s.skew = io.io == kVecSkew;
    s.phase = s.skew ? io.phase : 0u;
    s.out0_phase = s.skew ? io.out0_phase : 0u;
    s.scatter = s.skew && io.scatter;
    s.wave_local = io.io == kVecRows && T <= kWave * kK && (kWave * kK) % T == 0;
    s.waves = (T <= kWave * kK || T >= 1024 || num_envs < kOneWaveMinRows) ? 8 : 1;
    if (s.vec && T >= kWideMinSteps &&
        num_envs <= (s.skew ? kWideMaxRowsSkewed : kWideMaxRows))
        s.waves = 16;
    s.chunked = s.vec && take_chunked(num_envs, T, backward);
    s.f64 = false;  // set_precision
    s.quantum = 1;
    if (s.skew) {
        if (s.waves != 16) s.waves = 8;
        const int64_t tile = (int64_t)s.waves * kWave * kK;
        const int64_t q = aligned_rows((uint32_t)T);
        if (!s.chunked && T <= tile && T + max_skew((uint32_t)T, s.phase) > tile &&
            num_envs / q >= kSkewAlignedMinWindows)
            s.quantum = (uint32_t)q;
    }
    return s;
}

// ------------------------------------------------------------ validated calls

// A call whose arguments passed every check, ready to enqueue alone or in a
// batch.  `ins` / `outs` keep the byte ranges for cross-call aliasing checks.
struct Call {
    bool empty;  // num_envs * T == 0: nothing to enqueue
    bool backward;
    int est;          // backward estimator
    int forward;      // forward kind
    bool is_int;      // forward int32 prefix sum
    bool after_done;  // forward reset convention
    int storage;      // Storage of the real-valued arrays (kStoreF32 for int32 sums)
    LaunchShape shape;
    BackwardParams bp;
    ForwardParams fp;
    Span ins[12];
    int nin;
    Span outs[2];
    int nout;
};

// Checks shared by the backward estimators; fills the call's parameter
// block, byte ranges and launch shape.  Arrays an estimator does not use are
// passed as NULL and neither required nor read.  Real-valued arrays are
// stored as `storage`.
static rlca_status prepare_backward(int est, int storage, const void *rewards,
                                    const void *values, const void *expected_q,
                                    const void *behaviour_logp, const void *target_logp,
                                    const uint8_t *terminated, const uint8_t *truncated,
                                    const void *trunc_values, const void *bootstrap, void *out0,
                                    void *out1, int64_t num_envs, int64_t T, Call *c) {
    *c = Call{};
    if (storage < 0) return RLCA_ERR_INVALID_VALUE;
    const size_t es = storage_bytes(storage);
    int64_t n;
    rlca_status st = check_sizes(num_envs, T, &n);
    if (st != RLCA_OK) return st;
    c->empty = n == 0;
    if (c->empty) return RLCA_OK;
    const bool needs_values = est != kDiscounted;
    const bool needs_logp = est == kVtrace || est == kRetrace;
    const bool needs_flags = est != kAffineBackward;
    if (rewards == nullptr || out0 == nullptr) return RLCA_ERR_NULL_POINTER;
    if (needs_values && values == nullptr) return RLCA_ERR_NULL_POINTER;
    if (est == kRetrace && expected_q == nullptr) return RLCA_ERR_NULL_POINTER;
    if (needs_logp && (behaviour_logp == nullptr || target_logp == nullptr))
        return RLCA_ERR_NULL_POINTER;
    if (needs_flags && terminated == nullptr) return RLCA_ERR_NULL_POINTER;
    if (truncated != nullptr && trunc_values == nullptr) return RLCA_ERR_NULL_POINTER;
    if (!needs_flags) terminated = truncated = nullptr;
    if (truncated == nullptr) trunc_values = nullptr;
    if (!needs_values) values = nullptr;
    if (est != kRetrace) expected_q = nullptr;
    if (!needs_logp) behaviour_logp = target_logp = nullptr;
    const void *real[] = {rewards,      values,    expected_q, behaviour_logp, target_logp,
                          trunc_values, bootstrap, out0,       out1};
    st = check_aligned(real, 9, es);
    if (st != RLCA_OK) return st;
    const size_t fb = (size_t)n * es, ub = (size_t)n;
    const void *f32_steps[] = {rewards, values, expected_q, behaviour_logp, target_logp,
                               trunc_values};
    for (const void *p : f32_steps)
        if (p != nullptr) c->ins[c->nin++] = {p, fb};
    if (terminated != nullptr) c->ins[c->nin++] = {terminated, ub};
    if (truncated != nullptr) c->ins[c->nin++] = {truncated, ub};
    c->ins[c->nin++] = {bootstrap, (size_t)num_envs * es};
    c->outs[c->nout++] = {out0, fb};
    if (out1 != nullptr) c->outs[c->nout++] = {out1, fb};
    st = check_aliasing(c->outs, c->nout, c->ins, c->nin);
    if (st != RLCA_OK) return st;

    c->backward = true;
    c->est = est;
    c->storage = storage;
    BackwardParams &p = c->bp;
    p.rewards = rewards;
    p.values = values;
    p.expected_q = expected_q;
    p.behaviour_logp = behaviour_logp;
    p.target_logp = target_logp;
    p.terminated = terminated;
    p.truncated = truncated;
    p.trunc_values = trunc_values;
    p.bootstrap = bootstrap;
    p.out0 = out0;
    p.out1 = out1;
    p.geo.num_envs = num_envs;
    p.geo.T = (uint32_t)T;
    const void *u8[] = {terminated, truncated};
    const void *outs[] = {out0, out1};
    c->shape = choose_shape(num_envs, T, io_of(T, f32_steps, 6, es, u8, 2, outs, 2), true);
    if (launch_groups(num_envs, T, c->shape) > (int64_t)kOneShotMaxGrid)
        return RLCA_ERR_INVALID_SIZE;  // terabytes of input: no launch grid that large
    return RLCA_OK;
}

// Forward scans: x, beta, carry and out are stored as `storage`, or are
// int32 with `is_int` (then storage is kStoreF32, the 4-byte class).
static rlca_status prepare_forward(int kind, int storage, const void *x, bool is_int,
                                   const uint8_t *flags, int convention, float decay,
                                   double decay64,
                                   const void *beta, const void *carry, int64_t num_envs,
                                   int64_t T, void *out, Call *c) {
    *c = Call{};
    if (storage < 0) return RLCA_ERR_INVALID_VALUE;
    const size_t es = storage_bytes(storage);
    if (kind == kForwardFlags && convention != RLCA_RESET_ON_START &&
        convention != RLCA_RESET_AFTER_DONE)
        return RLCA_ERR_INVALID_VALUE;
    int64_t n;
    rlca_status st = check_sizes(num_envs, T, &n);
    if (st != RLCA_OK) return st;
    c->empty = n == 0;
    if (c->empty) return RLCA_OK;
    if (x == nullptr || out == nullptr) return RLCA_ERR_NULL_POINTER;
    if (kind == kForwardFlags && flags == nullptr) return RLCA_ERR_NULL_POINTER;
    if (kind == kForwardAffine && beta == nullptr) return RLCA_ERR_NULL_POINTER;
    if (kind == kForwardFlags) beta = carry = nullptr;
    if (kind == kForwardAffine) flags = nullptr;
    const void *al[] = {x, beta, carry, out};
    st = check_aligned(al, 4, es);
    if (st != RLCA_OK) return st;
    c->ins[c->nin++] = {x, (size_t)n * es};
    if (flags != nullptr) c->ins[c->nin++] = {flags, (size_t)n};
    if (beta != nullptr) c->ins[c->nin++] = {beta, (size_t)n * es};
    c->ins[c->nin++] = {carry, (size_t)num_envs * es};
    c->outs[c->nout++] = {out, (size_t)n * es};
    st = check_aliasing(c->outs, c->nout, c->ins, c->nin);
    if (st != RLCA_OK) return st;

    c->backward = false;
    c->forward = kind;
    c->is_int = is_int;
    c->storage = storage;
    c->after_done = kind == kForwardFlags && convention == RLCA_RESET_AFTER_DONE;
    ForwardParams &p = c->fp;
    p.x = x;
    p.flags = flags;
    p.beta = beta;
    p.carry = carry;
    p.out = out;
    p.decay = is_int ? __builtin_bit_cast(float, 1u) : decay;
    p.decay64 = decay64;
    p.geo.num_envs = num_envs;
    p.geo.T = (uint32_t)T;
    const void *wide[] = {x, beta};
    const void *u8[] = {flags};
    const void *outs[] = {out};
    c->shape = choose_shape(num_envs, T, io_of(T, wide, 2, es, u8, 1, outs, 1), false);
    if (launch_groups(num_envs, T, c->shape) > (int64_t)kOneShotMaxGrid)
        return RLCA_ERR_INVALID_SIZE;  // terabytes of input: no launch grid that large
    return RLCA_OK;
}

// Enqueue one call on its own.
static rlca_status launch_call(Call &c, hipStream_t stream) {
    if (c.empty) return RLCA_OK;
    if (c.backward) {
        switch (c.est) {
            case kGae: return launch_gae(c.bp, c.shape, c.storage, stream);
            case kTdLambda: return launch_td_lambda(c.bp, c.shape, c.storage, stream);
            case kDiscounted: return launch_discounted(c.bp, c.shape, c.storage, stream);
            case kVtrace: return launch_vtrace(c.bp, c.shape, c.storage, stream);
            case kRetrace: return launch_retrace(c.bp, c.shape, c.storage, stream);
            default: return launch_affine_backward(c.bp, c.shape, c.storage, stream);
        }
    }
    if (c.forward == kForwardAffine)
        return launch_affine_forward(c.fp, c.shape, c.storage, stream);
    return c.is_int ? launch_forward_u32(c.fp, c.after_done, c.shape, stream)
                    : launch_forward_float(c.fp, c.after_done, c.shape, c.storage, stream);
}

// The call as one member of a grouped launch, or false where it cannot be one.
static bool grouped_member(const Call &c, GroupedCall *g, int *variant, uint32_t *workgroups) {
    // Grouped launches run 8-wave workgroups: calls shaped for 8 waves take
    // one workgroup per group, one-wave calls one wave per group.  Both keep
    // the geometry of their own launch, so results match it bit for bit.
    // Calls that scan in fp64 run their own launch (their kernels are not
    // part of the grouped classes).
    if (!c.shape.vec || c.shape.chunked || c.shape.f64 ||
        (c.shape.waves != 1 && c.shape.waves != kGroupWaves))
        return false;
    const bool wl = c.shape.wave_local, one = c.shape.waves == 1, skew = c.shape.skew;
    uint32_t grid, groups;
    if (c.backward) {
        g->b = c.bp;
        g->b.geo = make_geometry(c.bp.geo.num_envs, c.bp.geo.T, c.shape, &grid);
        const bool trunc = c.bp.truncated != nullptr;
        *variant = skew ? grouped_skew_backward_variant(c.est, trunc)
                        : grouped_backward_variant(c.est, trunc, wl, one);
        groups = g->b.geo.num_groups;
    } else {
        g->f = c.fp;
        g->f.geo = make_geometry(c.fp.geo.num_envs, c.fp.geo.T, c.shape, &grid);
        if (skew)
            *variant = c.forward == kForwardAffine
                           ? kGroupedSkewAffineForward
                           : grouped_skew_forward_variant(c.is_int, c.after_done);
        else
            *variant = c.forward == kForwardAffine
                           ? grouped_affine_forward_variant(wl, one)
                           : grouped_forward_variant(c.is_int, c.after_done, wl, one);
        groups = g->f.geo.num_groups;
    }
    *workgroups = one ? (groups + kGroupWaves - 1) / kGroupWaves : groups;
    return *workgroups <= kMaxGrid;
}

static rlca_status prepare_gae(int storage, const void *rewards, const void *values,
                               const uint8_t *terminated, const uint8_t *truncated,
                               const void *trunc_values, const void *bootstrap, float gamma,
                               float lambda, int64_t num_envs, int64_t T, void *advantages,
                               void *returns, Call *c) {
    *c = Call{};
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLCA_ERR_INVALID_VALUE;
    const rlca_status st = prepare_backward(kGae, storage, rewards, values, nullptr, nullptr,
                                            nullptr, terminated, truncated, trunc_values,
                                            bootstrap, advantages, returns, num_envs, T, c);
    c->bp.gamma = gamma;
    c->bp.lambda = lambda;
    set_precision(c->shape, T, product_bound(gamma, lambda), false);
    return st;
}

static rlca_status prepare_td_lambda(int storage, const void *rewards, const void *values,
                                     const uint8_t *terminated, const uint8_t *truncated,
                                     const void *trunc_values, const void *bootstrap,
                                     float gamma, float lambda, int64_t num_envs, int64_t T,
                                     void *returns, Call *c) {
    *c = Call{};
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLCA_ERR_INVALID_VALUE;
    const rlca_status st = prepare_backward(kTdLambda, storage, rewards, values, nullptr,
                                            nullptr, nullptr, terminated, truncated,
                                            trunc_values, bootstrap, returns, nullptr, num_envs,
                                            T, c);
    c->bp.gamma = gamma;
    c->bp.lambda = lambda;
    set_precision(c->shape, T, product_bound(gamma, lambda), false);
    return st;
}

static rlca_status prepare_discounted(int storage, const void *rewards,
                                      const uint8_t *terminated, const uint8_t *truncated,
                                      const void *trunc_values, const void *bootstrap,
                                      float gamma, int64_t num_envs, int64_t T, void *returns,
                                      Call *c) {
    *c = Call{};
    if (!unit_interval(gamma)) return RLCA_ERR_INVALID_VALUE;
    const rlca_status st = prepare_backward(kDiscounted, storage, rewards, nullptr, nullptr,
                                            nullptr, nullptr, terminated, truncated,
                                            trunc_values, bootstrap, returns, nullptr, num_envs,
                                            T, c);
    c->bp.gamma = gamma;
    set_precision(c->shape, T, {gamma, true}, false);
    return st;
}

static rlca_status prepare_vtrace(int storage, const void *rewards, const void *values,
                                  const void *behaviour_logp, const void *target_logp,
                                  const uint8_t *terminated, const uint8_t *truncated,
                                  const void *trunc_values, const void *bootstrap, float gamma,
                                  float lambda, float rho_bar, float c_bar, int64_t num_envs,
                                  int64_t T, void *vs, void *pg_advantages, Call *c) {
    *c = Call{};
    if (!unit_interval(gamma) || !unit_interval(lambda) || !positive_finite(rho_bar) ||
        !trace_clip(c_bar))
        return RLCA_ERR_INVALID_VALUE;
    const rlca_status st =
        prepare_backward(kVtrace, storage, rewards, values, nullptr, behaviour_logp,
                         target_logp, terminated, truncated, trunc_values, bootstrap, vs,
                         pg_advantages, num_envs, T, c);
    c->bp.gamma = gamma;
    c->bp.lambda = lambda;
    c->bp.rho_bar = rho_bar;
    c->bp.c_bar = c_bar;
    set_precision(c->shape, T, weighted_bound(gamma, lambda, c_bar), false);
    return st;
}

static rlca_status prepare_retrace(int storage, const void *rewards, const void *q_values,
                                   const void *expected_q, const void *behaviour_logp,
                                   const void *target_logp, const uint8_t *terminated,
                                   const uint8_t *truncated, const void *trunc_values,
                                   const void *bootstrap, float gamma, float lambda, float c_bar,
                                   int64_t num_envs, int64_t T, void *q_ret, Call *c) {
    *c = Call{};
    if (!unit_interval(gamma) || !unit_interval(lambda) || !trace_clip(c_bar))
        return RLCA_ERR_INVALID_VALUE;
    const rlca_status st = prepare_backward(kRetrace, storage, rewards, q_values, expected_q,
                                            behaviour_logp, target_logp, terminated, truncated,
                                            trunc_values, bootstrap, q_ret, nullptr, num_envs, T,
                                            c);
    c->bp.gamma = gamma;
    c->bp.lambda = lambda;
    c->bp.c_bar = c_bar;
    set_precision(c->shape, T, weighted_bound(gamma, lambda, c_bar), false);
    return st;
}

static rlca_status prepare_eligibility(int storage, const void *increments,
                                       const uint8_t *flags, int convention, float gamma,
                                       float lambda, int64_t num_envs, int64_t T, void *traces,
                                       Call *c) {
    *c = Call{};
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLCA_ERR_INVALID_VALUE;
    const rlca_status st = prepare_forward(kForwardFlags, storage, increments, false, flags,
                                           convention, gamma * lambda,
                                           (double)gamma * (double)lambda, nullptr, nullptr,
                                           num_envs, T, traces, c);
    set_precision(c->shape, T, product_bound(gamma, lambda), false);
    return st;
}

// dtype: RLCA_I32 (exact, wrapping) or a real storage type.
static rlca_status prepare_prefix_sum(const void *x, int dtype, const uint8_t *flags,
                                      int convention, int64_t num_envs, int64_t T, void *out,
                                      Call *c) {
    *c = Call{};
    const bool is_int = dtype == RLCA_I32;
    const int storage = is_int ? (int)kStoreF32 : storage_of(dtype);
    if (storage < 0) return RLCA_ERR_INVALID_VALUE;
    const rlca_status st = prepare_forward(kForwardFlags, storage, x, is_int, flags, convention,
                                           1.0f, 1.0, nullptr, nullptr, num_envs, T, out, c);
    set_precision(c->shape, T, {1.0f, true}, is_int);
    return st;
}

static rlca_status prepare_affine(int storage, const void *alpha, const void *beta,
                                  const void *carry, int direction, int64_t num_envs, int64_t T,
                                  void *out, Call *c) {
    *c = Call{};
    if (direction != RLCA_BACKWARD && direction != RLCA_FORWARD) return RLCA_ERR_INVALID_VALUE;
    const rlca_status st =
        direction == RLCA_BACKWARD
            ? prepare_backward(kAffineBackward, storage, alpha, beta, nullptr, nullptr, nullptr,
                               nullptr, nullptr, nullptr, carry, out, nullptr, num_envs, T, c)
            : prepare_forward(kForwardAffine, storage, alpha, false, nullptr, 0, 0.f, 0.0, beta,
                              carry, num_envs, T, out, c);
    // the caller's beta is unknown: fp64 wherever a value crosses waves
    set_precision(c->shape, T, {INFINITY, false}, false);
    return st;
}

// One rlca_call of a batch, prepared like its own entry point; `dtype` gives
// the storage of every real-valued array (and int32 for the prefix sum).
static rlca_status prepare_op(const rlca_call &k, Call *c) {
    const int st = storage_of(k.dtype);  // -1 (rejected) for RLCA_I32 outside the prefix sum
    switch (enum_code(k.op)) {
        case RLCA_OP_GAE:
            return prepare_gae(st, k.rewards, k.values, k.terminated, k.truncated,
                               k.trunc_values, k.bootstrap, k.gamma, k.lambda, k.num_envs, k.T,
                               k.out0, k.out1, c);
        case RLCA_OP_TD_LAMBDA:
            return prepare_td_lambda(st, k.rewards, k.values, k.terminated, k.truncated,
                                     k.trunc_values, k.bootstrap, k.gamma, k.lambda, k.num_envs,
                                     k.T, k.out0, c);
        case RLCA_OP_DISCOUNTED_RETURNS:
            return prepare_discounted(st, k.rewards, k.terminated, k.truncated, k.trunc_values,
                                      k.bootstrap, k.gamma, k.num_envs, k.T, k.out0, c);
        case RLCA_OP_VTRACE:
            return prepare_vtrace(st, k.rewards, k.values, k.behaviour_logp, k.target_logp,
                                  k.terminated, k.truncated, k.trunc_values, k.bootstrap,
                                  k.gamma, k.lambda, k.rho_bar, k.c_bar, k.num_envs, k.T,
                                  k.out0, k.out1, c);
        case RLCA_OP_RETRACE:
            return prepare_retrace(st, k.rewards, k.values, k.expected_q, k.behaviour_logp,
                                   k.target_logp, k.terminated, k.truncated, k.trunc_values,
                                   k.bootstrap, k.gamma, k.lambda, k.c_bar, k.num_envs, k.T,
                                   k.out0, c);
        case RLCA_OP_ELIGIBILITY_TRACES:
            return prepare_eligibility(st, k.rewards, k.terminated, k.convention, k.gamma,
                                       k.lambda, k.num_envs, k.T, k.out0, c);
        case RLCA_OP_EPISODIC_PREFIX_SUM:
            return prepare_prefix_sum(k.rewards, k.dtype, k.terminated, k.convention, k.num_envs,
                                      k.T, k.out0, c);
        case RLCA_OP_AFFINE_SCAN:
            return prepare_affine(st, k.rewards, k.values, k.bootstrap, k.direction, k.num_envs,
                                  k.T, k.out0, c);
    }
    *c = Call{};
    return RLCA_ERR_INVALID_VALUE;
}

static rlca_status run_one(rlca_status prepared, Call &c, hipStream_t stream) {
    return prepared != RLCA_OK ? prepared : launch_call(c, stream);
}

}  // namespace rlca

using namespace rlca;

// ------------------------------------------------------------ fused consumers

// Statistics launches (fp64 partial sums, more registers) fit one 16-wave
// workgroup per CU.  Measured on MI355X, 16 waves were 5-14% faster up to 256
// rows of 8192..131072 steps and 19% slower at 384..512 rows of 8192 steps,
// so larger calls keep 8 waves (same results, bit for bit).
static constexpr int64_t kWideMaxRowsStats = 256;
static LaunchShape stats_shape(LaunchShape s, int64_t num_envs) {
    if (s.waves == 16 && num_envs > kWideMaxRowsStats) s.waves = 8;
    return s;
}

// One (sum, sum of squares) pair per workgroup of the GAE launch, for
// whichever launch shape the pointers will select.
static uint32_t gae_stats_pairs(int64_t num_envs, int64_t T) {
    IoChoice choices[2 + kK] = {{kScalarIO, 0, 0, false}, {kVecRows, 0, 0, false}};
    for (int phase = 0; phase < kK; ++phase)
        choices[2 + phase] = {kVecSkew, (uint32_t)phase, 0, false};
    uint32_t most = 0;
    for (int i = 0; i < 2 + kK; ++i) {
        if (choices[i].io == kVecRows && T % kK != 0) continue;
        const uint32_t g =
            launch_grid(stats_shape(choose_shape(num_envs, T, choices[i], true), num_envs),
                        num_envs, T, kStatsMaxGrid);
        most = g > most ? g : most;
    }
    return most;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// No span of `extra` may overlap another one or any of the call's arrays.
static rlca_status check_extra_aliasing(const Call &c, const Span *extra, int n) {
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < c.nin; ++j)
            if (overlaps(extra[i].p, extra[i].bytes, c.ins[j].p, c.ins[j].bytes))
                return RLCA_ERR_ALIASING;
        for (int j = 0; j < c.nout; ++j)
            if (overlaps(extra[i].p, extra[i].bytes, c.outs[j].p, c.outs[j].bytes))
                return RLCA_ERR_ALIASING;
        for (int j = i + 1; j < n; ++j)
            if (overlaps(extra[i].p, extra[i].bytes, extra[j].p, extra[j].bytes))
                return RLCA_ERR_ALIASING;
    }
    return RLCA_OK;
}

// -------------------------------------------- statistics without a workspace
// rlca_gae_stats_noalloc keeps its per-workgroup partial sums in this
// library-owned buffer instead of a caller's workspace: one (sum, sum of
// squares) pair per workgroup of the statistics launch, whose grid never
// exceeds kStatsMaxGrid, so every size fits.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names
// a host-side stand-in, never device memory: the kernels get the address
// hipGetSymbolAddress returns for the current device (scratch_address).
// Its first kTicketBytes hold the ticket counters of the statistics launch
// (see kernels.hpp, finish_in_last_workgroup), which must start at zero:
// the first call on each device clears them, on its stream, and every call
// leaves them at zero.  Every pair the last workgroup reads was written by
// the same launch.
constexpr uint32_t kScratchPairs = 4096;
static_assert(kScratchPairs >= kStatsMaxGrid, "one pair per statistics workgroup");
static_assert(kTicketBytes + 16 * kScratchPairs == RLCA_GAE_STATS_SCRATCH_BYTES,
              "the header states the buffer's size");
static __device__ __align__(256) double scratch[(kTicketBytes + 16 * kScratchPairs) / 8];

// Zero the buffer's ticket counters: run once per device, before its first
// use (every call leaves them at zero).
__global__ void clear_tickets(uint32_t *counters) {
    for (uint32_t i = threadIdx.x; i < kTicketBytes / 4; i += blockDim.x) counters[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;
static std::atomic<void *> scratch_ptr[kMaxScratchDevices];
static std::mutex scratch_mutex;

// The device address of `scratch` on the device that runs `stream`, looked
// up on the first call for that device (with it current) and kept; that
// first call also enqueues the clearing of its ticket counters on `stream`.
static rlca_status scratch_address(hipStream_t stream, void **out) {
    int device = -1;
    if (stream == nullptr ? hipGetDevice(&device) != hipSuccess
                          : hipStreamGetDevice(stream, &device) != hipSuccess)
        return RLCA_ERR_HIP;
    if (device < 0 || device >= kMaxScratchDevices) return RLCA_ERR_HIP;
    void *p = scratch_ptr[device].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_ptr[device].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int current = -1;
            if (hipGetDevice(&current) != hipSuccess) return RLCA_ERR_HIP;
            if (current != device && hipSetDevice(device) != hipSuccess) return RLCA_ERR_HIP;
            void *addr = nullptr;
            const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (current != device && hipSetDevice(current) != hipSuccess) return RLCA_ERR_HIP;
            if (e != hipSuccess || addr == nullptr) return RLCA_ERR_HIP;
            uint32_t *counters = static_cast<uint32_t *>(addr);
            void *args[] = {&counters};
            if (hipLaunchKernel((const void *)clear_tickets, dim3(1), dim3(256), args, 0,
                                stream) != hipSuccess)
                return RLCA_ERR_HIP;
            p = addr;
            scratch_ptr[device].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RLCA_OK;
}

extern "C" {

rlca_status rlca_gae(const float *rewards, const float *values, const uint8_t *terminated,
                     const uint8_t *truncated, const float *trunc_values,
                     const float *bootstrap, float gamma, float lambda, int64_t num_envs,
                     int64_t T, float *advantages, float *returns, hipStream_t stream) {
    Call c;
    const rlca_status st =
        prepare_gae(kStoreF32, rewards, values, terminated, truncated, trunc_values, bootstrap,
                    gamma, lambda, num_envs, T, advantages, returns, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_td_lambda(const float *rewards, const float *values,
                           const uint8_t *terminated, const uint8_t *truncated,
                           const float *trunc_values, const float *bootstrap, float gamma,
                           float lambda, int64_t num_envs, int64_t T, float *returns,
                           hipStream_t stream) {
    Call c;
    const rlca_status st =
        prepare_td_lambda(kStoreF32, rewards, values, terminated, truncated, trunc_values,
                          bootstrap, gamma, lambda, num_envs, T, returns, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_discounted_returns(const float *rewards, const uint8_t *terminated,
                                    const uint8_t *truncated, const float *trunc_values,
                                    const float *bootstrap, float gamma, int64_t num_envs,
                                    int64_t T, float *returns, hipStream_t stream) {
    Call c;
    const rlca_status st =
        prepare_discounted(kStoreF32, rewards, terminated, truncated, trunc_values, bootstrap,
                           gamma, num_envs, T, returns, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_vtrace(const float *rewards, const float *values, const float *behaviour_logp,
                        const float *target_logp, const uint8_t *terminated,
                        const uint8_t *truncated, const float *trunc_values,
                        const float *bootstrap, float gamma, float lambda, float rho_bar,
                        float c_bar, int64_t num_envs, int64_t T, float *vs,
                        float *pg_advantages, hipStream_t stream) {
    Call c;
    const rlca_status st =
        prepare_vtrace(kStoreF32, rewards, values, behaviour_logp, target_logp, terminated,
                       truncated, trunc_values, bootstrap, gamma, lambda, rho_bar, c_bar,
                       num_envs, T, vs, pg_advantages, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_retrace(const float *rewards, const float *q_values, const float *expected_q,
                         const float *behaviour_logp, const float *target_logp,
                         const uint8_t *terminated, const uint8_t *truncated,
                         const float *trunc_values, const float *bootstrap, float gamma,
                         float lambda, float c_bar, int64_t num_envs, int64_t T,
                         float *q_ret, hipStream_t stream) {
    Call c;
    const rlca_status st =
        prepare_retrace(kStoreF32, rewards, q_values, expected_q, behaviour_logp, target_logp,
                        terminated, truncated, trunc_values, bootstrap, gamma, lambda, c_bar,
                        num_envs, T, q_ret, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_eligibility_traces(const float *increments, const uint8_t *flags,
                                    rlca_reset_convention convention, float gamma,
                                    float lambda, int64_t num_envs, int64_t T, float *traces,
                                    hipStream_t stream) {
    Call c;
    const rlca_status st = prepare_eligibility(kStoreF32, increments, flags,
                                               enum_code(convention), gamma, lambda, num_envs, T,
                                               traces, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_episodic_prefix_sum(const void *x, rlca_dtype dtype, const uint8_t *flags,
                                     rlca_reset_convention convention, int64_t num_envs,
                                     int64_t T, void *out, hipStream_t stream) {
    Call c;
    const rlca_status st = prepare_prefix_sum(x, enum_code(dtype), flags, enum_code(convention),
                                              num_envs, T, out, &c);
    return run_one(st, c, stream);
}

rlca_status rlca_affine_scan(const float *alpha, const float *beta, const float *carry,
                             rlca_direction direction, int64_t num_envs, int64_t T, float *out,
                             hipStream_t stream) {
    Call c;
    const rlca_status st =
        prepare_affine(kStoreF32, alpha, beta, carry, enum_code(direction), num_envs, T, out, &c);
    return run_one(st, c, stream);
}

size_t rlca_gae_stats_workspace_size(int64_t num_envs, int64_t T) {
    int64_t n;
    if (check_sizes(num_envs, T, &n) != RLCA_OK || n == 0) return 0;
    return kTicketBytes + 16 * (size_t)gae_stats_pairs(num_envs, T);
}

rlca_status rlca_gae_stats(const float *rewards, const float *values, const uint8_t *terminated,
                           const uint8_t *truncated, const float *trunc_values,
                           const float *bootstrap, float gamma, float lambda, int64_t num_envs,
                           int64_t T, float *advantages, float *returns, double *stats,
                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    Call c;
    rlca_status st = prepare_gae(kStoreF32, rewards, values, terminated, truncated,
                                 trunc_values, bootstrap, gamma, lambda, num_envs, T, advantages,
                                 returns, &c);
    if (st != RLCA_OK || c.empty) return st;
    c.shape = stats_shape(c.shape, num_envs);
    if (stats == nullptr || workspace == nullptr) return RLCA_ERR_NULL_POINTER;
    if (!aligned(stats, 8) || !aligned(workspace, 8)) return RLCA_ERR_MISALIGNED;
    const uint32_t pairs = launch_grid(c.shape, num_envs, T, kStatsMaxGrid);
    const size_t need = kTicketBytes + 16 * (size_t)pairs;
    if (workspace_bytes < need) return RLCA_ERR_INVALID_SIZE;
    const Span extra[] = {{stats, 16}, {workspace, need}};
    st = check_extra_aliasing(c, extra, 2);
    if (st != RLCA_OK) return st;
    c.bp.stats_partials =
        reinterpret_cast<double *>(static_cast<char *>(workspace) + kTicketBytes);
    c.bp.stats = stats;
    c.bp.stats_count = num_envs * T;
    return launch_gae_stats(c.bp, c.shape, stream);
}

rlca_status rlca_gae_stats_noalloc(const float *rewards, const float *values,
                                   const uint8_t *terminated, const uint8_t *truncated,
                                   const float *trunc_values, const float *bootstrap, float gamma,
                                   float lambda, int64_t num_envs, int64_t T, float *advantages,
                                   float *returns, double *stats, hipStream_t stream) {
    Call c;
    rlca_status st = prepare_gae(kStoreF32, rewards, values, terminated, truncated,
                                 trunc_values, bootstrap, gamma, lambda, num_envs, T, advantages,
                                 returns, &c);
    if (st != RLCA_OK || c.empty) return st;
    c.shape = stats_shape(c.shape, num_envs);
    if (stats == nullptr) return RLCA_ERR_NULL_POINTER;
    if (!aligned(stats, 8)) return RLCA_ERR_MISALIGNED;
    const uint32_t pairs = launch_grid(c.shape, num_envs, T, kStatsMaxGrid);
    if (pairs > kScratchPairs) return RLCA_ERR_INVALID_SIZE;
    const Span extra[] = {{stats, 16}};
    st = check_extra_aliasing(c, extra, 1);
    if (st != RLCA_OK) return st;
    void *buffer = nullptr;
    st = scratch_address(stream, &buffer);
    if (st != RLCA_OK) return st;
    c.bp.stats_partials = reinterpret_cast<double *>(static_cast<char *>(buffer) + kTicketBytes);
    c.bp.stats = stats;
    c.bp.stats_count = num_envs * T;
    return launch_gae_stats(c.bp, c.shape, stream);
}

size_t rlca_ppo_clip_loss_workspace_size(int64_t num_envs, int64_t T) {
    int64_t n;
    if (check_sizes(num_envs, T, &n) != RLCA_OK || n == 0) return 0;
    return kTicketBytes + 8 * (size_t)ppo_grid(n);
}

rlca_status rlca_ppo_clip_loss(const float *advantages, const double *stats,
                               const float *logp_new, const float *logp_old, float clip_eps,
                               float norm_eps, int64_t num_envs, int64_t T, float *grad_logp_new,
                               double *loss, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    int64_t n;
    rlca_status st = check_sizes(num_envs, T, &n);
    if (st != RLCA_OK) return st;
    if (!(clip_eps >= 0.f && clip_eps < 1.f) || !(norm_eps >= 0.f && isfinite(norm_eps)))
        return RLCA_ERR_INVALID_VALUE;
    if (n == 0) return RLCA_OK;
    if (advantages == nullptr || logp_new == nullptr || logp_old == nullptr || loss == nullptr ||
        workspace == nullptr)
        return RLCA_ERR_NULL_POINTER;
    const void *f32[] = {advantages, logp_new, logp_old, grad_logp_new};
    st = check_aligned(f32, 4, 4);
    if (st != RLCA_OK) return st;
    if (!aligned(stats, 8) || !aligned(loss, 8) || !aligned(workspace, 8))
        return RLCA_ERR_MISALIGNED;
    const size_t need = kTicketBytes + 8 * (size_t)ppo_grid(n);
    if (workspace_bytes < need) return RLCA_ERR_INVALID_SIZE;
    Call c = Call{};  // byte ranges only, for the aliasing check
    const size_t fb = (size_t)n * 4;
    c.ins[c.nin++] = {advantages, fb};
    c.ins[c.nin++] = {logp_new, fb};
    c.ins[c.nin++] = {logp_old, fb};
    c.ins[c.nin++] = {stats, 16};
    const Span outs[] = {{grad_logp_new, fb}, {loss, 8}, {workspace, need}};
    st = check_extra_aliasing(c, outs, 3);
    if (st != RLCA_OK) return st;
    const bool vec = aligned(advantages, 16) && aligned(logp_new, 16) && aligned(logp_old, 16) &&
                     aligned(grad_logp_new, 16);
    return launch_ppo_clip_loss(advantages, stats, logp_new, logp_old, clip_eps, norm_eps, n,
                                vec, grad_logp_new, workspace, loss, stream);
}

rlca_status rlca_run_batch(const rlca_call *calls, int count, hipStream_t stream) {
    if (count < 0 || count > RLCA_MAX_BATCH) return RLCA_ERR_INVALID_SIZE;
    if (count > 0 && calls == nullptr) return RLCA_ERR_NULL_POINTER;
    Call prepared[RLCA_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        const rlca_status st = prepare_op(calls[i], &prepared[i]);
        if (st != RLCA_OK) return st;
    }
    // The calls run concurrently: no call may write what another reads or writes.
    for (int i = 0; i < count; ++i) {
        for (int j = 0; j < count; ++j) {
            if (i == j || prepared[i].empty || prepared[j].empty) continue;
            const Call &a = prepared[i], &b = prepared[j];
            for (int o = 0; o < a.nout; ++o) {
                for (int k = 0; k < b.nin; ++k)
                    if (overlaps(a.outs[o].p, a.outs[o].bytes, b.ins[k].p, b.ins[k].bytes))
                        return RLCA_ERR_ALIASING;
                for (int k = 0; k < b.nout; ++k)
                    if (overlaps(a.outs[o].p, a.outs[o].bytes, b.outs[k].p, b.outs[k].bytes))
                        return RLCA_ERR_ALIASING;
            }
        }
    }
    // Vector-path, single-launch calls share grouped launches; the rest
    // (unaligned, chunked or beyond the grid cap) are enqueued one by one.  Members of one grouped
    // launch share a shape class (one kernel per class) and the storage type
    // of their real-valued arrays (int32 sums join the 4-byte group).  A
    // grouped launch that would hold one call runs that call's own kernel.
    struct Pending {
        GroupedLaunch launch;
        int members[kMaxGroupedCalls];
        int count;
        int storage;
    };
    Pending pending[kGroupClasses];
    for (Pending &g : pending) g.count = 0, g.storage = kStoreF32, g.launch.workgroups = 0;
    auto flush = [&](int cls) -> rlca_status {
        Pending &g = pending[cls];
        if (g.count == 0) return RLCA_OK;
        const int n = g.count;
        g.count = 0;
        if (n == 1) return launch_call(prepared[g.members[0]], stream);
        for (int m = n; m < kMaxGroupedCalls; ++m) g.launch.head[m] = kHeadEndMask;
        return launch_grouped(g.launch, g.storage, cls, stream);
    };
    for (int i = 0; i < count; ++i) {
        Call &c = prepared[i];
        if (c.empty) continue;
        GroupedCall member;
        int variant = 0;
        uint32_t wgs = 0;
        if (!grouped_member(c, &member, &variant, &wgs)) {
            const rlca_status st = launch_call(c, stream);
            if (st != RLCA_OK) return st;
            continue;
        }
        const bool weighted = c.backward && (c.est == kVtrace || c.est == kRetrace);
        const int cls = group_class(c.shape, weighted);
        Pending &g = pending[cls];
        if (g.count == kMaxGroupedCalls || g.launch.workgroups + wgs > kMaxGrid ||
            (g.count > 0 && c.storage != g.storage)) {
            const rlca_status st = flush(cls);
            if (st != RLCA_OK) return st;
        }
        if (g.count == 0) g.launch.workgroups = 0, g.storage = c.storage;
        g.launch.workgroups += wgs;
        g.launch.args.calls[g.count] = member;
        g.launch.head[g.count] = g.launch.workgroups | ((uint32_t)variant << kHeadVariantShift);
        g.members[g.count++] = i;
    }
    for (int cls = 0; cls < kGroupClasses; ++cls) {
        const rlca_status st = flush(cls);
        if (st != RLCA_OK) return st;
    }
    return RLCA_OK;
}

const char *rlca_status_string(rlca_status status) {
    switch (enum_code(status)) {
        case RLCA_OK: return "ok";
        case RLCA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case RLCA_ERR_INVALID_SIZE: return "invalid size (negative, too large or overflowing)";
        case RLCA_ERR_INVALID_VALUE: return "invalid parameter value";
        case RLCA_ERR_ALIASING: return "an output overlaps an input or another output";
        case RLCA_ERR_MISALIGNED:
            return "an array is not aligned to its element size (8 bytes for workspace, stats "
                   "and loss)";
        case RLCA_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
