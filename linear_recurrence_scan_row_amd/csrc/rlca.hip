// rlca.hip -- fused credit-assignment scans for MI355X (gfx950) behind the C ABI of rlca.h.
//
// One launch per call.  Each workgroup owns a contiguous range of whole rows
// of the [num_envs, T] rollout (rows are independent; "rl-triton", paperlayer.ai
// summary, §4 Kernel design) and walks it in tiles of NW*64*K steps:
//   1. coalesced loads of the raw rollout, each element read once (dwordx4 per
//      lane for fp32 streams, one dword per four flag bytes);
//   2. boundary resolution and the estimator's (alpha_t, beta_t) built in
//      registers (summary §3.1 / §3.2; §4 Fusion);
//   3. the shared affine scan of scan_core.hpp (lane fold, wave64 DPP scan,
//      LDS wave totals, tile carry);
//   4. one store of each output.
// Short rows are packed many to a tile: the window edge is folded into
// alpha_{T-1} with beta_{T-1} = 0, so a row end is a chain cut like any done
// step and rows never interact.  Long rows take several tiles with the carry
// kept in registers, so there is no length limit and no LDS growth with T.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rlca.h"
#include "scan_core.hpp"

namespace rlca {

// Tile shape: NW waves per workgroup, K consecutive steps per lane.
constexpr int kNW = 4;
constexpr int kK = 4;
constexpr int kThreads = kNW * kWave;
constexpr uint32_t kTile = kThreads * kK;
// Upper bound on the launch grid; larger problems loop over row groups.
constexpr uint32_t kMaxGrid = 1u << 20;

enum Estimator : int { kGae = 0, kTdLambda = 1, kDiscounted = 2, kVtrace = 3, kRetrace = 4 };

struct Geometry {
    int64_t num_envs;
    uint32_t T;
    uint32_t rows_per_group;  // whole rows owned by one workgroup iteration
    uint32_t num_groups;
};

struct BackwardParams {
    const float *rewards;
    const float *values;  // V(s_t); Q(s_t, a_t) for Retrace
    const float *expected_q;
    const float *behaviour_logp;
    const float *target_logp;
    const uint8_t *terminated;
    const uint8_t *truncated;
    const float *trunc_values;
    const float *bootstrap;
    float *out0;  // advantages / returns / vs / q_ret
    float *out1;  // GAE returns or V-Trace pg advantages; may be null
    float gamma, lambda, rho_bar, c_bar;
    Geometry geo;
};

struct ForwardParams {
    const void *x;
    const uint8_t *flags;
    void *out;
    float decay;  // gamma*lambda for traces, 1 for prefix sums
    Geometry geo;
};

// ---------------------------------------------------------------- memory access

// `p` points at the workgroup's first element; `off` is the lane's first step
// relative to it and `L` the number of valid steps.  With VEC the caller
// guarantees 16-byte alignment of p + off and L % 4 == 0, so a 4-step group
// is either wholly valid or wholly past the end.

template <bool VEC, typename E>
__device__ __forceinline__ void load_steps(E (&x)[kK], const E *__restrict__ p, uint32_t off,
                                           uint32_t L) {
    static_assert(sizeof(E) == 4, "32-bit elements");
    // Element-typed vector: its lanes are read by value (no bit cast of a
    // vector element, which this compiler lowers as a read of element 0).
    typedef E vec4 __attribute__((ext_vector_type(4)));
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < kK; j += 4) {
            vec4 q = {E(0), E(0), E(0), E(0)};
            if (off + j < L) q = *reinterpret_cast<const vec4 *>(p + off + j);
            x[j + 0] = q.x;
            x[j + 1] = q.y;
            x[j + 2] = q.z;
            x[j + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kK; ++i) x[i] = (off + i < L) ? p[off + i] : E(0);
    }
}

template <bool VEC>
__device__ __forceinline__ void load_flags(bool (&f)[kK], const uint8_t *__restrict__ p,
                                           uint32_t off, uint32_t L) {
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < kK; j += 4) {
            uint32_t q = 0;
            if (off + j < L) q = *reinterpret_cast<const uint32_t *>(p + off + j);
#pragma unroll
            for (int i = 0; i < 4; ++i) f[j + i] = ((q >> (8 * i)) & 0xffu) != 0;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kK; ++i) f[i] = (off + i < L) ? (p[off + i] != 0) : false;
    }
}

template <bool VEC, typename E>
__device__ __forceinline__ void store_steps(E *__restrict__ p, const E (&x)[kK], uint32_t off,
                                            uint32_t L) {
    typedef E vec4 __attribute__((ext_vector_type(4)));
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < kK; j += 4) {
            if (off + j < L) {
                const vec4 q = {x[j], x[j + 1], x[j + 2], x[j + 3]};
                __builtin_nontemporal_store(q, reinterpret_cast<vec4 *>(p + off + j));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kK; ++i)
            if (off + i < L) p[off + i] = x[i];
    }
}

// Row-local step index t and row offset of each of the lane's K steps.
__device__ __forceinline__ void step_positions(uint32_t off, uint32_t T, uint32_t (&t)[kK],
                                               uint32_t (&row)[kK]) {
    uint32_t r = off / T;
    uint32_t s = off - r * T;
#pragma unroll
    for (int i = 0; i < kK; ++i) {
        t[i] = s;
        row[i] = r;
        if (++s == T) {
            s = 0;
            ++r;
        }
    }
}

__device__ __forceinline__ float importance_ratio(float target_logp, float behaviour_logp) {
    const float l = fminf(fmaxf(target_logp - behaviour_logp, -RLCA_LOG_RATIO_CLIP),
                          RLCA_LOG_RATIO_CLIP);
    return expf(l);
}

// ------------------------------------------------------------- backward kernel
// A_t = alpha_t + beta_t * A_{t+1}.  Lanes take chunks in reverse time order, so
// the lane-order scan of scan_core.hpp runs from the end of the tile backwards.
template <int EST, bool TRUNC, bool VEC>
__global__ __launch_bounds__(kThreads) void backward_scan(BackwardParams p) {
    __shared__ float lds_a[2 * kNW], lds_b[2 * kNW];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint32_t chunk = (kNW - 1 - w) * kWave + (kWave - 1 - lane);
    const uint32_t T = p.geo.T;
    const float gamma = p.gamma;
    int parity = 0;

    for (uint32_t g = blockIdx.x; g < p.geo.num_groups; g += gridDim.x) {
        const int64_t row0 = (int64_t)g * p.geo.rows_per_group;
        const int64_t rows_left = p.geo.num_envs - row0;
        const uint32_t rows =
            rows_left < (int64_t)p.geo.rows_per_group ? (uint32_t)rows_left : p.geo.rows_per_group;
        const uint32_t L = rows * T;
        const int64_t base = row0 * (int64_t)T;
        const uint32_t ntiles = (L + kTile - 1) / kTile;
        float carry = 0.f;  // A just after the current tile (A_T = 0: edges live in alpha)

        for (uint32_t it = 0; it < ntiles; ++it) {
            const uint32_t off = (ntiles - 1 - it) * kTile + chunk * kK;
            uint32_t t[kK], row[kK];
            step_positions(off, T, t, row);

            // ---- 1. loads (each input element once)
            float r[kK], v[kK], eq[kK], mu[kK], pi[kK], tv[kK];
            bool term[kK], trunc[kK];
            load_steps<VEC>(r, p.rewards + base, off, L);
            if constexpr (EST != kDiscounted) load_steps<VEC>(v, p.values + base, off, L);
            if constexpr (EST == kRetrace) load_steps<VEC>(eq, p.expected_q + base, off, L);
            if constexpr (EST == kVtrace || EST == kRetrace) {
                load_steps<VEC>(mu, p.behaviour_logp + base, off, L);
                load_steps<VEC>(pi, p.target_logp + base, off, L);
            }
            load_flags<VEC>(term, p.terminated + base, off, L);
            if constexpr (TRUNC) {
                load_flags<VEC>(trunc, p.truncated + base, off, L);
                load_steps<VEC>(tv, p.trunc_values + base, off, L);
            }

            // Loads whose addresses depend only on positions are issued with
            // the main batch: the bootstrap of rows ending in this chunk, and
            // for lane 0 the first step of the next chunk in time (its
            // neighbour lane - 1 sits in another wave or tile).
            bool valid[kK];
            float boot[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                valid[i] = off + i < L;
                boot[i] = 0.f;
                if (valid[i] && t[i] == T - 1 && p.bootstrap != nullptr)
                    boot[i] = p.bootstrap[row0 + row[i]];
            }
            const bool halo_in_mem = lane == 0 && off + kK < L;
            const int64_t jh = base + off + kK;
            float v_first = 0.f, mu_first = 0.f, pi_first = 0.f, eq_first = 0.f;
            if (halo_in_mem) {
                if constexpr (EST == kGae || EST == kTdLambda || EST == kVtrace)
                    v_first = p.values[jh];
                if constexpr (EST == kRetrace) {
                    mu_first = p.behaviour_logp[jh];
                    pi_first = p.target_logp[jh];
                    eq_first = p.expected_q[jh];
                }
            }

            // ---- 2. boundary resolution
            bool cont[kK];
            float succ[kK];  // successor value where the chain stops
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const bool tr = TRUNC && trunc[i] && !term[i];
                const bool edge = t[i] == T - 1;
                cont[i] = valid[i] && !term[i] && !tr && !edge;
                float s = term[i] ? 0.f : boot[i];
                if constexpr (TRUNC) {
                    if (tr) s = tv[i];
                }
                succ[i] = s;
            }

            // ---- 3. halo: the first step of the next chunk in time, from lane - 1
            float v_next = 0.f, c_next = 0.f, eq_next = 0.f;
            if constexpr (EST == kGae || EST == kTdLambda || EST == kVtrace)
                v_next = from_lower_lane(v[0], v_first);
            float c[kK];
            if constexpr (EST == kVtrace || EST == kRetrace) {
#pragma unroll
                for (int i = 0; i < kK; ++i)
                    c[i] = p.lambda * fminf(p.c_bar, importance_ratio(pi[i], mu[i]));
            }
            if constexpr (EST == kRetrace) {
                const float c_first =
                    p.lambda * fminf(p.c_bar, importance_ratio(pi_first, mu_first));
                c_next = from_lower_lane(c[0], c_first);
                eq_next = from_lower_lane(eq[0], eq_first);
            }

            // ---- 4. coefficients in registers
            float alpha[kK], beta[kK], aux[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const bool k = cont[i];
                float a, b, x = 0.f;
                if constexpr (EST == kGae) {
                    const float vn = i + 1 < kK ? v[i + 1] : v_next;
                    a = r[i] + gamma * (k ? vn : succ[i]) - v[i];
                    b = k ? gamma * p.lambda : 0.f;
                } else if constexpr (EST == kTdLambda) {
                    const float vn = i + 1 < kK ? v[i + 1] : v_next;
                    a = k ? r[i] + gamma * (1.f - p.lambda) * vn : r[i] + gamma * succ[i];
                    b = k ? gamma * p.lambda : 0.f;
                } else if constexpr (EST == kDiscounted) {
                    a = k ? r[i] : r[i] + gamma * succ[i];
                    b = k ? gamma : 0.f;
                } else if constexpr (EST == kVtrace) {
                    const float vn = i + 1 < kK ? v[i + 1] : v_next;
                    const float rho = fminf(p.rho_bar, importance_ratio(pi[i], mu[i]));
                    a = rho * (r[i] + gamma * (k ? vn : succ[i]) - v[i]);
                    b = k ? gamma * c[i] : 0.f;
                    x = k ? gamma * rho : 0.f;  // pg_t = alpha_t + gamma rho_t A_{t+1}
                } else {  // Retrace: decay uses the next step's trace coefficient
                    const float cn = i + 1 < kK ? c[i + 1] : c_next;
                    const float en = i + 1 < kK ? eq[i + 1] : eq_next;
                    a = r[i] + gamma * (k ? en : succ[i]) - v[i];
                    b = k ? gamma * cn : 0.f;
                }
                alpha[i] = valid[i] ? a : 0.f;
                beta[i] = valid[i] ? b : 1.f;
                aux[i] = x;
            }

            // ---- 5. scan: lane fold (latest step first), then wave / workgroup
            float fa = 0.f, fb = 1.f;  // identity; step i applied after the later steps
#pragma unroll
            for (int i = kK - 1; i >= 0; --i) {
                fa = alpha[i] + beta[i] * fa;
                fb = beta[i] * fb;
            }
            float carry_out;
            float A = block_carry_in<kNW>(fa, fb, carry, lds_a, lds_b, parity, carry_out);
            parity ^= 1;
            carry = carry_out;

            // ---- 6. outputs, one store each
            float o0[kK], o1[kK];
#pragma unroll
            for (int i = kK - 1; i >= 0; --i) {
                const float An = A;  // A_{t+1}
                A = alpha[i] + beta[i] * An;
                if constexpr (EST == kGae) {
                    o0[i] = A;
                    o1[i] = A + v[i];
                } else if constexpr (EST == kVtrace) {
                    o0[i] = v[i] + A;
                    o1[i] = alpha[i] + aux[i] * An;
                } else if constexpr (EST == kRetrace) {
                    o0[i] = v[i] + A;
                    o1[i] = 0.f;
                } else {
                    o0[i] = A;
                    o1[i] = 0.f;
                }
            }
            store_steps<VEC>(p.out0 + base, o0, off, L);
            if constexpr (EST == kGae || EST == kVtrace) {
                if (p.out1 != nullptr) store_steps<VEC>(p.out1 + base, o1, off, L);
            }
        }
    }
}

// -------------------------------------------------------------- forward kernel
// A_t = alpha_t + beta_t * A_{t-1} with alpha = x, beta = decay, beta = 0 where a
// new episode starts (summary §5: the forward scans cut where d_{t-1} = 1).
// V = float (traces, f32 sums) or uint32_t (int32 sums, wrap-around).
template <typename V, bool AFTER_DONE, bool VEC>
__global__ __launch_bounds__(kThreads) void forward_scan(ForwardParams p) {
    __shared__ V lds_a[2 * kNW], lds_b[2 * kNW];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint32_t chunk = w * kWave + lane;
    const uint32_t T = p.geo.T;
    const V decay = __builtin_bit_cast(V, __builtin_bit_cast(uint32_t, p.decay));
    const V *__restrict__ xs = static_cast<const V *>(p.x);
    V *__restrict__ out = static_cast<V *>(p.out);
    int parity = 0;

    for (uint32_t g = blockIdx.x; g < p.geo.num_groups; g += gridDim.x) {
        const int64_t row0 = (int64_t)g * p.geo.rows_per_group;
        const int64_t rows_left = p.geo.num_envs - row0;
        const uint32_t rows =
            rows_left < (int64_t)p.geo.rows_per_group ? (uint32_t)rows_left : p.geo.rows_per_group;
        const uint32_t L = rows * T;
        const int64_t base = row0 * (int64_t)T;
        const uint32_t ntiles = (L + kTile - 1) / kTile;
        V carry = V(0);

        for (uint32_t it = 0; it < ntiles; ++it) {
            const uint32_t off = it * kTile + chunk * kK;
            uint32_t t[kK], row[kK];
            step_positions(off, T, t, row);
            V x[kK];
            bool f[kK];
            load_steps<VEC>(x, xs + base, off, L);
            load_flags<VEC>(f, p.flags + base, off, L);
            bool prev_done = false;  // flag of the step before the lane's chunk
            if constexpr (AFTER_DONE) {
                const bool first = (lane == 0 && off > 0 && off - 1 < L)
                                       ? p.flags[base + off - 1] != 0
                                       : false;
                prev_done = from_lower_lane<uint32_t>(f[kK - 1] ? 1u : 0u, first ? 1u : 0u) != 0;
            }
            V alpha[kK], beta[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const bool valid = off + i < L;
                bool reset = t[i] == 0;
                if constexpr (AFTER_DONE) {
                    reset = reset || (i == 0 ? prev_done : f[i - 1]);
                } else {
                    reset = reset || f[i];
                }
                alpha[i] = valid ? x[i] : V(0);
                beta[i] = valid ? (reset ? V(0) : decay) : V(1);
            }
            V fa = V(0), fb = V(1);
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                fa = alpha[i] + beta[i] * fa;
                fb = beta[i] * fb;
            }
            V carry_out;
            V A = block_carry_in<kNW>(fa, fb, carry, lds_a, lds_b, parity, carry_out);
            parity ^= 1;
            carry = carry_out;
            V o[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                A = alpha[i] + beta[i] * A;
                o[i] = A;
            }
            store_steps<VEC>(out + base, o, off, L);
            (void)row;
        }
    }
}

// ------------------------------------------------------------------ host side

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

static bool vec_ok(int64_t T, const void *const *f32, int nf, const void *const *u8, int nu) {
    if (T % 4 != 0) return false;
    for (int i = 0; i < nf; ++i)
        if (f32[i] != nullptr && ((uintptr_t)f32[i] & 15u) != 0) return false;
    for (int i = 0; i < nu; ++i)
        if (u8[i] != nullptr && ((uintptr_t)u8[i] & 3u) != 0) return false;
    return true;
}

static Geometry make_geometry(int64_t num_envs, int64_t T, uint32_t *grid) {
    Geometry g;
    g.num_envs = num_envs;
    g.T = (uint32_t)T;
    g.rows_per_group = (uint32_t)T <= kTile ? kTile / (uint32_t)T : 1u;
    const int64_t groups = (num_envs + g.rows_per_group - 1) / g.rows_per_group;
    g.num_groups = (uint32_t)groups;
    *grid = groups < (int64_t)kMaxGrid ? (uint32_t)groups : kMaxGrid;
    return g;
}

template <typename P>
static rlca_status launch(const void *kernel, uint32_t grid, P &params, hipStream_t stream) {
    void *args[] = {&params};
    const hipError_t e =
        hipLaunchKernel(kernel, dim3(grid), dim3(kThreads), args, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

template <int EST>
static rlca_status launch_backward(BackwardParams &p, bool trunc, bool vec, uint32_t grid,
                                   hipStream_t s) {
    const void *k;
    if (trunc)
        k = vec ? (const void *)backward_scan<EST, true, true>
                : (const void *)backward_scan<EST, true, false>;
    else
        k = vec ? (const void *)backward_scan<EST, false, true>
                : (const void *)backward_scan<EST, false, false>;
    return launch(k, grid, p, s);
}

static rlca_status run_backward(int est, BackwardParams &p, int64_t T, hipStream_t s) {
    const void *f32[] = {p.rewards, p.values, p.expected_q, p.behaviour_logp, p.target_logp,
                         p.trunc_values, p.out0, p.out1};
    const void *u8[] = {p.terminated, p.truncated};
    const bool vec = vec_ok(T, f32, 8, u8, 2);
    const bool trunc = p.truncated != nullptr;
    uint32_t grid;
    p.geo = make_geometry(p.geo.num_envs, T, &grid);
    switch (est) {
        case kGae: return launch_backward<kGae>(p, trunc, vec, grid, s);
        case kTdLambda: return launch_backward<kTdLambda>(p, trunc, vec, grid, s);
        case kDiscounted: return launch_backward<kDiscounted>(p, trunc, vec, grid, s);
        case kVtrace: return launch_backward<kVtrace>(p, trunc, vec, grid, s);
        default: return launch_backward<kRetrace>(p, trunc, vec, grid, s);
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
    const bool vec = vec_ok(T, f32, 2, u8, 1);
    ForwardParams p = {};
    p.x = x;
    p.flags = flags;
    p.out = out;
    p.decay = is_int ? __builtin_bit_cast(float, 1u) : decay;
    uint32_t grid;
    p.geo = make_geometry(num_envs, T, &grid);
    const bool after = conv == RLCA_RESET_AFTER_DONE;
    const void *k;
    if (is_int) {
        if (after)
            k = vec ? (const void *)forward_scan<uint32_t, true, true>
                    : (const void *)forward_scan<uint32_t, true, false>;
        else
            k = vec ? (const void *)forward_scan<uint32_t, false, true>
                    : (const void *)forward_scan<uint32_t, false, false>;
    } else {
        if (after)
            k = vec ? (const void *)forward_scan<float, true, true>
                    : (const void *)forward_scan<float, true, false>;
        else
            k = vec ? (const void *)forward_scan<float, false, true>
                    : (const void *)forward_scan<float, false, false>;
    }
    return launch(k, grid, p, stream);
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
