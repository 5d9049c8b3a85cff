// kernels.hpp -- the fused credit-assignment kernels for MI355X (gfx950).
//
// Each workgroup owns a window of the [num_envs, T] rollout (rows are
// independent; "rl-triton", paperlayer.ai summary, §4 Kernel design) and walks
// it in tiles of NW*64*K steps:
//   1. coalesced loads of the raw rollout, each element read once (dwordx4 per
//      lane for fp32 streams, one dword per four flag bytes);
//   2. boundary resolution and the estimator's (alpha_t, beta_t) built in
//      registers (summary §3.1 / §3.2; §4 Fusion);
//   3. the shared affine scan of scan_core.hpp (lane fold, wave64 DPP scan,
//      LDS wave totals, tile carry);
//   4. one store of each output.
// Full mode: a window is a range of whole rows.  Short rows are packed many
// to a tile: the window edge is folded into alpha_{T-1} with beta_{T-1} = 0,
// so a row end is a chain cut like any done step and rows never interact.
// Long rows take several tiles with the carry kept in registers, so there is
// no length limit and no LDS growth with T.
// Chunk modes (few long rows): a window is one tile-sized chunk of one row,
// so every chunk of every row runs in parallel.  Three launches: each chunk
// folds its steps into one affine map (aggregate mode), a small kernel scans
// the chunk maps of each row into per-chunk carries, and each chunk runs
// again from its carry (apply mode).  Both hand-offs go through the first
// word(s) of the chunk's own slice of the first output array, which the
// apply pass overwrites last; no other memory is used.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rlca.h"
#include "scan_core.hpp"

namespace rlca {

// K = 4 consecutive steps per lane: one dwordx4 load per fp32 stream (dwordx2
// for 16-bit storage, one dword per flag stream).  Wider per-lane chunks make
// one load instruction touch lanes 32+ bytes apart and lose coalescing;
// narrower ones measured no faster at 4096 x 128 and slower beyond.
constexpr int kK = 4;

// Waves per workgroup in the chunk modes; the chunk is one tile.
constexpr int kChunkWaves = 8;
constexpr uint32_t kChunkSteps = kChunkWaves * kWave * kK;
// Steps per chunk, and chunks per row: every chunk but the last in scan
// order spans `span` steps, the last the rest of the row (1 to span steps).
// Windows widened to K-aligned starts (kVecSkew below) leave room in the tile
// for the skew (< K <= 4 steps) and give the last chunk 4 to span + 3 steps,
// room for its hand-off word (chunk_slot).
constexpr uint32_t chunk_span(bool skew) { return skew ? kChunkSteps - 8 : kChunkSteps; }
constexpr uint32_t chunk_count(uint32_t T, bool skew) {
    return (T - (skew ? 4u : 1u)) / chunk_span(skew) + 1;
}

enum Estimator : int {
    kGae = 0,
    kTdLambda = 1,
    kDiscounted = 2,
    kVtrace = 3,
    kRetrace = 4,
    kAffineBackward = 5,  // caller-supplied (alpha, beta), backward in time
};

enum ForwardKind : int {
    kForwardFlags = 0,   // alpha = x, beta = decay except at episode starts
    kForwardAffine = 1,  // caller-supplied (alpha, beta), forward in time
};

enum Mode : int { kFull = 0, kChunkAggregate = 1, kChunkApply = 2 };

struct Geometry {
    int64_t num_envs;
    uint32_t T;
    uint32_t rows_per_group;  // full mode: whole rows owned by one workgroup iteration
    uint32_t num_groups;
    uint32_t chunks_per_row;  // chunk modes: chunk_count(T, skew)
    // kVecSkew: phase of the per-step inputs (the element index mod K at which
    // their K-aligned blocks start, the same for every input), phase of out0,
    // and whether the outputs' phase differs from the inputs' (then they are
    // written element by element).  0, 0, 0 on the other paths.
    uint32_t phase, out0_phase, scatter;
};

// Real-valued arrays are stored as S (float, __bf16 or _Float16: the kernels'
// storage-type parameter) and computed on in fp32; the pointers below are
// untyped and take the kernel's S.
struct BackwardParams {
    const void *rewards;  // alpha for kAffineBackward
    const void *values;   // V(s_t); Q(s_t, a_t) for Retrace; beta for kAffineBackward
    const void *expected_q;
    const void *behaviour_logp;
    const void *target_logp;
    const uint8_t *terminated;
    const uint8_t *truncated;
    const void *trunc_values;
    const void *bootstrap;  // carry A_T for kAffineBackward
    void *out0;             // advantages / returns / vs / q_ret / A
    void *out1;             // GAE returns or V-Trace pg advantages; may be null
    // with STATS: (sum, sum of squares) of out0 per workgroup, after the
    // workspace's ticket counter (kTicketBytes); the last workgroup writes
    // {mean, sample std} to stats
    double *stats_partials;
    double *stats;
    int64_t stats_count;  // N * T
    float gamma, lambda, rho_bar, c_bar;
    Geometry geo;
};

struct ForwardParams {
    const void *x;         // alpha for kForwardAffine
    const uint8_t *flags;  // kForwardFlags
    const void *beta;      // kForwardAffine
    const void *carry;     // kForwardAffine: A_{-1} per row, may be null
    void *out;
    float decay;     // gamma*lambda for traces (rounded to fp32), 1 for prefix sums
    double decay64;  // the same, exact (fp64 product of the fp32 factors): fp64 scans
    Geometry geo;
};

// Storage types of real-valued arrays.
enum Storage : int { kStoreF32 = 0, kStoreBF16 = 1, kStoreF16 = 2 };

// Launch configuration chosen on the host.
struct LaunchShape {
    int waves;        // NW: 1, 2, 4 or 8 waves per workgroup
    bool wave_local;  // rows end at wave boundaries (T divides 64*K)
    bool vec;         // K-wide accesses: per-step inputs at one phase
    bool skew;        // ... other than T % K == 0 with every per-step array
                      // K-aligned: windows widened to K-aligned starts
                      // (kVecSkew below; 8 waves, never wave-local)
    uint32_t quantum;  // skewed path: rows per window a multiple of this (skew_rows)
    uint32_t phase, out0_phase;  // skewed path: as in Geometry
    bool scatter;                // skewed path: as in Geometry
    bool chunked;     // few long rows: the three chunk-mode launches
    bool f64;         // fp64 scan (ScanOf): rows span waves with beta near 1
};

// ---------------------------------------------------------------- memory access
// `p` points at the workgroup's first element; `off` is the lane's first step
// relative to it and `L` the number of valid steps.  The memory path VEC:
//   kScalarIO   one access per element (any alignment, any T);
//   kVecRows    K-wide accesses; T % K == 0 and K-element alignment of p + off,
//               so a lane's K steps are wholly valid or wholly past the end,
//               and lie in one row;
//   kVecSkew    K-wide reads for any T with every per-step input at one
//               phase (its K-aligned blocks start at the same element index
//               mod K): the window is widened at its start to the block
//               boundary before it (by its skew, < K steps, read but never
//               written), so a lane's steps may cross a row end, and its
//               first and last K steps may be partly valid (`lo` .. `L`):
//               those are written element by element, and so is every step
//               when the outputs are at another phase.
enum IoPath : int { kScalarIO = 0, kVecRows = 1, kVecSkew = 2 };
//
// Stored values S widen to the scan type E on load (bf16 and fp16 widen
// exactly to fp32) and narrow on store (to nearest even: v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 on gfx950).

template <typename E, typename S>
__device__ __forceinline__ E widen(S x) {
    return static_cast<E>(x);
}
template <typename S, typename E>
__device__ __forceinline__ S narrow(E x) {
    return static_cast<S>(x);
}

template <typename E, int N>
struct VecOf {
    typedef E type __attribute__((ext_vector_type(N)));
};

// Unsigned integer holding K flag bytes.
template <int N>
struct FlagWord;
template <>
struct FlagWord<4> {
    typedef uint32_t type;
};

// LAST: this is the last read of the data, so the vector loads carry the
// non-temporal hint (measured 3-5% faster for streams read once; the chunk
// modes' aggregate pass, whose inputs the apply pass reads again, keeps
// them cacheable).
//
// kVecSkew reads whole aligned K-element blocks: a lane whose first step is
// below L reads its K steps even where later ones lie past L, up to K - 1
// elements past the window and, for the array's last window, past the
// array's end (and, for inputs at a nonzero phase, up to K - 1 elements
// before the array's start).  Such a block holds an element of the array
// and is aligned, so it never crosses a page boundary and cannot fault; the
// steps outside the window are invalid and their values are never used (the
// scan takes them as identity by selection, not arithmetic).  Writes stay
// inside [lo, L).
template <int VEC, bool LAST = true, typename E, typename S>
__device__ __forceinline__ void load_steps(E (&x)[kK], const S *__restrict__ p, uint32_t off,
                                           uint32_t L) {
    static_assert(sizeof(E) == 4 && (sizeof(S) == 4 || sizeof(S) == 2), "32-bit scan values");
    // Element-typed vector: its lanes are read by value (no bit cast of a
    // vector element, which this compiler lowers as a read of element 0).
    typedef typename VecOf<S, kK>::type vec;
    if constexpr (VEC != kScalarIO) {
        vec q = {};
        if (off < L) {
            const vec *src = reinterpret_cast<const vec *>(p + off);
            q = LAST ? __builtin_nontemporal_load(src) : *src;
        }
#pragma unroll
        for (int i = 0; i < kK; ++i) x[i] = widen<E>(q[i]);
    } else {
#pragma unroll
        for (int i = 0; i < kK; ++i) x[i] = (off + i < L) ? widen<E>(p[off + i]) : E(0);
    }
}

template <int VEC, bool LAST = true>
__device__ __forceinline__ void load_flags(bool (&f)[kK], const uint8_t *__restrict__ p,
                                           uint32_t off, uint32_t L) {
    if constexpr (VEC != kScalarIO) {
        typedef typename FlagWord<kK>::type word;
        uint32_t q = 0;
        if (off < L) {
            const word *src = reinterpret_cast<const word *>(p + off);
            q = LAST ? __builtin_nontemporal_load(src) : *src;
        }
#pragma unroll
        for (int i = 0; i < kK; ++i) f[i] = ((q >> (8 * i)) & 0xffu) != 0;
    } else {
#pragma unroll
        for (int i = 0; i < kK; ++i) f[i] = (off + i < L) ? (p[off + i] != 0) : false;
    }
}

// kVecSkew: a lane whose K steps straddle the window's start (lo) or end,
// and every lane when `scatter` (outputs at another phase than the inputs),
// writes its steps in [lo, L) element by element.
template <int VEC, typename S, typename E>
__device__ __forceinline__ void store_steps(S *__restrict__ p, const E (&x)[kK], uint32_t off,
                                            uint32_t L, uint32_t lo = 0, bool scatter = false) {
    typedef typename VecOf<S, kK>::type vec;
    if constexpr (VEC != kScalarIO) {
        if (VEC == kVecSkew && off < L && (scatter || off < lo || off + kK > L)) {
#pragma unroll
            for (int i = 0; i < kK; ++i)
                if (off + i >= lo && off + i < L) p[off + i] = narrow<S>(x[i]);
        } else if (off < L) {
            vec q;
#pragma unroll
            for (int i = 0; i < kK; ++i) q[i] = narrow<S>(x[i]);
            __builtin_nontemporal_store(q, reinterpret_cast<vec *>(p + off));
        }
    } else {
#pragma unroll
        for (int i = 0; i < kK; ++i)
            if (off + i < L) p[off + i] = narrow<S>(x[i]);
    }
}

// Chunk modes hand values between launches through the chunk's first output
// elements, as raw 32-bit words whatever S is: for 2-byte S from the chunk's
// first element at a 4-byte aligned address (the output's phase, out_phase,
// is its start's element index mod K).  Every chunk but the last in scan
// order holds its map, two scan values (four words for fp64 scans: it spans
// thousands of steps); the last receives only its carry, one word (its 1 or
// 2 elements lie in the chunk: with 2-byte S and an odd start it spans at
// least 4 steps).
template <typename E, typename S>
__device__ __forceinline__ E *chunk_slot(void *out, int64_t base, uint32_t out_phase) {
    if constexpr (sizeof(S) == 2) base += (base + out_phase) & 1;
    return reinterpret_cast<E *>(static_cast<S *>(out) + base);
}

// Hand-off words pass between launches: one workgroup writes them with
// plain stores, which the end of its launch makes visible to the whole
// device, and another reads them in a later launch, on any XCD.  The apply
// pass's carry, one workgroup-uniform word, is read with an agent-scope
// atomic load, so that it never comes through the scalar cache, where a
// plain load of a uniform address would go.  The carries pass reads each
// lane's own map with plain loads, which merge into one vector load.  On one
// row of 2^20 steps, per-word atomics measured slower: the map stores by
// 0.3-0.5 us per aggregate launch, the map loads by 2 us per carries launch.
__device__ __forceinline__ uint32_t load_word(const uint32_t *w) {
    return __hip_atomic_load(const_cast<uint32_t *>(w), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// A chunk's map (a, b) as scan values C, each as raw 32-bit words (two for
// fp64), from word 0 of the chunk's slot; the carry comes back in word 0 as
// one value of the kernel's value type.
template <typename C>
__device__ __forceinline__ void put_words(uint32_t *w, C x) {
    if constexpr (sizeof(C) == 4) {
        w[0] = __builtin_bit_cast(uint32_t, x);
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        w[0] = (uint32_t)u;
        w[1] = (uint32_t)(u >> 32);
    }
}
template <typename C, bool UNIFORM>
__device__ __forceinline__ C get_words(const uint32_t *w) {
    if constexpr (!UNIFORM) {  // per-lane addresses: plain (vector) loads
        if constexpr (sizeof(C) == 4) return __builtin_bit_cast(C, w[0]);
        else return __builtin_bit_cast(C, ((uint64_t)w[1] << 32) | w[0]);
    } else if constexpr (sizeof(C) == 4) {
        return __builtin_bit_cast(C, load_word(w));
    } else {
        return __builtin_bit_cast(C, ((uint64_t)load_word(w + 1) << 32) | load_word(w));
    }
}

// Chunk apply mode reads its carry from the chunk's first slot: an output
// element that one of the workgroup's waves overwrites later.  Each wave
// takes the value into hand here, before the barrier in block_carry_in (a
// chunk is one tile of kChunkWaves waves, so that barrier always runs and
// precedes every store): no wave can store over the slot while another
// wave's read of it is still in flight.  The slot load was issued ahead of
// the tile's loads, which return in order, so this wait costs nothing.
template <typename V>
__device__ __forceinline__ void hold_chunk_carry(V &carry) {
    asm volatile("" : "+v"(carry));
}

// The steps one workgroup iteration covers.
struct Window {
    int64_t row0;       // first row
    int64_t base;       // flat index of the window's first step
    uint32_t L;         // steps in the window
    uint32_t t0;        // row-local index of the first step (0 in full mode)
    uint32_t row_rest;  // steps from the window start to the end of its row
    uint32_t chunk;     // chunk index in scan order (chunk modes)
    uint32_t skew;      // (base + phase) % K: steps from the block boundary to base
};

// Chunk j (of m) of a row in scan order, `span` steps each but the last:
// backward scans count chunks from the row end, so the earliest chunk takes
// the rest of the row; forward scans count from the start.
__host__ __device__ inline void chunk_bounds(uint32_t T, uint32_t j, uint32_t m, bool backward,
                                             uint32_t span, uint32_t &lo, uint32_t &hi) {
    if (backward) {
        hi = T - j * span;
        lo = j + 1 < m ? hi - span : 0u;
    } else {
        lo = j * span;
        hi = j + 1 < m ? lo + span : T;
    }
}

template <int MODE, bool BACKWARD, int VEC = kVecRows>
__device__ __forceinline__ Window window_of(const Geometry &geo, uint32_t g) {
    Window w;
    if constexpr (MODE == kFull) {
        w.row0 = (int64_t)g * geo.rows_per_group;
        const int64_t rows_left = geo.num_envs - w.row0;
        const uint32_t rows =
            rows_left < (int64_t)geo.rows_per_group ? (uint32_t)rows_left : geo.rows_per_group;
        w.L = rows * geo.T;
        w.base = w.row0 * (int64_t)geo.T;
        w.t0 = 0;
        w.row_rest = w.L;
        w.chunk = 0;
    } else {
        const uint32_t n = g / geo.chunks_per_row;
        const uint32_t j = g - n * geo.chunks_per_row;
        uint32_t lo, hi;
        chunk_bounds(geo.T, j, geo.chunks_per_row, BACKWARD, chunk_span(VEC == kVecSkew), lo,
                     hi);
        w.row0 = n;
        w.base = (int64_t)n * geo.T + lo;
        w.L = hi - lo;
        w.t0 = lo;
        w.row_rest = geo.T - lo;
        w.chunk = j;
    }
    w.skew = ((uint32_t)w.base + geo.phase) & (kK - 1);
    return w;
}

// Row-local step index t and row offset (relative to row0) of each of the
// lane's K steps; `off` counts from the window start, widened by the skew on
// the kVecSkew path.  kVecRows: T % K == 0 and off % K == 0, so the K steps
// lie in one row and only the last can end it (only the first can start it).
// kVecSkew: the steps before the window (in the lane chunk at off = 0) are
// invalid and take the position of the window's first step.
// WAVE_LOCAL: T divides the 256-step wave span, so it is a power of two.
template <int MODE, int VEC = kScalarIO, bool WAVE_LOCAL = false>
__device__ __forceinline__ void step_positions(const Window &w, uint32_t off, uint32_t T,
                                               uint32_t (&t)[kK], uint32_t (&row)[kK]) {
    const uint32_t sk = VEC == kVecSkew ? w.skew : 0u;
    if constexpr (MODE == kFull) {
        const uint32_t head = off < sk ? sk - off : 0u;  // steps before the window
        const uint32_t u = off + head - sk;              // the first valid step
        uint32_t r, s;
        if constexpr (WAVE_LOCAL) {
            r = u >> __builtin_ctz(T);
            s = u & (T - 1);
        } else {
            r = u / T;
            s = u - r * T;
        }
        if constexpr (VEC == kVecRows) {
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                t[i] = s + i;
                row[i] = r;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                t[i] = s;
                row[i] = r;
                if ((uint32_t)i >= head && ++s == T) {
                    s = 0;
                    ++r;
                }
            }
        }
    } else {
        // steps before the window wrap around; they are invalid
#pragma unroll
        for (int i = 0; i < kK; ++i) {
            t[i] = w.t0 + off + i - sk;
            row[i] = 0;
        }
    }
}

// NaN-propagating clip and minimum (fminf / fmaxf would return the other
// operand and turn a NaN log-probability into a plausible ratio): a NaN
// input yields a NaN coefficient, kept inside its episode segment.
__device__ __forceinline__ float clip_to(float x, float lo, float hi) {
    x = x > hi ? hi : x;
    return x < lo ? lo : x;
}
__device__ __forceinline__ float min_keep_nan(float bound, float x) { return bound < x ? bound : x; }

// exp(x) for the clipped log-ratio, |x| <= RLCA_LOG_RATIO_CLIP, or NaN: the
// exponent x * log2(e) is split into its fp32 rounding hi and the rest lo
// (Cody and Waite's argument splitting, the product's rounding error
// recovered with one fused multiply-add), 2^hi comes from the hardware
// exp2 (v_exp_f32, exact at 0, no range reduction needed while
// |hi| < 126) and lo enters as 2^hi * (1 + lo * ln 2).  Measured on MI355X
// over every 97th fp32 value of [-5, 5]: at most 1.21 ulp from the exact
// exponential (the general expf: 0.82 ulp), in half its instructions.
static_assert(RLCA_LOG_RATIO_CLIP <= 80.0f, "the split exp assumes |x * log2(e)| < 126");
__device__ __forceinline__ float exp_clipped(float x) {
    constexpr float kLog2e = 1.44269502f;     // fp32 rounding of log2(e)
    constexpr float kLog2eLo = 1.925963e-8f;  // log2(e) - kLog2e
    constexpr float kLn2 = 0.693147181f;
    const float hi = x * kLog2e;
    float lo = __builtin_fmaf(x, kLog2e, -hi);
    lo = __builtin_fmaf(x, kLog2eLo, lo);
    const float p = __builtin_amdgcn_exp2f(hi);
    return __builtin_fmaf(p, lo * kLn2, p);
}

__device__ __forceinline__ float importance_ratio(float target_logp, float behaviour_logp) {
    return exp_clipped(
        clip_to(target_logp - behaviour_logp, -RLCA_LOG_RATIO_CLIP, RLCA_LOG_RATIO_CLIP));
}

// fp64 DPP step: x plus the value of the lane CTRL selects (0 where there
// is none), moved as two 32-bit halves.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL,
                                                              ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                              ROW_MASK, 0xf, false);
    return x + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double read_lane_f64(double x, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes of a wave, in a fixed order (the prefix pattern of
// wave_inclusive_scan; lane 63 ends with the total), returned to every lane.
__device__ __forceinline__ double wave_sum_f64(double x) {
    x = dpp_add_f64<0x111, 0xf>(x);  // row_shr:1
    x = dpp_add_f64<0x112, 0xf>(x);  // row_shr:2
    x = dpp_add_f64<0x114, 0xf>(x);  // row_shr:4
    x = dpp_add_f64<0x118, 0xf>(x);  // row_shr:8
    x = dpp_add_f64<0x142, 0xa>(x);  // row_bcast:15
    x = dpp_add_f64<0x143, 0xc>(x);  // row_bcast:31
    return read_lane_f64(x, kWave - 1);
}

// Sum of (a, b) over the workgroup, left in every lane: each wave's sum
// (wave_sum_f64), then the NW wave sums in order through LDS.  Every wave of
// the workgroup must call it.
template <int NW>
__device__ __forceinline__ void workgroup_sum2(double &a, double &b) {
    a = wave_sum_f64(a);
    b = wave_sum_f64(b);
    if constexpr (NW > 1) {
        __shared__ double lds[2 * NW];
        const int w = threadIdx.x / kWave;
        if ((threadIdx.x & (kWave - 1)) == 0) {
            lds[2 * w] = a;
            lds[2 * w + 1] = b;
        }
        __syncthreads();
        a = 0.0;
        b = 0.0;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            a += lds[2 * j];
            b += lds[2 * j + 1];
        }
    }
}

// ------------------------------------------------- last-workgroup reductions
// The fused consumers reduce over the whole launch in one launch: each
// workgroup publishes one partial (a pair of doubles, STRIDE 2, or one
// double, STRIDE 1) in a workspace that starts with ticket counters, and
// the workgroup that takes the last ticket adds all the partials in a fixed
// order (the same result whichever workgroup finishes last) and restores
// the counters to zero.  No workgroup waits for another.
//
// Visibility without a cache write-back: the partials are written and read
// with agent-scope atomic stores and loads, which the hardware performs
// coherently across the chip's XCDs by themselves (an agent-scope release
// fence would instead write back the XCD's whole L2, once per workgroup).
// A workgroup takes its ticket only after its stores have completed
// (s_waitcnt), and a ticket's holder issues later operations only after the
// ticket has returned, so the last ticket's holder sees every partial.
//
// Two levels of tickets: agent-scope atomics on one address serialize at
// about 12 ns each (measured: 512 workgroups add 5 us to a launch, 4096 add
// 44 us), while atomics on addresses 128 bytes apart proceed in parallel.
// Workgroup g takes a ticket on slot g % kTicketSlots; the last workgroup
// of each slot takes one on the top counter, and the last of those reduces.
constexpr int kTicketSlots = 32;
constexpr int kTicketStride = 32;  // words between counters: 128 bytes
constexpr size_t kTicketBytes = (size_t)(kTicketSlots + 1) * kTicketStride * 4;

__device__ __forceinline__ uint32_t *ticket_counters(double *partials) {
    return reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(partials) - kTicketBytes);
}

__device__ __forceinline__ void store_coherent(double *p, double x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_coherent(const double *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t take_ticket(uint32_t *counter) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the compiler's order too
    __builtin_amdgcn_s_waitcnt(0);             // earlier stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kFinishBatch = 16;  // independent loads in flight per lane

// Sum of `count` (a, b) partials (b only with STRIDE 2) in fixed order:
// strided over the NT threads in batches of independent loads, then across
// the workgroup.
template <int NT, int STRIDE>
__device__ __forceinline__ void sum_partials(const double *partials, uint32_t count, double &a,
                                             double &b) {
    a = 0.0;
    b = 0.0;
    for (uint32_t i0 = threadIdx.x; i0 < count; i0 += NT * kFinishBatch) {
        double va[kFinishBatch], vb[kFinishBatch];
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) {
            const uint32_t i = i0 + k * NT;
            va[k] = i < count ? load_coherent(partials + (size_t)i * STRIDE) : 0.0;
            vb[k] = i < count && STRIDE == 2 ? load_coherent(partials + (size_t)i * 2 + 1) : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) {
            a += va[k];
            b += vb[k];
        }
    }
    workgroup_sum2<NT / kWave>(a, b);
}

// Publish this workgroup's partial (a, b) -- the values thread 0 holds --
// and take tickets; the last workgroup sums every partial and calls
// done(a, b) on thread 0, then clears the top counter (each slot's last
// workgroup clears its slot's).  Every thread of the workgroup must call
// it; the barrier also separates this workgroup's own reduction from the
// final one (they share LDS).
template <int NT, int STRIDE, typename Done>
__device__ __forceinline__ void finish_in_last_workgroup(double *partials, double a, double b,
                                                         Done done) {
    __shared__ uint32_t last;
    uint32_t *counters = ticket_counters(partials);
    if (threadIdx.x == 0) {
        const uint32_t g = blockIdx.x, groups = gridDim.x;
        store_coherent(partials + (size_t)g * STRIDE, a);
        if constexpr (STRIDE == 2) store_coherent(partials + (size_t)g * 2 + 1, b);
        const uint32_t slot = g % kTicketSlots;
        const uint32_t in_slot = (groups - 1 - slot) / kTicketSlots + 1;  // workgroups of the slot
        uint32_t *slot_counter = counters + slot * kTicketStride;
        bool is_last = false;
        if (take_ticket(slot_counter) + 1 == in_slot) {
            __hip_atomic_store(slot_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t slots = groups < (uint32_t)kTicketSlots ? groups : kTicketSlots;
            is_last = take_ticket(counters + kTicketSlots * kTicketStride) + 1 == slots;
        }
        last = is_last ? 1u : 0u;  // the loads below wait for the tickets
    }
    __syncthreads();
    if (last == 0u) return;
    double sa, sb;
    sum_partials<NT, STRIDE>(partials, gridDim.x, sa, sb);
    if (threadIdx.x == 0) {
        done(sa, sb);
        __hip_atomic_store(counters + kTicketSlots * kTicketStride, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------- leading kernel arguments
// The geometry and the first five input arrays are passed as separate scalar
// kernel arguments ahead of the parameter block: gfx950 preloads leading
// kernel arguments into SGPRs before a wave starts (13 dwords here), so each
// wave can issue its first loads without a scalar-memory round trip for its
// arguments.  Which five arrays lead depends on the estimator.
#define LEAD_ARGS                                                                         \
    const void *lead0, const void *lead1, const void *lead2, const void *lead3,            \
        const void *lead4, uint32_t lead_T, uint32_t lead_rows_per_group, uint32_t lead_num_envs
#define LEAD_NAMES lead0, lead1, lead2, lead3, lead4, lead_T, lead_rows_per_group, lead_num_envs

struct Lead {
    const void *ptr[5];
    uint32_t T, rows_per_group, num_envs;
};

// Host side: the estimator's five leading arrays, in argument order.
template <int EST>
inline void lead_from(const BackwardParams &p, Lead &l) {
    if constexpr (EST == kGae || EST == kTdLambda) {
        l.ptr[0] = p.rewards, l.ptr[1] = p.values, l.ptr[2] = p.terminated;
        l.ptr[3] = p.truncated, l.ptr[4] = p.trunc_values;
    } else if constexpr (EST == kDiscounted) {
        l.ptr[0] = p.rewards, l.ptr[1] = p.terminated, l.ptr[2] = p.truncated;
        l.ptr[3] = p.trunc_values, l.ptr[4] = p.bootstrap;
    } else if constexpr (EST == kVtrace) {
        l.ptr[0] = p.rewards, l.ptr[1] = p.values, l.ptr[2] = p.behaviour_logp;
        l.ptr[3] = p.target_logp, l.ptr[4] = p.terminated;
    } else if constexpr (EST == kRetrace) {
        l.ptr[0] = p.rewards, l.ptr[1] = p.values, l.ptr[2] = p.expected_q;
        l.ptr[3] = p.behaviour_logp, l.ptr[4] = p.target_logp;
    } else {
        l.ptr[0] = p.rewards, l.ptr[1] = p.values, l.ptr[2] = p.bootstrap;
        l.ptr[3] = p.out0, l.ptr[4] = nullptr;
    }
}

inline void lead_from(const ForwardParams &p, Lead &l) {
    l.ptr[0] = p.x, l.ptr[1] = p.flags, l.ptr[2] = p.out, l.ptr[3] = p.beta, l.ptr[4] = p.carry;
}

// Device side: the same arrays and the geometry, taken from the preloaded
// arguments.
template <int EST>
__device__ __forceinline__ void adopt_lead(BackwardParams &p, LEAD_ARGS) {
    typedef const void *F;
    typedef const uint8_t *U;
    if constexpr (EST == kGae || EST == kTdLambda) {
        p.rewards = F(lead0), p.values = F(lead1), p.terminated = U(lead2);
        p.truncated = U(lead3), p.trunc_values = F(lead4);
    } else if constexpr (EST == kDiscounted) {
        p.rewards = F(lead0), p.terminated = U(lead1), p.truncated = U(lead2);
        p.trunc_values = F(lead3), p.bootstrap = F(lead4);
    } else if constexpr (EST == kVtrace) {
        p.rewards = F(lead0), p.values = F(lead1), p.behaviour_logp = F(lead2);
        p.target_logp = F(lead3), p.terminated = U(lead4);
    } else if constexpr (EST == kRetrace) {
        p.rewards = F(lead0), p.values = F(lead1), p.expected_q = F(lead2);
        p.behaviour_logp = F(lead3), p.target_logp = F(lead4);
    } else {
        p.rewards = F(lead0), p.values = F(lead1), p.bootstrap = F(lead2);
        p.out0 = const_cast<void *>(lead3);
        (void)lead4;
    }
    p.geo.T = lead_T;
    p.geo.rows_per_group = lead_rows_per_group;
    p.geo.num_envs = lead_num_envs;
}

__device__ __forceinline__ void adopt_lead(ForwardParams &p, LEAD_ARGS) {
    p.x = lead0;
    p.flags = static_cast<const uint8_t *>(lead1);
    p.out = const_cast<void *>(lead2);
    p.beta = lead3;
    p.carry = lead4;
    p.geo.T = lead_T;
    p.geo.rows_per_group = lead_rows_per_group;
    p.geo.num_envs = lead_num_envs;
}

// ------------------------------------------------------------- backward kernel
// A_t = alpha_t + beta_t * A_{t+1}.  Lanes take chunks in reverse time order, so
// the lane-order scan of scan_core.hpp runs from the end of the tile backwards.
// Workgroup g runs group g; with STATS the grid is capped (kStatsMaxGrid,
// one partial sum per workgroup) and groups g, g + g_stride, ... run
// through one workgroup.
// STATS: also sum out0 and its square over the workgroup's valid steps (in
// fp64) and store the pair in stats_partials[2 * blockIdx.x ...].
// F64: the scan runs in fp64 (ScanOf; the host's choice, in the chunk modes
// too); outputs are rounded to fp32 once.
template <int EST, bool TRUNC, int VEC, int NW, bool WAVE_LOCAL, int MODE, typename S,
          bool STATS = false, bool F64 = false>
__device__ __forceinline__ void backward_body(BackwardParams &p, uint32_t g, uint32_t g_stride) {
    static_assert(!STATS || MODE != kChunkAggregate, "statistics come from the outputs");
    static_assert(MODE == kFull || (NW == kChunkWaves && !WAVE_LOCAL),
                  "a chunk is one tile of kChunkWaves waves");
    typedef typename ScanOf<float, F64>::type SV;
    // the importance-weighted bodies compose with the legacy multiply
    // (scan_core.hpp): their beta is never infinite, and they are the ones
    // whose vector issue shows in their time (V-Trace, Retrace)
    constexpr bool kLegacy = (EST == kVtrace || EST == kRetrace) && !F64;
    typedef const S *__restrict__ In;
    const In rewards = static_cast<In>(p.rewards), values = static_cast<In>(p.values);
    const In expected_q = static_cast<In>(p.expected_q);
    const In behaviour_logp = static_cast<In>(p.behaviour_logp);
    const In target_logp = static_cast<In>(p.target_logp);
    const In trunc_values = static_cast<In>(p.trunc_values);
    const In bootstrap = static_cast<In>(p.bootstrap);
    S *__restrict__ out0 = static_cast<S *>(p.out0);
    S *__restrict__ out1 = static_cast<S *>(p.out1);
    double sum = 0.0, sum_sq = 0.0;  // STATS
    constexpr uint32_t kTile = NW * kWave * kK;
    constexpr bool kFlags = EST != kAffineBackward;
    __shared__ SV lds_a[2 * NW], lds_b[2 * NW];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = NW == 1 ? 0 : threadIdx.x / kWave;  // one-wave tiles: each wave alone
    const uint32_t chunk = (NW - 1 - w) * kWave + (kWave - 1 - lane);
    const uint32_t T = p.geo.T;
    const float gamma = p.gamma;
    int parity = 0;

    // The grid never exceeds the group count, so the first group always
    // exists; testing only at the bottom lets every kernel-argument load go
    // out together instead of after a first round trip for the bound.  Only
    // the statistics launches loop: a loop keeps the array pointers live
    // across iterations, which at eight waves per SIMD spilled the heavier
    // bodies' SGPRs (Retrace 2048 x 1024: 3% slower).
    do {
        const Window win = window_of<MODE, true, VEC>(p.geo, g);
        // Memory base and extent of the window: on the kVecSkew path widened
        // to the K-aligned step at or before its start, steps [sk, L) valid.
        const uint32_t sk = VEC == kVecSkew ? win.skew : 0u;
        const int64_t row0 = win.row0, base = win.base - sk;
        const uint32_t L = win.L + sk;
        const uint32_t ntiles = MODE == kFull ? (L + kTile - 1) / kTile : 1u;
        // A just after the current tile: 0 at a row end (edges live in alpha),
        // or the carry the chunk-carry pass left in the chunk's first slot.
        SV carry = SV(0);
        if constexpr (MODE == kChunkApply)  // issued ahead of the tile's loads
            carry = SV(get_words<float, true>(chunk_slot<uint32_t, S>(p.out0, win.base,
                                                                 p.geo.out0_phase)));

        for (uint32_t it = 0; it < ntiles; ++it) {
            const uint32_t off = (ntiles - 1 - it) * kTile + chunk * kK;

            // ---- 1. loads (each input element once)
            float r[kK], v[kK], eq[kK], mu[kK], pi[kK], tv[kK];
            bool term[kK], trunc[kK];
            constexpr bool kLast = MODE != kChunkAggregate;
            load_steps<VEC, kLast>(r, rewards + base, off, L);
            if constexpr (EST != kDiscounted) load_steps<VEC, kLast>(v, values + base, off, L);
            if constexpr (EST == kRetrace) load_steps<VEC, kLast>(eq, expected_q + base, off, L);
            if constexpr (EST == kVtrace || EST == kRetrace) {
                load_steps<VEC, kLast>(mu, behaviour_logp + base, off, L);
                load_steps<VEC, kLast>(pi, target_logp + base, off, L);
            }
            if constexpr (kFlags) load_flags<VEC, kLast>(term, p.terminated + base, off, L);
            if constexpr (TRUNC) {
                load_flags<VEC, kLast>(trunc, p.truncated + base, off, L);
                load_steps<VEC, kLast>(tv, trunc_values + base, off, L);
            }
            // Loads whose addresses depend only on positions go out with the
            // main batch: the bootstrap (carry) of rows ending in this chunk,
            // and the first step of the next chunk in time wherever lane - 1
            // does not hold it: lane 0 (its neighbour sits in another wave or
            // tile) and the lane whose chunk ends the window while its row
            // goes on (a partial chunk in the chunk modes).
            uint32_t t[kK], row[kK];
            step_positions<MODE, VEC, WAVE_LOCAL>(win, off, T, t, row);
            bool valid[kK], edge[kK];
            float boot[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                valid[i] = off + i >= sk && off + i < L;
                // with whole-row lane chunks only the lane's last step can end a row
                edge[i] = (VEC != kVecRows || i == kK - 1) && t[i] == T - 1;
                boot[i] = 0.f;
                if (valid[i] && edge[i] && bootstrap != nullptr)
                    boot[i] = widen<float>(bootstrap[row0 + row[i]]);
            }
            float v_first = 0.f, mu_first = 0.f, pi_first = 0.f, eq_first = 0.f;
            // With WAVE_LOCAL every wave (and so lane 0's chunk and the
            // window) ends at a row end: the halo is never used.
            const bool halo_from_memory =
                !WAVE_LOCAL && (lane == 0 || off + kK >= L) && off + kK < win.row_rest + sk;
            if (halo_from_memory) {
                const int64_t jh = base + off + kK;
                if constexpr (EST == kGae || EST == kTdLambda || EST == kVtrace)
                    v_first = widen<float>(values[jh]);
                if constexpr (EST == kRetrace) {
                    mu_first = widen<float>(behaviour_logp[jh]);
                    pi_first = widen<float>(target_logp[jh]);
                    eq_first = widen<float>(expected_q[jh]);
                }
            }

            // ---- 2. boundary resolution
            bool cont[kK];
            float succ[kK];  // successor value where the chain stops
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                if constexpr (kFlags) {
                    const bool tr = TRUNC && trunc[i] && !term[i];
                    cont[i] = valid[i] && !term[i] && !tr && !edge[i];
                    float sv = term[i] ? 0.f : boot[i];
                    if constexpr (TRUNC) {
                        if (tr) sv = tv[i];
                    }
                    succ[i] = sv;
                } else {
                    cont[i] = valid[i] && !edge[i];
                    succ[i] = boot[i];
                }
            }

            // ---- 3. halo: the first step of the next chunk in time, from lane - 1
            float v_next = 0.f, eq_next = 0.f;
            if constexpr (EST == kGae || EST == kTdLambda || EST == kVtrace) {
                v_next = from_lower_lane(v[0], v_first);
                if (halo_from_memory) v_next = v_first;
            }
            // clipped importance ratio min(c_bar, ratio_t); c_t = lambda * m_t
            float m[kK];
            if constexpr (EST == kVtrace || EST == kRetrace) {
#pragma unroll
                for (int i = 0; i < kK; ++i)
                    m[i] = min_keep_nan(p.c_bar, importance_ratio(pi[i], mu[i]));
            }
            float m_next = 0.f;
            if constexpr (EST == kRetrace) {
                const float m_first = min_keep_nan(p.c_bar, importance_ratio(pi_first, mu_first));
                m_next = from_lower_lane(m[0], m_first);
                eq_next = from_lower_lane(eq[0], eq_first);
                if (halo_from_memory) {
                    m_next = m_first;
                    eq_next = eq_first;
                }
            }

            // ---- 4. coefficients in registers.  The fp32 scans form beta_t
            // in fp32 (gamma * (lambda * m_t) for the importance-weighted
            // ones); the fp64 scans form it in fp64 from the same fp32
            // factors, so that a chain with beta near 1 runs on the exact
            // product of the parameters (such chains amplify a one-ulp
            // change of beta by orders of magnitude).
            float alpha[kK], aux[kK];
            SV beta[kK];
            const SV decay_s = SV(gamma) * SV(p.lambda);  // GAE, TD(lambda)
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const bool k = cont[i];
                float a, x = 0.f;
                SV b;
                if constexpr (EST == kGae) {
                    const float vn = i + 1 < kK ? v[i + 1] : v_next;
                    a = r[i] + gamma * (k ? vn : succ[i]) - v[i];
                    b = k ? decay_s : SV(0);
                } else if constexpr (EST == kTdLambda) {
                    const float vn = i + 1 < kK ? v[i + 1] : v_next;
                    a = k ? r[i] + gamma * (1.f - p.lambda) * vn : r[i] + gamma * succ[i];
                    b = k ? decay_s : SV(0);
                } else if constexpr (EST == kDiscounted) {
                    a = k ? r[i] : r[i] + gamma * succ[i];
                    b = k ? SV(gamma) : SV(0);
                } else if constexpr (EST == kVtrace) {
                    const float vn = i + 1 < kK ? v[i + 1] : v_next;
                    const float rho = min_keep_nan(p.rho_bar, importance_ratio(pi[i], mu[i]));
                    a = rho * (r[i] + gamma * (k ? vn : succ[i]) - v[i]);
                    if constexpr (F64)
                        b = k ? decay_s * SV(m[i]) : SV(0);
                    else
                        b = k ? gamma * (p.lambda * m[i]) : 0.f;
                    x = k ? gamma * rho : 0.f;  // pg_t = alpha_t + gamma rho_t A_{t+1}
                } else if constexpr (EST == kRetrace) {
                    // the decay uses the next step's trace coefficient
                    const float mn = i + 1 < kK ? m[i + 1] : m_next;
                    const float en = i + 1 < kK ? eq[i + 1] : eq_next;
                    x = r[i] + gamma * (k ? en : succ[i]);  // Q^ret_t - gamma c_{t+1} A_{t+1}
                    a = x - v[i];
                    if constexpr (F64)
                        b = k ? decay_s * SV(mn) : SV(0);
                    else
                        b = k ? gamma * (p.lambda * mn) : 0.f;
                } else {  // caller's (alpha, beta); the row's carry enters at t = T-1
                    a = k ? r[i] : apply_map(r[i], v[i], succ[i]);
                    b = k ? SV(v[i]) : SV(0);
                }
                alpha[i] = valid[i] ? a : 0.f;
                beta[i] = valid[i] ? b : SV(1);
                aux[i] = x;
            }

            // ---- 5. scan: lane fold (latest step first), then wave / workgroup
            SV fa = SV(0), fb = SV(1);  // identity; step i applied after the later steps
#pragma unroll
            for (int i = kK - 1; i >= 0; --i) {
                SV a_i = alpha[i], b_i = beta[i];
                compose<kLegacy>(a_i, b_i, fa, fb);
                fa = a_i;
                fb = b_i;
            }
            if constexpr (MODE == kChunkAggregate) {
                // hand the chunk's map to the chunk-carry pass (the earliest
                // chunk of a row, last in scan order, has no consumer)
                SV ta, tb;
                block_total<NW>(fa, fb, lds_a, lds_b, parity, ta, tb);
                parity ^= 1;
                if (threadIdx.x == 0 && win.chunk + 1 < p.geo.chunks_per_row) {
                    uint32_t *slot = chunk_slot<uint32_t, S>(p.out0, win.base, p.geo.out0_phase);
                    put_words(slot, ta);
                    put_words(slot + sizeof(SV) / 4, tb);
                }
            } else {
                SV carry_out;
                if constexpr (MODE == kChunkApply) hold_chunk_carry(carry);
                SV A = block_carry_in<NW, WAVE_LOCAL, kLegacy>(fa, fb, carry, lds_a, lds_b,
                                                                parity, carry_out);
                parity ^= 1;
                carry = carry_out;

                // ---- 6. outputs, one store each
                float o0[kK], o1[kK];
#pragma unroll
                for (int i = kK - 1; i >= 0; --i) {
                    const SV An = A;  // A_{t+1}
                    A = apply_map<kLegacy>(SV(alpha[i]), beta[i], An);
                    if constexpr (EST == kGae) {
                        o0[i] = (float)A;
                        o1[i] = (float)(A + SV(v[i]));
                    } else if constexpr (EST == kVtrace) {
                        o0[i] = (float)(SV(v[i]) + A);
                        o1[i] = (float)apply_map<kLegacy>(SV(alpha[i]), SV(aux[i]), An);
                    } else if constexpr (EST == kRetrace) {
                        // Q^ret_t = r_t + gamma E Q_{t+1} + beta_t A_{t+1}, without
                        // the Q_t that alpha_t subtracts and A_t + Q_t would add back
                        o0[i] = (float)apply_map<kLegacy>(SV(aux[i]), beta[i], An);
                        o1[i] = 0.f;
                    } else {
                        o0[i] = (float)A;
                        o1[i] = 0.f;
                    }
                }
                const bool scatter = p.geo.scatter != 0;
                store_steps<VEC>(out0 + base, o0, off, L, sk, scatter);
                if constexpr (EST == kGae || EST == kVtrace) {
                    if (out1 != nullptr) store_steps<VEC>(out1 + base, o1, off, L, sk, scatter);
                }
                if constexpr (STATS) {
#pragma unroll
                    for (int i = 0; i < kK; ++i) {
                        const double x = valid[i] ? (double)o0[i] : 0.0;
                        sum += x;
                        sum_sq += x * x;
                    }
                }
            }
        }
        g += g_stride;
    } while (STATS && g < p.geo.num_groups);
    if constexpr (STATS) {
        workgroup_sum2<NW>(sum, sum_sq);
        // stats = {mean, sample std (divisor M - 1; 0 when M < 2)}
        double *stats = p.stats;
        const int64_t M = p.stats_count;
        finish_in_last_workgroup<NW * kWave, 2>(p.stats_partials, sum, sum_sq,
                                                [=](double s1, double s2) {
            const double mean = s1 / (double)M;
            const double var = M > 1 ? fmax(s2 - s1 * mean, 0.0) / (double)(M - 1) : 0.0;
            store_coherent(stats, mean);  // read by the next launch
            store_coherent(stats + 1, sqrt(var));
        });
    }
}

// 8-wave kernels whose rows span waves ask for eight waves per SIMD: a
// one-shot launch of up to 1024 such workgroups needs every slot, and at the
// seven the compiler picks on its own for these heavier bodies (their SGPR
// count) an eighth of the waves waits for a second round.  The SGPRs over
// the limit spill to VGPR lanes.  Lighter variants reach eight by themselves
// and keep their registers.  The fp64 scans (F64) and the statistics
// epilogue (STATS, fp64 sums) do not ask: at eight waves their VGPRs would
// spill to memory, and a kernel with memory spills needs scratch memory.
#define RLCA_EIGHT_WAVES(NEED) __attribute__((amdgpu_waves_per_eu((NEED) ? 8 : 1)))

template <int EST, bool TRUNC, int VEC, int NW, bool WAVE_LOCAL, int MODE, typename S,
          bool STATS = false, bool F64 = false>
__global__ __launch_bounds__(NW * kWave)
RLCA_EIGHT_WAVES(NW == 8 && !WAVE_LOCAL && VEC != kScalarIO && !F64 && !STATS)
void backward_scan(LEAD_ARGS, BackwardParams p) {
    adopt_lead<EST>(p, LEAD_NAMES);
    backward_body<EST, TRUNC, VEC, NW, WAVE_LOCAL, MODE, S, STATS, F64>(p, blockIdx.x,
                                                                         gridDim.x);
}

// -------------------------------------------------------------- forward kernel
// A_t = alpha_t + beta_t * A_{t-1}.  kForwardFlags: alpha = x, beta = decay and
// beta = 0 where a new episode starts (summary §5: the forward scans cut where
// d_{t-1} = 1); V = float (traces, f32 sums) or uint32_t (int32 sums,
// wrap-around).  kForwardAffine: the caller's (alpha, beta), with the row's
// carry entering at t = 0.
// S: storage type of x, out (and beta, carry for kForwardAffine); uint32_t
// for the integer sums.
// F64 as in backward_body.
template <typename V, int KIND, bool AFTER_DONE, int VEC, int NW, bool WAVE_LOCAL, int MODE,
          typename S, bool F64 = false>
__device__ __forceinline__ void forward_body(ForwardParams &p, uint32_t g, uint32_t g_stride) {
    static_assert(MODE == kFull || (NW == kChunkWaves && !WAVE_LOCAL),
                  "a chunk is one tile of kChunkWaves waves");
    typedef typename ScanOf<V, F64>::type SV;
    constexpr uint32_t kTile = NW * kWave * kK;
    __shared__ SV lds_a[2 * NW], lds_b[2 * NW];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = NW == 1 ? 0 : threadIdx.x / kWave;  // one-wave tiles: each wave alone
    const uint32_t chunk = w * kWave + lane;
    const uint32_t T = p.geo.T;
    const V decay = __builtin_bit_cast(V, __builtin_bit_cast(uint32_t, p.decay));
    SV decay_s;  // fp64 scans take the exact product (see backward_body, step 4)
    if constexpr (__is_same(SV, double))
        decay_s = p.decay64;
    else
        decay_s = decay;
    const S *__restrict__ xs = static_cast<const S *>(p.x);
    const S *__restrict__ betas = static_cast<const S *>(p.beta);
    const S *__restrict__ carries = static_cast<const S *>(p.carry);
    S *__restrict__ out = static_cast<S *>(p.out);
    int parity = 0;

    do {  // the first group always exists (see backward_body)
        const Window win = window_of<MODE, false, VEC>(p.geo, g);
        const uint32_t sk = VEC == kVecSkew ? win.skew : 0u;  // as in backward_body
        const int64_t row0 = win.row0, base = win.base - sk;
        const uint32_t L = win.L + sk;
        const uint32_t ntiles = MODE == kFull ? (L + kTile - 1) / kTile : 1u;
        SV carry = SV(0);
        if constexpr (MODE == kChunkApply)  // issued ahead of the tile's loads
            carry = SV(get_words<V, true>(chunk_slot<uint32_t, S>(p.out, win.base,
                                                             p.geo.out0_phase)));

        for (uint32_t it = 0; it < ntiles; ++it) {
            const uint32_t off = it * kTile + chunk * kK;
            V x[kK];
            float bt[kK];
            bool f[kK];
            constexpr bool kLast = MODE != kChunkAggregate;
            load_steps<VEC, kLast>(x, xs + base, off, L);
            if constexpr (KIND == kForwardFlags) load_flags<VEC, kLast>(f, p.flags + base, off, L);
            if constexpr (KIND == kForwardAffine) load_steps<VEC, kLast>(bt, betas + base, off, L);
            uint32_t t[kK], row[kK];
            step_positions<MODE, VEC, WAVE_LOCAL>(win, off, T, t, row);
            bool start[kK];  // t = 0: with whole-row lane chunks only the lane's first step
            bool valid[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                start[i] = (VEC != kVecRows || i == 0) && t[i] == 0;
                valid[i] = off + i >= sk && off + i < L;
            }
            // flag of the step before the lane's chunk (lane 0; with WAVE_LOCAL
            // every wave starts a row, so it is never needed)
            bool first = false;
            if constexpr (KIND == kForwardFlags && AFTER_DONE && !WAVE_LOCAL) {
                if (lane == 0 && win.t0 + off > sk && off <= L)
                    first = p.flags[base + off - 1] != 0;
            }
            float row_carry[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                row_carry[i] = 0.f;
                if constexpr (KIND == kForwardAffine) {
                    if (valid[i] && start[i] && carries != nullptr)
                        row_carry[i] = widen<float>(carries[row0 + row[i]]);
                }
            }
            bool prev_done = false;
            if constexpr (KIND == kForwardFlags && AFTER_DONE)
                prev_done = from_lower_lane<uint32_t>(f[kK - 1] ? 1u : 0u, first ? 1u : 0u) != 0;
            V alpha[kK];
            SV beta[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                V a;
                SV b;
                if constexpr (KIND == kForwardFlags) {
                    bool reset = start[i];
                    if constexpr (AFTER_DONE) {
                        reset = reset || (i == 0 ? prev_done : f[i - 1]);
                    } else {
                        reset = reset || f[i];
                    }
                    a = x[i];
                    b = reset ? SV(0) : decay_s;
                } else {
                    a = start[i] ? apply_map(x[i], bt[i], row_carry[i]) : x[i];
                    b = start[i] ? SV(0) : SV(bt[i]);
                }
                alpha[i] = valid[i] ? a : V(0);
                beta[i] = valid[i] ? b : SV(1);
            }
            SV fa = SV(0), fb = SV(1);
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                SV a_i = alpha[i], b_i = beta[i];
                compose(a_i, b_i, fa, fb);
                fa = a_i;
                fb = b_i;
            }
            if constexpr (MODE == kChunkAggregate) {
                SV ta, tb;
                block_total<NW>(fa, fb, lds_a, lds_b, parity, ta, tb);
                parity ^= 1;
                if (threadIdx.x == 0 && win.chunk + 1 < p.geo.chunks_per_row) {
                    uint32_t *slot = chunk_slot<uint32_t, S>(p.out, win.base, p.geo.out0_phase);
                    put_words(slot, ta);
                    put_words(slot + sizeof(SV) / 4, tb);
                }
            } else {
                SV carry_out;
                if constexpr (MODE == kChunkApply) hold_chunk_carry(carry);
                SV A = block_carry_in<NW, WAVE_LOCAL>(fa, fb, carry, lds_a, lds_b, parity,
                                                       carry_out);
                parity ^= 1;
                carry = carry_out;
                V o[kK];
#pragma unroll
                for (int i = 0; i < kK; ++i) {
                    A = apply_map(SV(alpha[i]), beta[i], A);
                    o[i] = V(A);
                }
                store_steps<VEC>(out + base, o, off, L, sk, p.geo.scatter != 0);
            }
        }
        g += g_stride;
    } while (false);  // one group per workgroup (no statistics launch here)
}

template <typename V, int KIND, bool AFTER_DONE, int VEC, int NW, bool WAVE_LOCAL, int MODE,
          typename S, bool F64 = false>
__global__ __launch_bounds__(NW * kWave)
RLCA_EIGHT_WAVES(NW == 8 && !WAVE_LOCAL && VEC != kScalarIO && !F64)
void forward_scan(LEAD_ARGS, ForwardParams p) {
    adopt_lead(p, LEAD_NAMES);
    forward_body<V, KIND, AFTER_DONE, VEC, NW, WAVE_LOCAL, MODE, S, F64>(p, blockIdx.x,
                                                                          gridDim.x);
}

// ------------------------------------------------------------ chunk carries
// Chunk modes, middle pass: one workgroup per row scans the row's chunk maps
// (left by the aggregate pass as scan values C in the first words of each
// chunk's slice of `slots`) in scan order and leaves in each chunk's first
// word the value of A entering that chunk, as a value of type R (the
// kernels' value type: fp32 for the float scans, whose maps are fp32 or fp64 as
// their scan is).
// Lane j of a tile holds chunk j; the last chunk in scan order has no map
// (identity) but receives its carry.
template <typename C, typename R, typename S, int NW>
__global__ __launch_bounds__(NW * kWave) void chunk_carries(void *slots, int64_t num_envs,
                                                            uint32_t T, uint32_t chunks_per_row,
                                                            uint32_t span, uint32_t out_phase,
                                                            int backward) {
    __shared__ C lds_a[2 * NW], lds_b[2 * NW];
    constexpr uint32_t kLanes = NW * kWave;
    int parity = 0;
    int64_t n = blockIdx.x;  // the grid never exceeds num_envs
    do {
        const int64_t row = n * (int64_t)T;
        C carry = C(0);
        for (uint32_t j0 = 0; j0 < chunks_per_row; j0 += kLanes) {
            const uint32_t j = j0 + threadIdx.x;
            uint32_t lo = 0, hi = 0;
            if (j < chunks_per_row) chunk_bounds(T, j, chunks_per_row, backward != 0, span, lo, hi);
            uint32_t *slot = chunk_slot<uint32_t, S>(slots, row + lo, out_phase);
            C a = C(0), b = C(1);
            if (j + 1 < chunks_per_row) {  // lane j's own map: plain vector loads
                a = get_words<C, false>(slot);
                b = get_words<C, false>(slot + sizeof(C) / 4);
            }
            C carry_out;
            const C in = block_carry_in<NW, false>(a, b, carry, lds_a, lds_b, parity, carry_out);
            parity ^= 1;
            carry = carry_out;
            if (j < chunks_per_row) put_words(slot, R(in));
        }
        n += gridDim.x;
    } while (n < num_envs);
}

// ------------------------------------------------------------------ launching

// Launch grids: one workgroup per group, up to HIP's largest grid (a call
// that would need more is refused on the host: it could only come from
// terabytes of input).  A grouped launch holds at most kMaxGrid workgroups
// per member (its head words keep workgroup indices in 24 bits).
constexpr uint32_t kOneShotMaxGrid = 0x7fffffffu;
constexpr uint32_t kMaxGrid = 1u << 20;
// Launches that leave one partial sum per workgroup use fewer, longer-lived
// workgroups (2048 are resident on the chip at once), which keeps the final
// reduction to one round of loads.
constexpr uint32_t kStatsMaxGrid = 4096;

inline uint32_t grid_for(int64_t groups, uint32_t cap = kOneShotMaxGrid) {
    return groups < (int64_t)cap ? (uint32_t)groups : cap;
}

constexpr uint32_t gcd_k(uint32_t x) {
    uint32_t d = kK;
    while (x % d != 0) d /= 2;  // K is a power of two
    return d;
}
// Largest skew a window of x steps can have: window g starts at g * x, and
// its skew is (g * x + phase) mod K, which runs over the residues of phase
// mod gcd(x, K).
constexpr uint32_t max_skew(uint32_t x, uint32_t phase) {
    return kK - gcd_k(x) + phase % gcd_k(x);
}
// Rows per window whose starts are all at one skew: K / gcd(T, K).
constexpr uint32_t aligned_rows(uint32_t T) { return kK / gcd_k(T); }

// Rows per window on the skewed path (windows widened to K-aligned starts):
// quantum 1 packs as many rows into one tile as leave room for the largest
// skew their windows can have (a row longer than that takes one window of
// several tiles); quantum q = aligned_rows(T) > 1 gives every window a
// multiple of q rows, so all start at the same skew, and each walks as many
// tiles as it needs (q rows when they exceed one tile).
inline uint32_t skew_rows(uint32_t T, uint32_t tile, uint32_t quantum, uint32_t phase) {
    if (quantum > 1) return T * quantum <= tile ? quantum * (tile / (T * quantum)) : quantum;
    uint32_t r = T <= tile ? tile / T : 1u;
    while (r > 1 && r * T + max_skew(r * T, phase) > tile) --r;
    return r;
}

// Geometry of a launch of shape s: chunked shapes use kChunkWaves-wave
// chunks, the scalar path 4-wave workgroups, the vector paths s.waves.
inline Geometry make_geometry(int64_t num_envs, int64_t T, const LaunchShape &s, uint32_t *grid,
                              uint32_t cap = kOneShotMaxGrid) {
    const int waves = s.chunked ? kChunkWaves : s.vec ? s.waves : 4;
    const uint32_t tile = (uint32_t)waves * kWave * kK;
    Geometry g;
    g.num_envs = num_envs;
    g.T = (uint32_t)T;
    g.phase = s.skew ? s.phase : 0u;
    g.out0_phase = s.skew ? s.out0_phase : 0u;
    g.scatter = s.skew && s.scatter ? 1u : 0u;
    int64_t groups;
    if (s.chunked) {
        g.rows_per_group = 1;
        g.chunks_per_row = chunk_count((uint32_t)T, s.skew);
        groups = num_envs * g.chunks_per_row;
    } else {
        g.rows_per_group = s.skew                ? skew_rows((uint32_t)T, tile, s.quantum, g.phase)
                           : (uint32_t)T <= tile ? tile / (uint32_t)T
                                                 : 1u;
        g.chunks_per_row = 1;
        groups = (num_envs + g.rows_per_group - 1) / g.rows_per_group;
    }
    g.num_groups = (uint32_t)groups;
    *grid = grid_for(groups, cap);
    return g;
}

// Groups of a launch of shape s, before any grid cap: a launch without a
// group loop needs this many workgroups.
inline int64_t launch_groups(int64_t num_envs, int64_t T, const LaunchShape &s) {
    uint32_t grid;
    const Geometry g = make_geometry(num_envs, T, s, &grid);
    return s.chunked ? num_envs * (int64_t)g.chunks_per_row
                     : (num_envs + g.rows_per_group - 1) / g.rows_per_group;
}

template <typename P>
inline rlca_status launch_kernel(const void *kernel, int waves, uint32_t grid, P &params,
                                 Lead &lead, hipStream_t stream) {
    lead.T = params.geo.T;
    lead.rows_per_group = params.geo.rows_per_group;
    lead.num_envs = (uint32_t)params.geo.num_envs;
    void *args[] = {&lead.ptr[0], &lead.ptr[1], &lead.ptr[2],         &lead.ptr[3],
                    &lead.ptr[4], &lead.T,      &lead.rows_per_group, &lead.num_envs,
                    &params};
    const hipError_t e =
        hipLaunchKernel(kernel, dim3(grid), dim3(waves * kWave), args, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

template <typename C, typename R, typename S>
inline rlca_status launch_chunk_carries(void *slots, const Geometry &geo, bool backward,
                                        bool skew, hipStream_t stream) {
    int64_t n = geo.num_envs;
    uint32_t T = geo.T, m = geo.chunks_per_row, span = chunk_span(skew), phase = geo.out0_phase;
    int dir = backward ? 1 : 0;
    void *args[] = {&slots, &n, &T, &m, &span, &phase, &dir};
    const hipError_t e =
        hipLaunchKernel((const void *)chunk_carries<C, R, S, kChunkWaves>, dim3(grid_for(n)),
                        dim3(kChunkWaves * kWave), args, 0, stream);
    return e == hipSuccess ? RLCA_OK : RLCA_ERR_HIP;
}

// The three chunk-mode launches, all on one stream: aggregate, carries,
// apply (the apply grid capped at `apply_cap`).  V: the kernels' value type;
// the chunk maps are scanned in ScanOf<V, F64>, the kernels' own scan type.
template <typename V, typename S, bool F64, typename P>
inline rlca_status launch_chunked(const void *aggregate, const void *apply, P &params, Lead &lead,
                                  void *slots, bool backward, const LaunchShape &s,
                                  hipStream_t stream, uint32_t apply_cap = kOneShotMaxGrid) {
    uint32_t grid;
    params.geo = make_geometry(params.geo.num_envs, params.geo.T, s, &grid);
    const uint32_t apply_grid = grid_for(params.geo.num_groups, apply_cap);
    rlca_status st = launch_kernel(aggregate, kChunkWaves, grid, params, lead, stream);
    if (st == RLCA_OK)
        st = launch_chunk_carries<typename ScanOf<V, F64>::type, V, S>(slots, params.geo,
                                                                        backward, s.skew, stream);
    if (st == RLCA_OK) st = launch_kernel(apply, kChunkWaves, apply_grid, params, lead, stream);
    return st;
}

template <typename P>
inline rlca_status launch_full(const void *kernel, const LaunchShape &s, P &params, Lead &lead,
                               hipStream_t stream, uint32_t cap = kOneShotMaxGrid) {
    uint32_t grid;
    params.geo = make_geometry(params.geo.num_envs, params.geo.T, s, &grid, cap);
    return launch_kernel(kernel, s.vec ? s.waves : 4, grid, params, lead, stream);
}

// Workgroups of the launch (the last one, for the chunk modes) of a call of
// this shape, the grid capped at `cap`: the scalar path runs 4-wave
// workgroups.
inline uint32_t launch_grid(const LaunchShape &s, int64_t num_envs, int64_t T,
                            uint32_t cap = kOneShotMaxGrid) {
    uint32_t grid;
    make_geometry(num_envs, T, s, &grid, cap);
    return grid;
}

// The memory path of a launch shape.
inline int io_path(const LaunchShape &s) {
    return !s.vec ? kScalarIO : s.skew ? kVecSkew : kVecRows;
}

// The whole-row vector path instantiates every wave count and the wave-local
// variant; the skewed and the scalar (unaligned) paths one configuration each.
// Calls whose chains need it (f64) take the fp64-scan instantiations.
template <int EST, bool TRUNC, typename S, bool STATS = false>
const void *backward_kernel(const LaunchShape &s) {
#define RLCA_PICK_F64(IO, NW)                                                                  \
    return s.f64                                                                               \
               ? (const void *)backward_scan<EST, TRUNC, IO, NW, false, kFull, S, STATS, true> \
               : (const void *)backward_scan<EST, TRUNC, IO, NW, false, kFull, S, STATS, false>
    if (!s.vec) RLCA_PICK_F64(kScalarIO, 4);
    if (s.waves == 16)  // rows of several 4096-step tiles, fp32 scans only
        return s.skew ? (const void *)backward_scan<EST, TRUNC, kVecSkew, 16, false, kFull, S, STATS>
                      : (const void *)backward_scan<EST, TRUNC, kVecRows, 16, false, kFull, S, STATS>;
    if (s.skew) RLCA_PICK_F64(kVecSkew, 8);
    if (s.waves == 8 && !s.wave_local) RLCA_PICK_F64(kVecRows, 8);
    if (s.waves == 1) RLCA_PICK_F64(kVecRows, 1);
#undef RLCA_PICK_F64
#define RLCA_PICK(NW)                                                                          \
    return s.wave_local                                                                        \
               ? (const void *)backward_scan<EST, TRUNC, kVecRows, NW, true, kFull, S, STATS> \
               : (const void *)backward_scan<EST, TRUNC, kVecRows, NW, false, kFull, S, STATS>
    switch (s.waves) {
        case 1: RLCA_PICK(1);
        case 2: RLCA_PICK(2);
        case 8: RLCA_PICK(8);
        default: RLCA_PICK(4);
    }
#undef RLCA_PICK
}

template <int EST, bool TRUNC, typename S, bool STATS = false>
rlca_status launch_backward_variant(BackwardParams &p, const LaunchShape &s, hipStream_t stream) {
    Lead lead;
    lead_from<EST>(p, lead);
    const uint32_t cap = STATS ? kStatsMaxGrid : kOneShotMaxGrid;
    if (s.chunked) {
#define RLCA_CHUNKED(IO, F64)                                                                  \
    return launch_chunked<float, S, F64>(                                                      \
        (const void *)                                                                         \
            backward_scan<EST, TRUNC, IO, kChunkWaves, false, kChunkAggregate, S, false, F64>,  \
        (const void *)                                                                         \
            backward_scan<EST, TRUNC, IO, kChunkWaves, false, kChunkApply, S, STATS, F64>,      \
        p, lead, p.out0, true, s, stream, cap)
        if (s.skew) {
            if (s.f64) RLCA_CHUNKED(kVecSkew, true);
            RLCA_CHUNKED(kVecSkew, false);
        }
        if (s.f64) RLCA_CHUNKED(kVecRows, true);
        RLCA_CHUNKED(kVecRows, false);
#undef RLCA_CHUNKED
    }
    return launch_full(backward_kernel<EST, TRUNC, S, STATS>(s), s, p, lead, stream, cap);
}

template <int EST, typename S>
rlca_status launch_backward_typed(BackwardParams &p, const LaunchShape &s, hipStream_t stream) {
    return p.truncated != nullptr ? launch_backward_variant<EST, true, S>(p, s, stream)
                                  : launch_backward_variant<EST, false, S>(p, s, stream);
}

template <int EST>
rlca_status launch_backward(BackwardParams &p, const LaunchShape &s, int storage,
                            hipStream_t stream) {
    switch (storage) {
        case kStoreBF16: return launch_backward_typed<EST, __bf16>(p, s, stream);
        case kStoreF16: return launch_backward_typed<EST, _Float16>(p, s, stream);
        default: return launch_backward_typed<EST, float>(p, s, stream);
    }
}

template <typename V, int KIND, bool AFTER_DONE, typename S>
const void *forward_kernel(const LaunchShape &s) {
#define RLCA_PICK_F64(IO, NW)                                                                   \
    return s.f64                                                                                \
               ? (const void *)forward_scan<V, KIND, AFTER_DONE, IO, NW, false, kFull, S, true> \
               : (const void *)forward_scan<V, KIND, AFTER_DONE, IO, NW, false, kFull, S, false>
    if (!s.vec) RLCA_PICK_F64(kScalarIO, 4);
    if (s.waves == 16)  // rows of several 4096-step tiles, fp32 scans only
        return s.skew ? (const void *)forward_scan<V, KIND, AFTER_DONE, kVecSkew, 16, false, kFull, S>
                      : (const void *)forward_scan<V, KIND, AFTER_DONE, kVecRows, 16, false, kFull, S>;
    if (s.skew) RLCA_PICK_F64(kVecSkew, 8);
    if (s.waves == 8 && !s.wave_local) RLCA_PICK_F64(kVecRows, 8);
    if (s.waves == 1) RLCA_PICK_F64(kVecRows, 1);
#undef RLCA_PICK_F64
#define RLCA_PICK(NW)                                                                          \
    return s.wave_local                                                                        \
               ? (const void *)forward_scan<V, KIND, AFTER_DONE, kVecRows, NW, true, kFull, S> \
               : (const void *)forward_scan<V, KIND, AFTER_DONE, kVecRows, NW, false, kFull, S>
    switch (s.waves) {
        case 1: RLCA_PICK(1);
        case 2: RLCA_PICK(2);
        case 8: RLCA_PICK(8);
        default: RLCA_PICK(4);
    }
#undef RLCA_PICK
}

template <typename V, int KIND, bool AFTER_DONE, typename S>
rlca_status launch_forward_variant(ForwardParams &p, const LaunchShape &s, hipStream_t stream) {
    Lead lead;
    lead_from(p, lead);
    if (s.chunked) {
#define RLCA_CHUNKED(IO, F64)                                                               \
    return launch_chunked<V, S, F64>(                                                       \
        (const void *)forward_scan<V, KIND, AFTER_DONE, IO, kChunkWaves, false,             \
                                   kChunkAggregate, S, F64>,                                \
        (const void *)forward_scan<V, KIND, AFTER_DONE, IO, kChunkWaves, false, kChunkApply, \
                                   S, F64>,                                                 \
        p, lead, p.out, false, s, stream)
        if (s.skew) {
            if (s.f64) RLCA_CHUNKED(kVecSkew, true);
            RLCA_CHUNKED(kVecSkew, false);
        }
        if (s.f64) RLCA_CHUNKED(kVecRows, true);
        RLCA_CHUNKED(kVecRows, false);
#undef RLCA_CHUNKED
    }
    return launch_full(forward_kernel<V, KIND, AFTER_DONE, S>(s), s, p, lead, stream);
}

// The float forward scans in the requested storage type.
template <int KIND, bool AFTER_DONE>
rlca_status launch_forward_float(ForwardParams &p, const LaunchShape &s, int storage,
                                 hipStream_t stream) {
    switch (storage) {
        case kStoreBF16:
            return launch_forward_variant<float, KIND, AFTER_DONE, __bf16>(p, s, stream);
        case kStoreF16:
            return launch_forward_variant<float, KIND, AFTER_DONE, _Float16>(p, s, stream);
        default: return launch_forward_variant<float, KIND, AFTER_DONE, float>(p, s, stream);
    }
}

// ------------------------------------------------------------- grouped launch
// Several calls in one launch of 8-wave workgroups.  Call c owns the
// workgroups [end(c-1), end(c)); each runs one group of an 8-wave call, or
// eight groups of a one-wave call (one per wave).  Every member uses the
// vector path and full mode; `variant` names the estimator body and wave
// count.  The 14 head words come first among the kernel arguments, which
// the launch preloads into SGPRs: bits 0..23 of word i hold end(i) (unused
// calls: kHeadEndMask, above any workgroup index), bits 24..31 the variant
// of call i.  A workgroup finds its call and variant without a memory load
// and then fetches only that call's parameters.
constexpr int kGroupWaves = 8;
constexpr int kMaxGroupedCalls = 14;
constexpr uint32_t kHeadEndMask = 0xffffffu;
constexpr int kHeadVariantShift = 24;

union GroupedCall {
    BackwardParams b;
    ForwardParams f;
};

struct GroupedArgs {
    GroupedCall calls[kMaxGroupedCalls];
};

struct GroupedLaunch {
    uint32_t head[kMaxGroupedCalls];
    GroupedArgs args;
    uint32_t workgroups;  // end of the last call's range
};

// Variant numbering.  8-wave bodies: backward estimators 0..21 (estimator x
// truncation x wave-local), flag-driven forward scans 24..31 (int32 x
// after-done x wave-local), forward affine scan 32..33.  One-wave bodies
// (never wave-local): backward 34..44 (estimator x truncation), forward
// 46..49 (int32 x after-done), forward affine 50.  Skewed-window bodies
// (T % K != 0; 8 waves): backward 64..74, forward 80..83, forward affine 84.
constexpr int grouped_backward_variant(int est, bool trunc, bool wave_local, bool one_wave) {
    return one_wave ? 34 + est * 2 + (trunc ? 1 : 0)
                    : est * 4 + (trunc ? 2 : 0) + (wave_local ? 1 : 0);
}
constexpr int grouped_forward_variant(bool is_int, bool after_done, bool wave_local,
                                      bool one_wave) {
    return one_wave ? 46 + (is_int ? 2 : 0) + (after_done ? 1 : 0)
                    : 24 + (is_int ? 4 : 0) + (after_done ? 2 : 0) + (wave_local ? 1 : 0);
}
constexpr int grouped_affine_forward_variant(bool wave_local, bool one_wave) {
    return one_wave ? 50 : 32 + (wave_local ? 1 : 0);
}
constexpr int grouped_skew_backward_variant(int est, bool trunc) {
    return 64 + est * 2 + (trunc ? 1 : 0);
}
constexpr int grouped_skew_forward_variant(bool is_int, bool after_done) {
    return 80 + (is_int ? 2 : 0) + (after_done ? 1 : 0);
}
constexpr int kGroupedSkewAffineForward = 84;

// Classes of grouped launches, one kernel each (see est_batch.hip): 8-wave
// calls whose rows end at wave boundaries (wave-local), split into the light
// bodies and the importance-weighted ones (V-Trace, Retrace: more registers);
// other 8-wave calls; one-wave calls; calls over skewed windows (T % K != 0).
enum GroupClass : int {
    kGroupWaveLocal = 0,
    kGroupWaveLocalWeighted = 1,
    kGroupWaves8 = 2,
    kGroupOneWave = 3,
    kGroupSkew = 4,
};
constexpr int kGroupClasses = 5;
// Minimum waves per SIMD each class kernel is compiled for (one-shot shapes
// need all eight slots; the light wave-local bodies fit eight by themselves).
constexpr int kGroupClassWaves[kGroupClasses] = {1, 8, 8, 8, 8};

inline int group_class(const LaunchShape &s, bool weighted) {
    if (s.skew) return kGroupSkew;
    if (s.waves == 1) return kGroupOneWave;
    if (!s.wave_local) return kGroupWaves8;
    return weighted ? kGroupWaveLocalWeighted : kGroupWaveLocal;
}

rlca_status launch_grouped(const GroupedLaunch &launch, int storage, int cls,
                           hipStream_t stream);

// One translation unit per estimator instantiates these (see est_*.hip).
rlca_status launch_gae(BackwardParams &p, const LaunchShape &s, int storage, hipStream_t stream);
// GAE (fp32) that also reduces the advantages to p.stats in the same launch:
// launch_grid(s, ..., kStatsMaxGrid) (sum, sum of squares) pairs at
// p.stats_partials, behind the workspace's ticket counter.
rlca_status launch_gae_stats(BackwardParams &p, const LaunchShape &s, hipStream_t stream);
// Fused consumers (est_ppo.hip).  `workspace` starts with the ticket counter.
uint32_t ppo_grid(int64_t M);
rlca_status launch_ppo_clip_loss(const float *adv, const double *stats, const float *logp_new,
                                 const float *logp_old, float clip_eps, float norm_eps,
                                 int64_t M, bool vec, float *grad, void *workspace,
                                 double *loss, hipStream_t stream);
rlca_status launch_td_lambda(BackwardParams &p, const LaunchShape &s, int storage,
                             hipStream_t stream);
rlca_status launch_discounted(BackwardParams &p, const LaunchShape &s, int storage,
                              hipStream_t stream);
rlca_status launch_vtrace(BackwardParams &p, const LaunchShape &s, int storage,
                          hipStream_t stream);
rlca_status launch_retrace(BackwardParams &p, const LaunchShape &s, int storage,
                           hipStream_t stream);
rlca_status launch_affine_backward(BackwardParams &p, const LaunchShape &s, int storage,
                                   hipStream_t stream);
rlca_status launch_forward_float(ForwardParams &p, bool after_done, const LaunchShape &s,
                                 int storage, hipStream_t stream);
rlca_status launch_forward_u32(ForwardParams &p, bool after_done, const LaunchShape &s,
                               hipStream_t stream);
rlca_status launch_affine_forward(ForwardParams &p, const LaunchShape &s, int storage,
                                  hipStream_t stream);

}  // namespace rlca
