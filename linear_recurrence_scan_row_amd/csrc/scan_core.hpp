// scan_core.hpp -- the shared affine scan of the credit-assignment kernels (gfx950, wave64).
//
// Every estimator is the first-order recurrence A_t = alpha_t + beta_t * A_{t+1}
// (backward) or A_t = alpha_t + beta_t * A_{t-1} (forward).  A step is the affine
// map x -> alpha + beta * x; a run of steps composes into one such map, and
// composition is associative ("rl-triton", paperlayer.ai summary, §2.2 Associative
// Scan and §5 Correctness analysis; operator printed in the gist.science technical
// summary, Methodology 1):
//     (a, b) after (a', b')  =  (a + b * a', b * b').
// (0, 1) is the identity, and beta = 0 cuts the chain: nothing from the other
// side of a boundary reaches the result (summary §5, Episode boundaries).
//
// Work split on the chip (one workgroup of NW waves):
//   * each lane owns K consecutive steps and folds them serially (work-efficient);
//   * a wave scans its 64 lane aggregates with DPP row_shr 1,2,4,8 and
//     row_bcast 15/31 (six dependent steps, no LDS);
//   * the NW wave totals meet in LDS behind one barrier (skipped when rows
//     end at wave boundaries);
//   * a tile carry passes between successive tiles of the workgroup's rows, so
//     a row of any length streams through registers and LDS never grows with T.
// Lanes are numbered in *scan order*: for backward scans the lane order is
// reversed time order, so the same "inclusive prefix over lower lanes" serves
// both directions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlca {

constexpr int kWave = 64;

// ------------------------------------------------------------------ arithmetic
// Scan values are float, or uint32 for the integer prefix sum (unsigned, so
// additions wrap modulo 2^32 exactly as two's-complement int32 does).

template <typename V>
__device__ __forceinline__ int as_bits(V x) {
    return __builtin_bit_cast(int, x);
}
template <typename V>
__device__ __forceinline__ V from_bits(int x) {
    return __builtin_bit_cast(V, x);
}

// Map arithmetic with chain cuts.  A step with beta = 0 severs the chain: its
// map is x -> alpha whatever x is, and so is every composition that contains
// it (summary §5 Correctness analysis).  IEEE arithmetic gives that only for
// finite x (0 * NaN and 0 * inf are NaN), so the float forms select instead
// of multiplying by zero: a NaN or infinity on the far side of an episode
// boundary, or in another row of the tile, stays there.  For finite values
// the results are the same.  One test of the later map's beta serves both
// halves of a composition: when that beta is NaN the composed value is NaN
// already, so a NaN composed beta changes nothing.  The int32 prefix sums
// (uint32 here) have no NaN and keep plain arithmetic.  The double forms
// serve the fp64 scans (see ScanOf).
//
// LEGACY (fp32 only): the hardware's legacy multiply, v_mul_legacy_f32,
// whose product is 0 whenever an operand is 0 (even against NaN or
// infinity), gives the same cut-safe results in three instructions instead
// of five (compare, FMA, multiply, two selects): a + b*x as a legacy
// product and an add, so the fp32 result rounds twice instead of once.
// It differs from the selects only for an infinite beta (inf * 0 = 0),
// which the importance-weighted estimators, the only users, never have:
// their beta is gamma * lambda * min(c_bar, ratio), in [0, 1], or NaN.
extern "C" __device__ float rlca_fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");

template <bool LEGACY = false, typename V>
__device__ __forceinline__ V apply_map(V a, V b, V x) {
    if constexpr (__is_same(V, uint32_t)) {
        return a + b * x;
    } else if constexpr (LEGACY && __is_same(V, float)) {
        return a + rlca_fmul_legacy(b, x);
    } else {
        return b == V(0) ? a : a + b * x;
    }
}

// (a, b) <- (a, b) after (pa, pb): the map of a later run in scan order
// applied after the map of the earlier run.
template <bool LEGACY = false, typename V>
__device__ __forceinline__ void compose(V &a, V &b, V pa, V pb) {
    if constexpr (__is_same(V, uint32_t)) {
        a = a + b * pa;
        b = b * pb;
    } else if constexpr (LEGACY && __is_same(V, float)) {
        a = a + rlca_fmul_legacy(b, pa);
        b = rlca_fmul_legacy(b, pb);
    } else {
        const bool cut = b == V(0);
        a = cut ? a : a + b * pa;
        b = cut ? b : b * pb;
    }
}

// Scan type of a kernel over values of type V.  fp32 rounding hurts where a
// value is carried across waves along a chain that barely decays: a product
// of n factors beta carries a relative error of up to about n * 2^-24, and it
// scales the carried value once per wave, over the ~1 / (1 - beta^256) waves
// the chain remembers; at beta = 1 the products are exact, but the carried
// sums' own rounding then accumulates over the whole row.  Kernels whose
// calls have rows spanning waves with beta near 1 (the host's choice, F64)
// therefore scan in fp64 from the lane fold on and round each output to
// fp32 once.  Integer sums are exact in any case.
template <typename V, bool F64>
struct ScanOf {
    typedef V type;
};
template <>
struct ScanOf<float, true> {
    typedef double type;
};

// Value of lane CTRL selects (DPP), or `old` where there is none; 64-bit
// values move as two 32-bit halves.
template <int CTRL, int ROW_MASK, typename V>
__device__ __forceinline__ V dpp_move(V x, V old) {
    if constexpr (sizeof(V) == 4) {
        return from_bits<V>(__builtin_amdgcn_update_dpp(as_bits(old), as_bits(x), CTRL, ROW_MASK,
                                                        0xf, false));
    } else {
        static_assert(sizeof(V) == 8, "32- or 64-bit values");
        const uint64_t u = __builtin_bit_cast(uint64_t, x), o = __builtin_bit_cast(uint64_t, old);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(
            (int)(uint32_t)o, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
            (int)(uint32_t)(o >> 32), (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
        return __builtin_bit_cast(V, ((uint64_t)hi << 32) | lo);
    }
}

// Value of `lane` (uniform), 32- or 64-bit.
template <typename V>
__device__ __forceinline__ V read_lane(V x, int lane) {
    if constexpr (sizeof(V) == 4) {
        return from_bits<V>(__builtin_amdgcn_readlane(as_bits(x), lane));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
        return __builtin_bit_cast(V, ((uint64_t)hi << 32) | lo);
    }
}

// One DPP step: fetch (a, b) from the lane selected by CTRL and compose.
// Lanes whose source is outside the row or whose row is masked off keep the
// identity (0, 1) as fetched value (bound_ctrl = 0 keeps `old`).
template <int CTRL, int ROW_MASK, bool LEGACY, typename V>
__device__ __forceinline__ void dpp_compose(V &a, V &b) {
    const V pa = dpp_move<CTRL, ROW_MASK>(a, V(0));
    const V pb = dpp_move<CTRL, ROW_MASK>(b, V(1));
    compose<LEGACY>(a, b, pa, pb);
}

// Inclusive scan over the 64 lanes of a wave, lane 0 first.
template <bool LEGACY = false, typename V>
__device__ __forceinline__ void wave_inclusive_scan(V &a, V &b) {
    dpp_compose<0x111, 0xf, LEGACY>(a, b);  // row_shr:1
    dpp_compose<0x112, 0xf, LEGACY>(a, b);  // row_shr:2
    dpp_compose<0x114, 0xf, LEGACY>(a, b);  // row_shr:4
    dpp_compose<0x118, 0xf, LEGACY>(a, b);  // row_shr:8  -> prefix within each row of 16
    dpp_compose<0x142, 0xa, LEGACY>(a, b);  // row_bcast:15 into rows 1 and 3
    dpp_compose<0x143, 0xc, LEGACY>(a, b);  // row_bcast:31 into rows 2 and 3
}

// Value held by lane - 1 (lane 0 receives `first`): one DPP wave_shr:1 move,
// whose lane 0 has no source and keeps the `old` operand.
template <typename V>
__device__ __forceinline__ V from_lower_lane(V x, V first) {
    return dpp_move<0x138, 0xf>(x, first);
}

// Workgroup-wide scan of per-lane maps (a, b) given in scan order, with an
// incoming carry for the whole tile.  Returns the value of A just before this
// lane's chunk in scan order (= after the preceding lanes), and writes the
// value after the whole tile to `carry_out`.  The NW wave totals meet in LDS
// behind one barrier; `lds_a` / `lds_b` hold 2*NW slots and `parity`
// alternates between tiles so one barrier per tile suffices.
//
// WAVE_LOCAL: every wave's segment starts, in scan order, with a chain cut
// (rows end at wave boundaries), so whatever enters a wave from outside is
// multiplied by an exact zero before it reaches any output.  The LDS exchange
// and the barrier are then skipped and 0 enters each wave instead; the
// results are the same values the exchange would give.
template <int NW, bool WAVE_LOCAL, bool LEGACY = false, typename V>
__device__ __forceinline__ V block_carry_in(V a, V b, V carry_in, V *lds_a, V *lds_b, int parity,
                                            V &carry_out) {
    const int lane = threadIdx.x & (kWave - 1);
    // the wave index is uniform: as a scalar, the fold's `j == w` tests
    // below are scalar compares, not per-lane masks held across the fold
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    wave_inclusive_scan<LEGACY>(a, b);
    const V ea = from_lower_lane(a, V(0));
    const V eb = from_lower_lane(b, V(1));
    if constexpr (WAVE_LOCAL) {
        carry_out = V(0);
        return apply_map<LEGACY>(ea, eb, V(0));
    }
    if constexpr (NW == 1) {
        // One wave: its total is lane 63's inclusive value; no LDS, no
        // barrier (so waves of one workgroup may run unrelated tiles).
        const V ta = read_lane(a, kWave - 1);
        const V tb = read_lane(b, kWave - 1);
        carry_out = apply_map<LEGACY>(ta, tb, carry_in);
        return apply_map<LEGACY>(ea, eb, carry_in);
    }
    if (lane == kWave - 1) {
        lds_a[parity * NW + w] = a;
        lds_b[parity * NW + w] = b;
    }
    __syncthreads();
    V x = carry_in;   // A entering wave 0
    V xw = carry_in;  // A entering this lane's wave
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        if (j == w) xw = x;
        x = apply_map<LEGACY>(lds_a[parity * NW + j], lds_b[parity * NW + j], x);
    }
    carry_out = x;
    return apply_map<LEGACY>(ea, eb, xw);
}

// The map of the whole tile: the NW wave totals composed in scan order.  Used
// where a tile's result is handed to another workgroup instead of applied.
// Like block_carry_in, the wave totals go to the half of the 2*NW LDS slots
// that `parity` selects, and the caller alternates it between tiles: a wave
// that runs ahead into the next tile writes the other half, so it cannot
// overwrite a total another wave is still reading (one barrier per tile).
template <int NW, typename V>
__device__ __forceinline__ void block_total(V a, V b, V *lds_a, V *lds_b, int parity, V &ta,
                                            V &tb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    wave_inclusive_scan(a, b);
    if (lane == kWave - 1) {
        lds_a[parity * NW + w] = a;
        lds_b[parity * NW + w] = b;
    }
    __syncthreads();
    ta = V(0);
    tb = V(1);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        V a_j = lds_a[parity * NW + j], b_j = lds_b[parity * NW + j];
        compose(a_j, b_j, ta, tb);
        ta = a_j;
        tb = b_j;
    }
}

}  // namespace rlca
