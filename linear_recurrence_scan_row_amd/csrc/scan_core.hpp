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
// (uint32 here) have no NaN and keep plain arithmetic.
__device__ __forceinline__ float apply_map(float a, float b, float x) {
    return b == 0.f ? a : a + b * x;
}
__device__ __forceinline__ uint32_t apply_map(uint32_t a, uint32_t b, uint32_t x) {
    return a + b * x;
}

// (a, b) <- (a, b) after (pa, pb): the map of a later run in scan order
// applied after the map of the earlier run.
__device__ __forceinline__ void compose(float &a, float &b, float pa, float pb) {
    const bool cut = b == 0.f;
    a = cut ? a : a + b * pa;
    b = cut ? b : b * pb;
}
__device__ __forceinline__ void compose(uint32_t &a, uint32_t &b, uint32_t pa, uint32_t pb) {
    a = a + b * pa;
    b = b * pb;
}

// One DPP step: fetch (a, b) from the lane selected by CTRL and compose.
// Lanes whose source is outside the row or whose row is masked off keep the
// identity (0, 1) as fetched value (bound_ctrl = 0 keeps `old`).
template <int CTRL, int ROW_MASK, typename V>
__device__ __forceinline__ void dpp_compose(V &a, V &b) {
    const V pa = from_bits<V>(__builtin_amdgcn_update_dpp(as_bits(V(0)), as_bits(a), CTRL,
                                                          ROW_MASK, 0xf, false));
    const V pb = from_bits<V>(__builtin_amdgcn_update_dpp(as_bits(V(1)), as_bits(b), CTRL,
                                                          ROW_MASK, 0xf, false));
    compose(a, b, pa, pb);
}

// Inclusive scan over the 64 lanes of a wave, lane 0 first.
template <typename V>
__device__ __forceinline__ void wave_inclusive_scan(V &a, V &b) {
    dpp_compose<0x111, 0xf>(a, b);  // row_shr:1
    dpp_compose<0x112, 0xf>(a, b);  // row_shr:2
    dpp_compose<0x114, 0xf>(a, b);  // row_shr:4
    dpp_compose<0x118, 0xf>(a, b);  // row_shr:8  -> prefix within each row of 16
    dpp_compose<0x142, 0xa>(a, b);  // row_bcast:15 into rows 1 and 3
    dpp_compose<0x143, 0xc>(a, b);  // row_bcast:31 into rows 2 and 3
}

// Value held by lane - 1 (lane 0 receives `first`): one DPP wave_shr:1 move,
// whose lane 0 has no source and keeps the `old` operand.
template <typename V>
__device__ __forceinline__ V from_lower_lane(V x, V first) {
    return from_bits<V>(
        __builtin_amdgcn_update_dpp(as_bits(first), as_bits(x), 0x138, 0xf, 0xf, false));
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
template <int NW, bool WAVE_LOCAL, typename V>
__device__ __forceinline__ V block_carry_in(V a, V b, V carry_in, V *lds_a, V *lds_b, int parity,
                                            V &carry_out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    wave_inclusive_scan(a, b);
    const V ea = from_lower_lane(a, V(0));
    const V eb = from_lower_lane(b, V(1));
    if constexpr (WAVE_LOCAL) {
        carry_out = V(0);
        return apply_map(ea, eb, V(0));
    }
    if constexpr (NW == 1) {
        // One wave: its total is lane 63's inclusive value; no LDS, no
        // barrier (so waves of one workgroup may run unrelated tiles).
        const V ta = from_bits<V>(__builtin_amdgcn_readlane(as_bits(a), kWave - 1));
        const V tb = from_bits<V>(__builtin_amdgcn_readlane(as_bits(b), kWave - 1));
        carry_out = apply_map(ta, tb, carry_in);
        return apply_map(ea, eb, carry_in);
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
        x = apply_map(lds_a[parity * NW + j], lds_b[parity * NW + j], x);
    }
    carry_out = x;
    return apply_map(ea, eb, xw);
}

// The map of the whole tile: the NW wave totals composed in scan order.  Used
// where a tile's result is handed to another workgroup instead of applied.
template <int NW, typename V>
__device__ __forceinline__ void block_total(V a, V b, V *lds_a, V *lds_b, V &ta, V &tb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    wave_inclusive_scan(a, b);
    if (lane == kWave - 1) {
        lds_a[w] = a;
        lds_b[w] = b;
    }
    __syncthreads();
    ta = V(0);
    tb = V(1);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        V a_j = lds_a[j], b_j = lds_b[j];
        compose(a_j, b_j, ta, tb);
        ta = a_j;
        tb = b_j;
    }
}

}  // namespace rlca
