// bench_floor.hip -- the streaming floor of a benchmark step (measurement aid
// for bench.py; not part of the library).
//
// One launch moves exactly the bytes of a step's calls with the library's
// tiling and access widths, and does no arithmetic beyond folding the loaded
// words into the stored ones: 2048-step tiles of 8 waves x 64 lanes x 4
// consecutive steps, one workgroup per tile, every call of the step in the
// same launch (as the grouped launch runs them).  Each lane reads its 4 steps
// of every per-step input with one access (16 bytes for 4-byte elements, 8
// for 2-byte ones, 4 for a flag stream), reads the per-row value of a row
// that ends in its 4 steps, and writes its 4 steps of every output with one
// access, all non-temporal.  The time this takes is what the estimator
// kernels' memory traffic costs by itself at that size and shape.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxIn = 9, kMaxOut = 2, kMaxCalls = 8;
constexpr int kLanes = 512, kSteps = 4, kTile = kLanes * kSteps;

struct FloorCall {
    const void *in[kMaxIn];
    void *out[kMaxOut];
    const void *row;    // per-row input (bootstrap), nullable
    uint64_t steps;     // num_envs * T, a multiple of 4
    uint32_t T;         // a multiple of 4
    uint32_t tiles;     // ceil(steps / 2048)
    uint8_t in_bytes[kMaxIn];    // element size of each input: 4, 2 or 1
    uint8_t out_bytes[kMaxOut];  // 4 or 2
    uint8_t row_bytes;           // 4 or 2
    uint8_t nin, nout;
};

struct FloorLaunch {
    FloorCall calls[kMaxCalls];
    uint32_t ncalls;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t load_steps(const void *p, int bytes, uint64_t i) {
    if (bytes == 4) {
        const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p) + i / 4);
        return v.x ^ v.y ^ v.z ^ v.w;
    }
    if (bytes == 2) {
        const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2 *>(p) + i / 4);
        return v.x ^ v.y;
    }
    return __builtin_nontemporal_load(static_cast<const uint32_t *>(p) + i / 4);
}

__device__ __forceinline__ void store_steps(void *p, int bytes, uint64_t i, uint32_t x) {
    if (bytes == 4) {
        const u32x4 v = {x, x ^ 1u, x ^ 2u, x ^ 3u};
        __builtin_nontemporal_store(v, static_cast<u32x4 *>(p) + i / 4);
    } else {
        const u32x2 v = {x, x ^ 1u};
        __builtin_nontemporal_store(v, static_cast<u32x2 *>(p) + i / 4);
    }
}

__global__ __launch_bounds__(kLanes) void stream_floor(FloorLaunch l) {
    // the call whose tile range holds this workgroup
    uint32_t c = 0, first = 0;
    for (uint32_t k = 0; k + 1 < l.ncalls; ++k) {
        if (blockIdx.x >= first + l.calls[k].tiles) {
            first += l.calls[k].tiles;
            c = k + 1;
        }
    }
    const FloorCall &f = l.calls[c];
    const uint64_t i = ((uint64_t)(blockIdx.x - first) * kLanes + threadIdx.x) * kSteps;
    if (i >= f.steps) return;
    uint32_t v[kMaxIn + 1];
#pragma unroll
    for (int k = 0; k < kMaxIn; ++k) v[k] = k < f.nin ? load_steps(f.in[k], f.in_bytes[k], i) : 0u;
    v[kMaxIn] = 0u;
    if (f.row != nullptr && (i + kSteps) % f.T == 0) {
        const uint64_t r = (i + kSteps) / f.T - 1;
        v[kMaxIn] = f.row_bytes == 4 ? static_cast<const uint32_t *>(f.row)[r]
                                     : static_cast<const uint16_t *>(f.row)[r];
    }
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k <= kMaxIn; ++k) x ^= v[k];
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k)
        if (k < f.nout) store_steps(f.out[k], f.out_bytes[k], i, x + k);
}

}  // namespace

// Enqueue one floor launch on `stream`; returns the hipError_t of the launch
// (0 on success), or -1 for a description the kernel does not take.
extern "C" int bench_floor_launch(const FloorLaunch *l, hipStream_t stream) {
    if (l == nullptr || l->ncalls == 0 || l->ncalls > (uint32_t)kMaxCalls) return -1;
    uint32_t tiles = 0;
    for (uint32_t k = 0; k < l->ncalls; ++k) {
        const FloorCall &f = l->calls[k];
        if (f.nin > kMaxIn || f.nout > kMaxOut || f.T == 0 || f.T % kSteps != 0 ||
            f.steps % kSteps != 0 || f.tiles != (f.steps + kTile - 1) / kTile)
            return -1;
        tiles += f.tiles;
    }
    FloorLaunch copy = *l;
    void *args[] = {&copy};
    return (int)hipLaunchKernel((const void *)stream_floor, dim3(tiles), dim3(kLanes), args, 0,
                                stream);
}

// sizeof(FloorLaunch), for the caller's structure layout check
extern "C" size_t bench_floor_launch_bytes() { return sizeof(FloorLaunch); }
