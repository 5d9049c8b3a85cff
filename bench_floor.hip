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
//
// Every stream's load goes out back to back, before any loaded value is
// used: inputs come ordered by element size (4-byte, then 2-byte, then
// 1-byte), each call runs a straight-line body for its counts of streams, and
// the row-end test divides by T with a multiply-high (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994,
// the round-up method for an N-bit dividend), its constants set on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxIn = 9, kMaxOut = 2, kMaxCalls = 8;
constexpr int kLanes = 512, kSteps = 4, kTile = kLanes * kSteps;

struct FloorCall {
    const void *in[kMaxIn];  // n4 4-byte streams, then n2 2-byte, then n1 1-byte
    void *out[kMaxOut];
    const void *row;         // per-row input (bootstrap), nullable
    uint64_t steps;          // num_envs * T, a multiple of 4, at most 2^31
    uint32_t T;              // a multiple of 4
    uint32_t tiles;          // ceil(steps / 2048)
    uint32_t magic, shift;   // n / T == (h + ((n - h) >> 1)) >> shift, h = mulhi(n, magic)
                             // (set by bench_floor_prepare)
    uint8_t n4, n2, n1, nout;
    uint8_t out_bytes;       // 4 or 2, every output of the call
    uint8_t row_bytes;       // 4 or 2
    uint8_t sig;             // index of (n4, n2, n1, nout, out_bytes) in kSigs (likewise)
    uint8_t pad;
};

struct FloorLaunch {
    FloorCall calls[kMaxCalls];
    uint32_t ncalls;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The stream signatures the benchmark's calls have: (4-byte inputs, 2-byte
// inputs, 1-byte inputs, outputs, output element bytes).  A call's body is
// straight-line code for its signature, every load issued before any value
// is used.
struct Sig {
    int n4, n2, n1, nout, ob;
};
constexpr Sig kSigs[] = {
    {2, 0, 1, 2, 4}, {3, 0, 2, 2, 4}, {2, 0, 1, 1, 4}, {3, 0, 2, 1, 4}, {4, 0, 1, 2, 4},
    {6, 0, 2, 1, 4}, {1, 0, 1, 1, 4}, {3, 0, 0, 1, 4}, {0, 2, 1, 2, 2}, {0, 3, 2, 2, 2},
    {0, 2, 1, 1, 2}, {0, 3, 2, 1, 2}, {0, 4, 1, 2, 2}, {0, 6, 2, 1, 2}, {0, 1, 1, 1, 2},
};
constexpr int kNumSigs = sizeof(kSigs) / sizeof(kSigs[0]);

template <int S>
__device__ __forceinline__ void floor_body(const FloorCall &f, uint32_t i) {
    constexpr Sig g = kSigs[S];
    const uint32_t q = i / kSteps;  // this lane's 4-step group
    u32x4 a[g.n4 > 0 ? g.n4 : 1];
    u32x2 b[g.n2 > 0 ? g.n2 : 1];
    uint32_t c[g.n1 > 0 ? g.n1 : 1];
#pragma unroll
    for (int k = 0; k < g.n4; ++k)
        a[k] = __builtin_nontemporal_load(static_cast<const u32x4 *>(f.in[k]) + q);
#pragma unroll
    for (int k = 0; k < g.n2; ++k)
        b[k] = __builtin_nontemporal_load(static_cast<const u32x2 *>(f.in[g.n4 + k]) + q);
#pragma unroll
    for (int k = 0; k < g.n1; ++k)
        c[k] = __builtin_nontemporal_load(static_cast<const uint32_t *>(f.in[g.n4 + g.n2 + k]) + q);
    // the row ending in these 4 steps: (i + 4) % T == 0 (T % 4 == 0)
    const uint32_t n = i + kSteps;
    const uint32_t h = __umulhi(n, f.magic);
    const uint32_t r = (h + ((n - h) >> 1)) >> f.shift;  // n / T
    uint32_t x = 0u;
    if (f.row != nullptr && r * f.T == n)
        x = f.row_bytes == 4 ? static_cast<const uint32_t *>(f.row)[r - 1]
                             : static_cast<const uint16_t *>(f.row)[r - 1];
#pragma unroll
    for (int k = 0; k < g.n4; ++k) x ^= a[k].x ^ a[k].y ^ a[k].z ^ a[k].w;
#pragma unroll
    for (int k = 0; k < g.n2; ++k) x ^= b[k].x ^ b[k].y;
#pragma unroll
    for (int k = 0; k < g.n1; ++k) x ^= c[k];
#pragma unroll
    for (int k = 0; k < g.nout; ++k) {
        if constexpr (g.ob == 4) {
            const u32x4 o = {x + k, x ^ 1u, x ^ 2u, x ^ 3u};
            __builtin_nontemporal_store(o, static_cast<u32x4 *>(f.out[k]) + q);
        } else {
            const u32x2 o = {x + k, x ^ 1u};
            __builtin_nontemporal_store(o, static_cast<u32x2 *>(f.out[k]) + q);
        }
    }
}

template <int S>
__device__ __forceinline__ void dispatch(const FloorCall &f, uint32_t i) {
    if constexpr (S < kNumSigs) {
        if (f.sig == S)
            floor_body<S>(f, i);
        else
            dispatch<S + 1>(f, i);
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
    const uint32_t i = ((blockIdx.x - first) * kLanes + threadIdx.x) * kSteps;
    if (i >= (uint32_t)f.steps) return;
    dispatch<0>(f, i);
}

// The round-up constants for dividing 32-bit n by d >= 2: with l = ceil(log2 d),
// magic = floor(2^32 (2^l - d) / d) + 1 and shift = l - 1.
bool division_constants(uint32_t d, uint32_t &magic, uint32_t &shift) {
    if (d < 2) return false;
    uint32_t l = 0;
    while ((uint64_t)1 << l < d) ++l;
    magic = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
    shift = l - 1;
    return true;
}

}  // namespace

// Check a launch description and fill in each call's division constants
// and signature index; returns the launch's workgroup count, or -1 for a
// description the kernel does not take.  No GPU call.
extern "C" int64_t bench_floor_prepare(FloorLaunch *l) {
    if (l == nullptr || l->ncalls == 0 || l->ncalls > (uint32_t)kMaxCalls) return -1;
    int64_t tiles = 0;
    for (uint32_t k = 0; k < l->ncalls; ++k) {
        FloorCall &f = l->calls[k];
        if (f.n4 + f.n2 + f.n1 > kMaxIn || f.nout > kMaxOut || f.T % kSteps != 0 ||
            f.steps % kSteps != 0 || f.steps > ((uint64_t)1 << 31) ||
            f.tiles != (f.steps + kTile - 1) / kTile || (f.out_bytes != 4 && f.out_bytes != 2) ||
            (f.row != nullptr && f.row_bytes != 4 && f.row_bytes != 2) ||
            !division_constants(f.T, f.magic, f.shift))
            return -1;
        f.sig = kNumSigs;
        for (int g = 0; g < kNumSigs; ++g)
            if (kSigs[g].n4 == f.n4 && kSigs[g].n2 == f.n2 && kSigs[g].n1 == f.n1 &&
                kSigs[g].nout == f.nout && kSigs[g].ob == f.out_bytes)
                f.sig = (uint8_t)g;
        if (f.sig == kNumSigs) return -1;
        tiles += f.tiles;
    }
    return tiles;
}

// Enqueue one floor launch on `stream` (the description as bench_floor_prepare
// takes it; the caller's copy is not changed); returns the hipError_t of the
// launch (0 on success), or -1 for a description the kernel does not take.
extern "C" int bench_floor_launch(const FloorLaunch *l, hipStream_t stream) {
    if (l == nullptr) return -1;
    FloorLaunch copy = *l;
    const int64_t tiles = bench_floor_prepare(&copy);
    if (tiles < 0) return -1;
    void *args[] = {&copy};
    return (int)hipLaunchKernel((const void *)stream_floor, dim3((uint32_t)tiles), dim3(kLanes),
                                args, 0, stream);
}

// sizeof(FloorLaunch), for the caller's structure layout check
extern "C" size_t bench_floor_launch_bytes() { return sizeof(FloorLaunch); }

// n / d by the kernel's method, on the host: for the caller's check of the
// constants (returns UINT32_MAX for a divisor the kernel does not take).
extern "C" uint32_t bench_floor_divide(uint32_t n, uint32_t d) {
    uint32_t magic, shift;
    if (!division_constants(d, magic, shift)) return UINT32_MAX;
    const uint32_t h = (uint32_t)(((uint64_t)n * magic) >> 32);
    return (h + ((n - h) >> 1)) >> shift;
}
