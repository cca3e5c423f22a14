// The ring AllReduce in one launch (gfx950): the 2(N-1) steps of tirogla.com
// "Ring all-reduce" ("How it works") run inside a single persistent grid,
// separated by grid-wide barriers instead of kernel boundaries.
//
// Each step is exactly the work of the one-launch-per-step ring
// (ring_reduce_tiles, ring_copy_tiles): the blocks stride over every chunk's
// tiles, then all of them meet at a barrier before the next step reads what
// this one wrote.  The barrier is the cooperative-groups grid barrier, which
// needs every block resident at once: the kernel is only ever started with
// hipLaunchCooperativeKernel, on a grid no larger than the number of blocks
// the device can hold at once (the runtime refuses a larger one), and every
// block runs the same sequence of barriers (no block leaves early).  The
// barrier's agent-scope fences make one step's stores visible to the next
// step's loads on every XCD.

#include <hip/hip_cooperative_groups.h>

#include <atomic>

#include "ar_device.h"

namespace arimpl {
namespace {

template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_persistent(const KernelArgs a) {
    namespace cg = cooperative_groups;
    cg::grid_group grid = cg::this_grid();
    const int n = a.nranks;
    for (int s = 0; s < n - 1; ++s) {      // reduce-scatter steps
        ring_reduce_tiles<DT, OP, VEC>(a, s);
        grid.sync();
    }
    for (int s = 0; s < n - 1; ++s) {      // all-gather steps
        ring_copy_tiles<DT, VEC>(a, s, 0);
        if (s + 1 < n - 1) grid.sync();
    }
}

constexpr int kMaxDevices = 64;

// Blocks per compute unit the persistent grid uses.  Every block pays for
// the barrier's fences (a write-back and invalidation of its L2), so fewer
// blocks barrier faster; measured on MI355X at 8 x 2^26 float32, 2 per CU
// (4,877 -> 2,544 us against the 8 the device could hold) beats 1, 4 and 8.
constexpr int kPersistentBlocksPerCu = 2;

// Blocks of this instance the persistent grid may use on the current device:
// at most what the device holds at once (cached per device; 0 until queried).
template <int DT, int OP, int VEC>
hipError_t resident_blocks(int* out) {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) {
            *out = v;
            return hipSuccess;
        }
    }
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring_persistent<DT, OP, VEC>, kThreads, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int v = (per_cu < kPersistentBlocksPerCu ? per_cu : kPersistentBlocksPerCu) * cus;
    if (v <= 0) return hipErrorInvalidConfiguration;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
    *out = v;
    return hipSuccess;
}

template <int DT, int OP, int VEC>
hipError_t launch_t(const Launch& l, const KernelArgs& a, hipStream_t s) {
    int resident = 0;
    hipError_t e = resident_blocks<DT, OP, VEC>(&resident);
    if (e != hipSuccess) return e;
    const unsigned blocks = l.blocks < static_cast<unsigned>(resident) ? l.blocks : static_cast<unsigned>(resident);
    KernelArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_ring_persistent<DT, OP, VEC>),
                                      dim3(blocks > 0 ? blocks : 1), dim3(kThreads), params, 0, s);
}

template <int DT, int OP>
hipError_t by_vec(const Launch& l, const KernelArgs& a, hipStream_t s) {
    constexpr int V = 16 / elem_size<DT>();
    return l.vec ? launch_t<DT, OP, V>(l, a, s) : launch_t<DT, OP, 1>(l, a, s);
}

template <int DT>
hipError_t by_op(const Launch& l, const KernelArgs& a, hipStream_t s) {
    switch (l.op) {
        case AR_SUM: return by_vec<DT, AR_SUM>(l, a, s);
        case AR_PROD: return by_vec<DT, AR_PROD>(l, a, s);
        case AR_MIN: return by_vec<DT, AR_MIN>(l, a, s);
        case AR_MAX: return by_vec<DT, AR_MAX>(l, a, s);
        case AR_AVG: return by_vec<DT, AR_AVG>(l, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_persistent(const Launch& l, const KernelArgs& a, hipStream_t stream) {
    // Never inside a stream capture: a captured launch could replay without
    // the cooperative guarantees the grid barrier depends on.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    switch (l.dtype) {
        case AR_FLOAT32: return by_op<AR_FLOAT32>(l, a, stream);
        case AR_BFLOAT16: return by_op<AR_BFLOAT16>(l, a, stream);
        case AR_INT32: return by_op<AR_INT32>(l, a, stream);
        case AR_FLOAT16: return by_op<AR_FLOAT16>(l, a, stream);
        default: return hipErrorInvalidValue;   // float32 partials have no persistent form
    }
}

}  // namespace arimpl
