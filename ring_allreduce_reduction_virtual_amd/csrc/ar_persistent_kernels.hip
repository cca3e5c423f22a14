// The ring AllReduce in one launch (gfx950): the 2(N-1) steps of tirogla.com
// "Ring all-reduce" ("How it works") without a launch per step, in two
// forms.
//
// k_ring_persistent runs the steps inside a single persistent grid,
// separated by grid-wide barriers instead of kernel boundaries.  Each step
// is exactly the work of the one-launch-per-step ring (ring_reduce_tiles,
// ring_copy_tiles): the blocks stride over every chunk's tiles, then all of
// them meet at a barrier before the next step reads what this one wrote.
// The barrier is the cooperative-groups grid barrier, which needs every
// block resident at once: the kernel is only ever started with
// hipLaunchCooperativeKernel, on a grid no larger than the number of blocks
// the device can hold at once (the runtime refuses a larger one), and every
// block runs the same sequence of barriers (no block leaves early).  The
// barrier's agent-scope fences make one step's stores visible to the next
// step's loads on every XCD.
//
// k_ring_pipelined instead pipelines slices of the chunks through the ring,
// as "AllReduce, All the Way Down" describes the tensor being divided into
// chunks that are pipelined: a block takes one slice (one tile: 8 KiB per
// rank) of one chunk and carries it through all 2(N-1) steps in order.  A
// step of the ring reads only what the previous step wrote at the same
// positions, and each thread keeps the same positions in every step, so a
// thread only ever reads back its own earlier stores: no barrier, no
// flag, no cross-block ordering.  Every step still goes through memory:
// the incoming partial is loaded from the sender's buffer, not forwarded
// in registers.
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

// A unit stored with a cache-allocating store: the next step of the
// same thread reads it back.
template <int DT, int VEC>
__device__ __forceinline__ void store_unit_cached(char* tb, uint32_t off, typename Unit<DT, VEC>::T x) {
    if constexpr (VEC > 1) {
        *reinterpret_cast<u32x4*>(tb + off) = x;
    } else if constexpr (elem_size<DT>() == 2) {
        *reinterpret_cast<uint16_t*>(tb + off) = static_cast<uint16_t>(x);
    } else {
        *reinterpret_cast<uint32_t*>(tb + off) = x;
    }
}

// Keeps the compiler from forwarding a step's stores to the next step's
// loads: each step receives its partial from the sender's buffer.
__device__ __forceinline__ void step_boundary() { __asm__ __volatile__("" ::: "memory"); }

// The slice of chunk c that a block owns, through the ring's reduce-scatter
// (step s: rank c+s+1 adds its own value to the partial of rank c+s, the
// last step completing the chunk) and all-gather (step s: rank c+s copies
// the finished chunk from rank c+s-1).  The chunk's head and tail elements
// go through the same steps, one element per thread, in the chunk's first
// block.
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_pipelined(const KernelArgs a) {
    static_assert(!acc_f32<DT>(), "float32 partials have no pipelined form");
    using U = Unit<DT, VEC>;                 // the send buffers: read once, nontemporal
    using UC = Unit<DT, VEC, false>;         // partials: read back from the cache
    using F = Fold<DT, OP, VEC>;
    using F1 = Fold<DT, OP, 1>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            const uint64_t b = i * ESZ;
            for (int s = 0; s < n - 1; ++s) {
                const int r = ring_rank(c, s + 1, n);
                const int p = ring_rank(c, s, n);
                const uint32_t in = load_elem<ESZ>((s == 0 ? a.send[p] : a.recv[p]) + b);
                uint32_t v = F1::add(load_elem<ESZ>(a.send[r] + b), in);
                if (s == n - 2) v = F1::done(v, n);
                store_unit_cached<DT, 1>(a.recv[r] + b, 0u, v);
                step_boundary();
            }
            for (int s = 0; s < n - 1; ++s) {
                const int r = ring_rank(c, s, n);
                const int p = ring_rank(r, n - 1, n);
                store_unit_cached<DT, 1>(a.recv[r] + b, 0u, load_elem<ESZ>(a.recv[p] + b));
                step_boundary();
            }
        }
    }
    for (int s = 0; s < n - 1; ++s) {        // reduce-scatter
        const int r = ring_rank(c, s + 1, n);
        const int p = ring_rank(c, s, n);
        const char* tl = U::tile(a.send[r] - adj, tv0);
        const char* ti = UC::tile((s == 0 ? a.send[p] : a.recv[p]) - adj, tv0);
        typename U::T x[kUnroll], y[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) {
                x[u] = U::load(tl, U::lane_off(u));
                y[u] = UC::load(ti, U::lane_off(u));
            }
        }
        char* to = U::tile(a.recv[r] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!live[u]) continue;
            typename U::T z = F::add(x[u], y[u]);
            if (s == n - 2) z = F::done(z, n);
            store_unit_cached<DT, VEC>(to, U::lane_off(u), z);
        }
        step_boundary();
    }
    for (int s = 0; s < n - 1; ++s) {        // all-gather
        const int r = ring_rank(c, s, n);
        const int p = ring_rank(r, n - 1, n);
        const char* ts = UC::tile(a.recv[p] - adj, tv0);
        typename U::T x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) x[u] = UC::load(ts, U::lane_off(u));
        }
        char* td = U::tile(a.recv[r] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) store_unit_cached<DT, VEC>(td, U::lane_off(u), x[u]);
        }
        step_boundary();
    }
    AR_TILE_LOOP_END
}

// The pipelined ring with its reduce-scatter partials in the workspace: one
// partial per position, which every step of the slice's owner reads and
// overwrites (the ring's reduce-scatter as k_ring_reduce_step_ws runs it,
// slice by slice).  mode 0, reduce-scatter: the last step writes the
// finished value into shard c of rank c.  mode 1, AllReduce (float32
// partials of bf16): the last step writes it, rounded, into chunk c of rank
// c-1's own buffer, and the all-gather steps follow as in k_ring_pipelined.
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_pipelined_ws(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    using UC = Unit<DT, VEC, false>;
    using F = Fold<DT, OP, VEC>;
    using F1 = Fold<DT, OP, 1>;
    using P = Partials<DT, VEC>;
    using P1 = Partials<DT, 1>;
    constexpr int ESZ = elem_size<DT>();
    const bool allreduce = a.mode == 1;
    const char* ws_base = a.ws - static_cast<int64_t>(a.ofs) * P::kElemBytes;
    AR_TILE_LOOP_BEGIN
    char* shard = a.recv[c];
    const int owner = ring_rank(c, n - 1, n);    // rank c-1 finishes chunk c
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            const uint64_t b = i * ESZ;
            for (int s = 0; s < n - 1; ++s) {
                const int r = ring_rank(c, s + 1, n);
                const typename F1::A in = (s == 0) ? F1::first(load_elem<ESZ>(a.send[c] + b)) : P1::load(a.ws, i);
                const typename F1::A v = F1::add_acc(F1::first(load_elem<ESZ>(a.send[r] + b)), in);
                if (s < n - 2) {
                    P1::store(const_cast<char*>(a.ws), i, v);
                } else if (allreduce) {
                    store_unit_cached<DT, 1>(a.recv[owner] + b, 0u, F1::done(v, n));
                } else {
                    store_elem<ESZ>(shard + (i - sp.s) * ESZ, F1::done(v, n));
                }
                step_boundary();
            }
            if (allreduce) {
                for (int s = 0; s < n - 1; ++s) {
                    const int r = ring_rank(c, s, n);
                    const int p = ring_rank(r, n - 1, n);
                    store_unit_cached<DT, 1>(a.recv[r] + b, 0u, load_elem<ESZ>(a.recv[p] + b));
                    step_boundary();
                }
            }
        }
    }
    const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
    for (int s = 0; s < n - 1; ++s) {        // reduce-scatter, partials in the workspace
        const int r = ring_rank(c, s + 1, n);
        const char* tl = U::tile(a.send[r] - adj, tv0);
        const char* ts = UC::tile(a.send[c] - adj, tv0);
        typename U::T x[kUnroll];
        typename F::A y[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) {
                x[u] = U::load(tl, U::lane_off(u));
                y[u] = (s == 0) ? F::first(UC::load(ts, U::lane_off(u))) : P::load(ws_base, tv0 + U::lane_unit(u));
            }
        }
        char* to = allreduce ? U::tile(a.recv[owner] - adj, tv0) : nullptr;   // rank c-1's own chunk c
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!live[u]) continue;
            const typename F::A z = F::add_acc(F::first(x[u]), y[u]);
            if (s < n - 2) {
                P::store(const_cast<char*>(ws_base), tv0 + U::lane_unit(u), z);
            } else if (allreduce) {
                store_unit_cached<DT, VEC>(to, U::lane_off(u), F::done(z, n));
            } else {
                store_shard_unit<DT, VEC>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u), F::done(z, n));
            }
        }
        step_boundary();
    }
    if (allreduce) {
        for (int s = 0; s < n - 1; ++s) {    // all-gather
            const int r = ring_rank(c, s, n);
            const int p = ring_rank(r, n - 1, n);
            const char* ts = UC::tile(a.recv[p] - adj, tv0);
            typename U::T x[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) x[u] = UC::load(ts, U::lane_off(u));
            }
            char* td = U::tile(a.recv[r] - adj, tv0);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) store_unit_cached<DT, VEC>(td, U::lane_off(u), x[u]);
            }
            step_boundary();
        }
    }
    AR_TILE_LOOP_END
}

// The ring all-gather pipelined: shard c is placed at position start(c) of
// rank c, then copied from rank c+s to rank c+s+1 at step s (the standalone
// all-gather ring of ramchalamkr.github.io "NCCL Primitives Deep Dive",
// section "Ring All-Gather"), slice by slice.
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_pipelined_gather(const KernelArgs a) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    using UC = Unit<DT, VEC, false>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    const char* shard = a.send[c];
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            const uint64_t b = i * ESZ;
            char* first = a.recv[c] + b;
            const char* src = shard + (i - sp.s) * ESZ;
            if (first != src) store_unit_cached<DT, 1>(first, 0u, load_elem<ESZ>(src));
            step_boundary();
            for (int s = 0; s < n - 1; ++s) {
                const int p = ring_rank(c, s, n);
                const int r = ring_rank(c, s + 1, n);
                store_unit_cached<DT, 1>(a.recv[r] + b, 0u, load_elem<ESZ>(a.recv[p] + b));
                step_boundary();
            }
        }
    }
    {
        const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
        const bool in_place = a.recv[c] + sp.s * ESZ == shard;
        typename U::T x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) x[u] = load_shard_unit<DT, VEC, AR_NT_LOADS_COPY>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u));
        }
        if (!in_place) {
            char* td = U::tile(a.recv[c] - adj, tv0);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) store_unit_cached<DT, VEC>(td, U::lane_off(u), x[u]);
            }
        }
        step_boundary();
    }
    for (int s = 0; s < n - 1; ++s) {
        const int p = ring_rank(c, s, n);
        const int r = ring_rank(c, s + 1, n);
        const char* ts = UC::tile(a.recv[p] - adj, tv0);
        typename U::T x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) x[u] = UC::load(ts, U::lane_off(u));
        }
        char* td = U::tile(a.recv[r] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) store_unit_cached<DT, VEC>(td, U::lane_off(u), x[u]);
        }
        step_boundary();
    }
    AR_TILE_LOOP_END
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
hipError_t launch_cooperative(const Launch& l, const KernelArgs& a, hipStream_t s) {
    int resident = 0;
    hipError_t e = resident_blocks<DT, OP, VEC>(&resident);
    if (e != hipSuccess) return e;
    const unsigned blocks = l.blocks < static_cast<unsigned>(resident) ? l.blocks : static_cast<unsigned>(resident);
    KernelArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_ring_persistent<DT, OP, VEC>),
                                      dim3(blocks > 0 ? blocks : 1), dim3(kThreads), params, 0, s);
}

template <int DT, int OP, int VEC>
hipError_t launch_t(const Launch& l, const KernelArgs& a, hipStream_t s) {
    // the pipelined forms are ordinary launches: one block per slice
    if (l.kind == Kind::kRingPipelinedWs) {
        hipLaunchKernelGGL((k_ring_pipelined_ws<DT, OP, VEC>), dim3(l.blocks), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    if constexpr (acc_f32<DT>()) {
        return hipErrorInvalidValue;         // float32 partials need the workspace form
    } else {
        if (l.kind == Kind::kRingPipelined) {
            hipLaunchKernelGGL((k_ring_pipelined<DT, OP, VEC>), dim3(l.blocks), dim3(kThreads), 0, s, a);
            return hipGetLastError();
        }
        return launch_cooperative<DT, OP, VEC>(l, a, s);
    }
}

template <int DT>
hipError_t launch_gather(const Launch& l, const KernelArgs& a, hipStream_t s) {
    constexpr int V = 16 / elem_size<DT>();
    if (l.vec) {
        hipLaunchKernelGGL((k_ring_pipelined_gather<DT, V>), dim3(l.blocks), dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_ring_pipelined_gather<DT, 1>), dim3(l.blocks), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
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
    if (l.kind == Kind::kRingPersistent) {
        // Never inside a stream capture: a captured launch could replay without
        // the cooperative guarantees the grid barrier depends on.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess) return e;
        if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    } else if (l.kind == Kind::kRingPipelinedGather) {
        // copies move bit patterns: the 2-byte types as bf16, the 4-byte ones as float32
        const bool two_bytes = l.dtype == AR_BFLOAT16 || l.dtype == AR_FLOAT16 || l.dtype == AR_BFLOAT16_ACC_F32;
        return two_bytes ? launch_gather<AR_BFLOAT16>(l, a, stream) : launch_gather<AR_FLOAT32>(l, a, stream);
    } else if (l.kind != Kind::kRingPipelined && l.kind != Kind::kRingPipelinedWs) {
        return hipErrorInvalidValue;
    }
    switch (l.dtype) {
        case AR_FLOAT32: return by_op<AR_FLOAT32>(l, a, stream);
        case AR_BFLOAT16: return by_op<AR_BFLOAT16>(l, a, stream);
        case AR_INT32: return by_op<AR_INT32>(l, a, stream);
        case AR_FLOAT16: return by_op<AR_FLOAT16>(l, a, stream);
        case AR_BFLOAT16_ACC_F32: return by_op<AR_BFLOAT16_ACC_F32>(l, a, stream);   // workspace form only
    }
    return hipErrorInvalidValue;
}

}  // namespace arimpl
