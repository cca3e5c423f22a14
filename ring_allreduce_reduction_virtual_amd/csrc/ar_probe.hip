// HBM ceiling probes (gfx950), for measurement only: libarprobe.so, loaded
// by bench.py's --ceiling mode, never by the library or its binding.
//
// Each probe streams n buffers of nvec 16-byte vectors with the fused
// AllReduce's access pattern: one block of 256 threads per tile of 512
// vectors (8 KiB) of every buffer, two vectors per thread per buffer, loads
// and stores with the nontemporal hint.  What differs is only the direction
// of the traffic:
//   kind 0  read:  load all n buffers (n*S bytes read), keep an xor
//   kind 1  write: store all n destination buffers (n*S bytes written)
//   kind 2  copy:  buffer r to destination r (n*S read, n*S written)
//   kind 3  mix:   load the n buffers, add them as integers, store the sum to
//                  all n destinations: the AllReduce's traffic (n*S read,
//                  n*S written) with none of its chunk logic or float work
// so that the time of the read and write streams alone bounds the time of
// any kernel that moves the same bytes.
//
// extern "C" int arprobe_stream(int kind, const void* const* src,
//     void* const* dst, int n, uint64_t nvec, void* sink, hipStream_t s)
//   src, dst: n device pointers each, 16-byte aligned, nvec vectors long
//   (dst unused by kind 0, src by kind 1); sink: 16 bytes of device memory
//   (kind 0 writes it only if the xor of everything read hits one fixed
//   value, which keeps the loads alive); n in [1, 128]; nvec a multiple of
//   512.  Returns 0 on success, 1 for bad arguments, 2 for a launch error.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeMax = 128;   // two tables of 128 pointers: 2 KiB of kernel arguments
constexpr int kThreads = 256;
constexpr int kPerThread = 2;
constexpr uint64_t kTile = kThreads * kPerThread;   // vectors per buffer per block

struct Table {
    const u32x4* src[kProbeMax];
    u32x4* dst[kProbeMax];
    int n;
};

__device__ __forceinline__ u32x4 ld(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__global__ __launch_bounds__(kThreads) void k_read(const Table t, u32x4* sink) {
    const uint64_t v0 = blockIdx.x * kTile + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int r = 0; r < t.n; ++r) {
        acc ^= ld(t.src[r] + v0);
        acc ^= ld(t.src[r] + v0 + kThreads);
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) *sink = acc;
}

__global__ __launch_bounds__(kThreads) void k_write(const Table t) {
    const uint64_t v0 = blockIdx.x * kTile + threadIdx.x;
    const u32x4 v = {static_cast<uint32_t>(v0), 1u, 2u, 3u};
    for (int r = 0; r < t.n; ++r) {
        st(t.dst[r] + v0, v);
        st(t.dst[r] + v0 + kThreads, v);
    }
}

__global__ __launch_bounds__(kThreads) void k_copy(const Table t) {
    const uint64_t v0 = blockIdx.x * kTile + threadIdx.x;
    for (int r = 0; r < t.n; ++r) {
        const u32x4 a = ld(t.src[r] + v0);
        const u32x4 b = ld(t.src[r] + v0 + kThreads);
        st(t.dst[r] + v0, a);
        st(t.dst[r] + v0 + kThreads, b);
    }
}

__global__ __launch_bounds__(kThreads) void k_mix(const Table t) {
    const uint64_t v0 = blockIdx.x * kTile + threadIdx.x;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    for (int r = 0; r < t.n; r += 8) {          // eight buffers' loads in flight, as the AllReduce
        u32x4 x[8], y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (r + j < t.n) {
                x[j] = ld(t.src[r + j] + v0);
                y[j] = ld(t.src[r + j] + v0 + kThreads);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (r + j < t.n) {
                a += x[j];
                b += y[j];
            }
        }
    }
    for (int r = 0; r < t.n; ++r) {
        st(t.dst[r] + v0, a);
        st(t.dst[r] + v0 + kThreads, b);
    }
}

}  // namespace

extern "C" int arprobe_stream(int kind, const void* const* src, void* const* dst, int n, uint64_t nvec, void* sink,
                              hipStream_t s) {
    if (n < 1 || n > kProbeMax || nvec == 0 || nvec % kTile != 0 || nvec / kTile > 0x7fffffffull) return 1;
    if (kind < 0 || kind > 3) return 1;
    Table t{};
    t.n = n;
    for (int r = 0; r < n; ++r) {
        if (kind != 1) {
            if (src == nullptr || src[r] == nullptr || reinterpret_cast<uintptr_t>(src[r]) % 16 != 0) return 1;
            t.src[r] = static_cast<const u32x4*>(src[r]);
        }
        if (kind != 0) {
            if (dst == nullptr || dst[r] == nullptr || reinterpret_cast<uintptr_t>(dst[r]) % 16 != 0) return 1;
            t.dst[r] = static_cast<u32x4*>(dst[r]);
        }
    }
    if (kind == 0 && sink == nullptr) return 1;
    const dim3 grid(static_cast<unsigned>(nvec / kTile)), block(kThreads);
    switch (kind) {
        case 0: hipLaunchKernelGGL(k_read, grid, block, 0, s, t, static_cast<u32x4*>(sink)); break;
        case 1: hipLaunchKernelGGL(k_write, grid, block, 0, s, t); break;
        case 2: hipLaunchKernelGGL(k_copy, grid, block, 0, s, t); break;
        default: hipLaunchKernelGGL(k_mix, grid, block, 0, s, t); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
