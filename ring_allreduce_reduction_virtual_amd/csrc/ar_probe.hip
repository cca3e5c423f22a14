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

// Patterned streams: each block moves one contiguous run of `run` vectors of
// ONE buffer, so a wave reads or writes long stretches of a single buffer.
// order 0 (buffer-major): consecutive blocks walk buffer 0's runs, then
// buffer 1's; order 1 (tile-major): consecutive blocks take run j of
// buffers 0, 1, ..., n-1 in turn.  Each thread moves 4 vectors per pass of
// the block over its run (16 KiB per block per pass).  Block b's run lies in
// [0, nvec) of one buffer by construction: runs = nvec / run, blocks = n * runs.
template <bool WRITE, bool NT>
__global__ __launch_bounds__(kThreads) void k_pattern(const Table t, uint64_t run, uint64_t runs, int order,
                                                      u32x4* sink) {
    const uint64_t b = blockIdx.x;
    const int q = order == 0 ? static_cast<int>(b / runs) : static_cast<int>(b % static_cast<uint64_t>(t.n));
    const uint64_t j = order == 0 ? b % runs : b / static_cast<uint64_t>(t.n);
    const uint64_t first = j * run;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const u32x4 v = {static_cast<uint32_t>(b), 1u, 2u, 3u};
    for (uint64_t k = threadIdx.x; k < run; k += 4 * kThreads) {
        if constexpr (WRITE) {
            u32x4* d = t.dst[q] + first + k;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (k + u * kThreads < run) {
                    if constexpr (NT) {
                        st(d + u * kThreads, v);
                    } else {
                        d[u * kThreads] = v;
                    }
                }
            }
        } else {
            const u32x4* p = t.src[q] + first + k;
            u32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (k + u * kThreads < run) x[u] = NT ? ld(p + u * kThreads) : p[u * kThreads];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (k + u * kThreads < run) acc ^= x[u];
            }
        }
    }
    if constexpr (!WRITE) {
        if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) *sink = acc;
    }
}

// The kernels' write pattern with plain (cache-allocating) stores: k_write
// without the nontemporal hint.
__global__ __launch_bounds__(kThreads) void k_write_plain(const Table t) {
    const uint64_t v0 = blockIdx.x * kTile + threadIdx.x;
    const u32x4 v = {static_cast<uint32_t>(v0), 1u, 2u, 3u};
    for (int r = 0; r < t.n; ++r) {
        t.dst[r][v0] = v;
        t.dst[r][v0 + kThreads] = v;
    }
}

// Writes in which XCD x (workgroups are handed to MI355X's 8 XCDs in turn,
// block b to XCD b mod 8) writes buffer x only: block b writes tile b / 8
// (8 KiB) of buffer b mod 8, and blocks whose b mod 8 >= n do nothing, so
// with n < 8 some XCDs idle.  Grid: 8 * tiles blocks.
__global__ __launch_bounds__(kThreads) void k_xcd_write(const Table t) {
    const uint64_t b = blockIdx.x;
    const int x = static_cast<int>(b % 8);
    if (x >= t.n) return;
    const uint64_t v0 = (b / 8) * kTile + threadIdx.x;
    const u32x4 v = {static_cast<uint32_t>(b), 1u, 2u, 3u};
    t.dst[x][v0] = v;
    t.dst[x][v0 + kThreads] = v;
}

// Broadcast shapes: src (one buffer, just written) copied to n destinations.
// mode 0: one block per 8 KiB tile, loading it once and storing it to every
//   destination (the staged broadcast's shape);
// mode 1: XCD x copies to destination x only: block b copies tile b / 8 of
//   src to destination b mod 8 (blocks with b mod 8 >= n idle), so each tile
//   is loaded by n blocks on n XCDs.  Grid: 8 * tiles blocks.
// Plain loads (the source sits in the last-level cache) and plain stores.
__global__ __launch_bounds__(kThreads) void k_bcast(const Table t, int mode) {
    const uint64_t b = blockIdx.x;
    if (mode == 0) {
        const uint64_t v0 = b * kTile + threadIdx.x;
        const u32x4 a = t.src[0][v0], c = t.src[0][v0 + kThreads];
        for (int q = 0; q < t.n; ++q) {
            t.dst[q][v0] = a;
            t.dst[q][v0 + kThreads] = c;
        }
        return;
    }
    const int x = static_cast<int>(b % 8);
    if (x >= t.n) return;
    const uint64_t v0 = (b / 8) * kTile + threadIdx.x;
    const u32x4 a = t.src[0][v0], c = t.src[0][v0 + kThreads];
    t.dst[x][v0] = a;
    t.dst[x][v0 + kThreads] = c;
}

// Copies of n buffers (src[q] -> dst[q], 8 KiB per workgroup) in the block
// orders of k_pattern: order 0 buffer-major, 1 tile-major.  Nontemporal loads;
// stores nontemporal (nt) or plain.  Grid: n * tiles blocks.
template <bool NT>
__global__ __launch_bounds__(kThreads) void k_copy_order(const Table t, uint64_t tiles, int order) {
    const uint64_t b = blockIdx.x;
    const int q = order == 0 ? static_cast<int>(b / tiles) : static_cast<int>(b % static_cast<uint64_t>(t.n));
    const uint64_t j = order == 0 ? b % tiles : b / static_cast<uint64_t>(t.n);
    const uint64_t v0 = j * kTile + threadIdx.x;
    const u32x4 a = ld(t.src[q] + v0), c = ld(t.src[q] + v0 + kThreads);
    if constexpr (NT) {
        st(t.dst[q] + v0, a);
        st(t.dst[q] + v0 + kThreads, c);
    } else {
        t.dst[q][v0] = a;
        t.dst[q][v0 + kThreads] = c;
    }
}

// Writes of n buffers, one 8 KiB tile per workgroup, in one of five
// workgroup -> (buffer, tile) maps (T tiles per buffer; workgroups are dealt
// to the 8 XCDs in turn, so workgroup b runs on XCD b mod 8):
//   0 grouped per XCD as the staged broadcast: b = x + 8m -> tile
//     8 floor(m / n) + x, buffer m mod n (a tile's n workgroups on XCD x);
//   1 tile-major: buffer b mod n, tile floor(b / n);
//   2 buffer-major: buffer floor(b / T), tile b mod T;
//   3 one contiguous range per XCD of the n*T (buffer, tile) units taken
//     buffer-major: XCD x writes units [x nT/8, (x+1) nT/8) in order;
//   4 the same with the units taken tile-major (each XCD a contiguous range
//     of tiles, every buffer);
//   5, 6, 7 each XCD a contiguous eighth of the tiles (T a multiple of 8K),
//     walked in sub-ranges of K = 16, 64, 256 tiles, each sub-range buffer by
//     buffer: runs of K tiles per buffer, and a sub-range's source tiles
//     (K x 8 KiB) reread from that XCD's L2 for every buffer after the first.
// SRC: each workgroup first loads its tile from src[0] (cache-allocating
// loads), as a broadcast does, else stores a constant.  Grid: n*T for maps 1
// and 2, 8 ceil(T/8) n for map 0, 8 ceil(nT/8) for maps 3 and 4; workgroups
// beyond the units write nothing; maps 5-7 use n*T workgroups.
template <bool SRC>
__global__ __launch_bounds__(kThreads) void k_wmap(const Table t, uint64_t tiles, int map) {
    const uint64_t n = static_cast<uint64_t>(t.n), b = blockIdx.x;
    uint64_t buf, tile;
    if (map == 1) {
        buf = b % n;
        tile = b / n;
    } else if (map == 2) {
        buf = b / tiles;
        tile = b % tiles;
    } else if (map == 0) {
        const uint64_t x = b & 7u, m = b >> 3;
        tile = 8 * (m / n) + x;
        buf = m % n;
    } else if (map <= 4) {
        const uint64_t units = n * tiles, x = b & 7u, m = b >> 3;
        const uint64_t u = units * x / 8 + m;
        if (u >= units * (x + 1) / 8) return;
        buf = map == 3 ? u / tiles : u % n;
        tile = map == 3 ? u % tiles : u / n;
    } else {
        const uint64_t k = map == 5 ? 16 : (map == 6 ? 64 : 256);
        const uint64_t per = tiles / 8, x = b & 7u, m = b >> 3;
        const uint64_t j = m / (n * k), r = m % (n * k);
        buf = r / k;
        tile = x * per + j * k + r % k;
        if (j * k + r % k >= per) return;
    }
    if (buf >= n || tile >= tiles) return;
    const uint64_t v0 = tile * kTile + threadIdx.x;
    u32x4 a, c;
    if constexpr (SRC) {
        a = t.src[0][v0];
        c = t.src[0][v0 + kThreads];
    } else {
        a = u32x4{static_cast<uint32_t>(v0), 1u, 2u, 3u};
        c = a;
    }
    st(t.dst[buf] + v0, a);
    st(t.dst[buf] + v0 + kThreads, c);
}

}  // namespace

// extern "C" int arprobe_copy_order(int order, int nt, const void* const* src,
//     void* const* dst, int n, uint64_t nvec, hipStream_t s)
//   k_copy_order over n buffers of nvec vectors (a multiple of 512).
//   Returns 0, 1 (bad arguments) or 2 (launch error).
extern "C" int arprobe_copy_order(int order, int nt, const void* const* src, void* const* dst, int n, uint64_t nvec,
                                  hipStream_t s) {
    if (n < 1 || n > kProbeMax || nvec == 0 || nvec % kTile != 0 || src == nullptr || dst == nullptr) return 1;
    if (order != 0 && order != 1) return 1;
    const uint64_t tiles = nvec / kTile;
    if (tiles * static_cast<uint64_t>(n) > 0x7fffffffull) return 1;
    Table t{};
    t.n = n;
    for (int r = 0; r < n; ++r) {
        if (src[r] == nullptr || dst[r] == nullptr || reinterpret_cast<uintptr_t>(src[r]) % 16 != 0 ||
            reinterpret_cast<uintptr_t>(dst[r]) % 16 != 0)
            return 1;
        t.src[r] = static_cast<const u32x4*>(src[r]);
        t.dst[r] = static_cast<u32x4*>(dst[r]);
    }
    const dim3 grid(static_cast<unsigned>(tiles * static_cast<uint64_t>(n))), block(kThreads);
    if (nt) hipLaunchKernelGGL((k_copy_order<true>), grid, block, 0, s, t, tiles, order);
    else hipLaunchKernelGGL((k_copy_order<false>), grid, block, 0, s, t, tiles, order);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// extern "C" int arprobe_xcd(int kind, const void* src, void* const* dst, int n,
//     uint64_t nvec, hipStream_t s)
//   kind 0: k_xcd_write over the n (<= 8) buffers dst of nvec vectors;
//   kind 1, 2: k_bcast mode 0, 1 from src (nvec vectors) to the n (<= 8)
//   destinations.  nvec a multiple of 512.  Returns 0, 1 (bad arguments) or 2.
extern "C" int arprobe_xcd(int kind, const void* src, void* const* dst, int n, uint64_t nvec, hipStream_t s) {
    if (n < 1 || n > 8 || nvec == 0 || nvec % kTile != 0 || nvec / kTile > 0x0fffffffull || dst == nullptr) return 1;
    if (kind < 0 || kind > 2 || (kind > 0 && (src == nullptr || reinterpret_cast<uintptr_t>(src) % 16 != 0))) return 1;
    Table t{};
    t.n = n;
    t.src[0] = static_cast<const u32x4*>(src);
    for (int r = 0; r < n; ++r) {
        if (dst[r] == nullptr || reinterpret_cast<uintptr_t>(dst[r]) % 16 != 0) return 1;
        t.dst[r] = static_cast<u32x4*>(dst[r]);
    }
    const uint64_t tiles = nvec / kTile;
    const dim3 block(kThreads);
    if (kind == 0) hipLaunchKernelGGL(k_xcd_write, dim3(static_cast<unsigned>(8 * tiles)), block, 0, s, t);
    else if (kind == 1) hipLaunchKernelGGL(k_bcast, dim3(static_cast<unsigned>(tiles)), block, 0, s, t, 0);
    else hipLaunchKernelGGL(k_bcast, dim3(static_cast<unsigned>(8 * tiles)), block, 0, s, t, 1);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// extern "C" int arprobe_pattern(int write, int nt, int order, uint64_t run,
//     const void* const* bufs, int n, uint64_t nvec, void* sink, hipStream_t s)
//   One patterned stream (k_pattern) over n buffers of nvec 16-byte vectors:
//   write != 0 stores, else loads (sink as for arprobe_stream); nt picks the
//   nontemporal hint; order 0 buffer-major, 1 tile-major; run vectors per
//   block, a divisor of nvec.  With run == 0 it is the kernels' own write
//   pattern with plain stores (k_write_plain; nvec a multiple of 512).
//   Returns 0 on success, 1 for bad arguments, 2 for a launch error.
extern "C" int arprobe_pattern(int write, int nt, int order, uint64_t run, const void* const* bufs, int n,
                               uint64_t nvec, void* sink, hipStream_t s) {
    if (n < 1 || n > kProbeMax || nvec == 0 || bufs == nullptr || (order != 0 && order != 1)) return 1;
    Table t{};
    t.n = n;
    for (int r = 0; r < n; ++r) {
        if (bufs[r] == nullptr || reinterpret_cast<uintptr_t>(bufs[r]) % 16 != 0) return 1;
        t.src[r] = static_cast<const u32x4*>(bufs[r]);
        t.dst[r] = static_cast<u32x4*>(const_cast<void*>(bufs[r]));
    }
    const dim3 block(kThreads);
    if (run == 0) {
        if (!write || nvec % kTile != 0 || nvec / kTile > 0x7fffffffull) return 1;
        hipLaunchKernelGGL(k_write_plain, dim3(static_cast<unsigned>(nvec / kTile)), block, 0, s, t);
        return hipGetLastError() == hipSuccess ? 0 : 2;
    }
    if (nvec % run != 0) return 1;
    const uint64_t runs = nvec / run;
    const uint64_t blocks = runs * static_cast<uint64_t>(n);
    if (blocks > 0x7fffffffull || (!write && sink == nullptr)) return 1;
    const dim3 grid(static_cast<unsigned>(blocks));
    u32x4* sk = static_cast<u32x4*>(sink);
    if (write) {
        if (nt) hipLaunchKernelGGL((k_pattern<true, true>), grid, block, 0, s, t, run, runs, order, sk);
        else hipLaunchKernelGGL((k_pattern<true, false>), grid, block, 0, s, t, run, runs, order, sk);
    } else {
        if (nt) hipLaunchKernelGGL((k_pattern<false, true>), grid, block, 0, s, t, run, runs, order, sk);
        else hipLaunchKernelGGL((k_pattern<false, false>), grid, block, 0, s, t, run, runs, order, sk);
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

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

// extern "C" int arprobe_wmap(int map, const void* src, void* const* dst,
//     int n, uint64_t nvec, hipStream_t s)
//   k_wmap over the n (<= 8) destinations dst of nvec vectors (a multiple of
//   512), in map 0-7; src (nvec vectors) loaded by each workgroup first, or
//   nullptr for writes alone.  Returns 0, 1 (bad arguments) or 2.
extern "C" int arprobe_wmap(int map, const void* src, void* const* dst, int n, uint64_t nvec, hipStream_t s) {
    if (n < 1 || n > 8 || nvec == 0 || nvec % kTile != 0 || dst == nullptr || map < 0 || map > 7) return 1;
    if (src != nullptr && reinterpret_cast<uintptr_t>(src) % 16 != 0) return 1;
    const uint64_t tiles = nvec / kTile;
    const uint64_t un = static_cast<uint64_t>(n);
    if (map >= 5 && tiles % (8 * (map == 5 ? 16u : (map == 6 ? 64u : 256u))) != 0) return 1;
    const uint64_t blocks = map == 0 ? 8 * ((tiles + 7) / 8) * un
                            : (map <= 2 || map >= 5 ? un * tiles : 8 * ((un * tiles + 7) / 8));
    if (blocks > 0x7fffffffull) return 1;
    Table t{};
    t.n = n;
    t.src[0] = static_cast<const u32x4*>(src);
    for (int r = 0; r < n; ++r) {
        if (dst[r] == nullptr || reinterpret_cast<uintptr_t>(dst[r]) % 16 != 0) return 1;
        t.dst[r] = static_cast<u32x4*>(dst[r]);
    }
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    if (src != nullptr) hipLaunchKernelGGL((k_wmap<true>), grid, block, 0, s, t, tiles, map);
    else hipLaunchKernelGGL((k_wmap<false>), grid, block, 0, s, t, tiles, map);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
