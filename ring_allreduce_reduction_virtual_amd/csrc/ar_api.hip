// Host side of libar.so: the C ABI declared in include/ar.h.
//
// Each entry point validates everything first (so an error launches
// nothing), plans the launch (vector or element path, tiles per chunk, grid)
// and enqueues kernels from ar_kernels.hip on the caller's stream.  No state
// is kept between calls apart from a per-device cache of the compute-unit
// count and the calling thread's last error text.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <string>
#include <vector>

#include "ar.h"
#include "ar_internal.h"

using arimpl::Kind;
using arimpl::KernelArgs;
using arimpl::Launch;

namespace {

thread_local std::string g_detail;

ar_result_t fail(ar_result_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_detail = buf;
    return code;
}

bool debug_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("AR_DEBUG");
        return v != nullptr && v[0] != '\0' && v[0] != '0';
    }();
    return on;
}

// Blocks launched per compute unit; 0 (the default, fastest when measured on
// MI355X) launches one block per tile, a positive value caps the grid at that
// many blocks per CU and the kernels stride over the tiles.
// AR_BLOCKS_PER_CU overrides the default.
unsigned blocks_per_cu() {
    static const unsigned v = [] {
        const char* e = std::getenv("AR_BLOCKS_PER_CU");
        if (e != nullptr && e[0] != '\0') return static_cast<unsigned>(std::strtoul(e, nullptr, 10));
        return 0u;
    }();
    return v;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

ar_result_t cu_count(int* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(AR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *out = cached;
            return AR_SUCCESS;
        }
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(AR_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    if (cus <= 0) cus = 1;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
    *out = cus;
    return AR_SUCCESS;
}

size_t esize(ar_dtype_t dt) {
    switch (dt) {
        case AR_FLOAT32: return 4;
        case AR_BFLOAT16: return 2;
        case AR_INT32: return 4;
        case AR_FLOAT16: return 2;
        case AR_BFLOAT16_ACC_F32: return 2;
    }
    return 0;
}

// Bytes of one partial sum between ring steps: float32 for AR_BFLOAT16_ACC_F32.
size_t partial_size(ar_dtype_t dt) { return dt == AR_BFLOAT16_ACC_F32 ? 4 : esize(dt); }

const char* dtype_name(ar_dtype_t dt) {
    switch (dt) {
        case AR_FLOAT32: return "f32";
        case AR_BFLOAT16: return "bf16";
        case AR_INT32: return "i32";
        case AR_FLOAT16: return "f16";
        case AR_BFLOAT16_ACC_F32: return "bf16acc32";
    }
    return "?";
}

// Chunk bounds in 64-bit integers; c*count cannot overflow because count is
// validated to be below 2^64 / AR_MAX_RANKS.
inline uint64_t chunk_start(int c, uint64_t count, int n) {
    return static_cast<uint64_t>(c) * count / static_cast<uint64_t>(n);
}

struct Interval {
    uintptr_t lo, hi;
    bool writable;
    int rank;
    int role;   // 0 send, 1 recv, 2 workspace
};

// Reject overlaps other than read-only buffers overlapping each other and the
// exact in-place layouts the collective allows (checked by the caller and
// passed in as `allowed(send_rank, recv_rank)`).
template <typename Allowed>
ar_result_t check_overlaps(std::vector<Interval>& v, Allowed allowed) {
    std::sort(v.begin(), v.end(), [](const Interval& a, const Interval& b) { return a.lo < b.lo; });
    std::vector<const Interval*> active;
    for (const Interval& cur : v) {
        active.erase(std::remove_if(active.begin(), active.end(),
                                    [&](const Interval* x) { return x->hi <= cur.lo; }),
                     active.end());
        for (const Interval* x : active) {
            if (!x->writable && !cur.writable) continue;
            const Interval* s = x->role == 0 ? x : (cur.role == 0 ? &cur : nullptr);
            const Interval* r = x->role == 1 ? x : (cur.role == 1 ? &cur : nullptr);
            if (s != nullptr && r != nullptr && s != r && allowed(*s, *r)) continue;
            static const char* names[] = {"sendbufs", "recvbufs", "workspace"};
            return fail(AR_ERR_INVALID_ARGUMENT, "%s[%d] overlaps %s[%d]", names[x->role], x->rank,
                        names[cur.role], cur.rank);
        }
        active.push_back(&cur);
    }
    return AR_SUCCESS;
}

// Where each buffer lives, checked once when a plan is made (two runtime
// queries per buffer would cost the one-shot calls as much as a small
// collective): device memory of the current device or managed memory, ending
// inside its allocation.  Plain and pinned host memory, another device's
// memory and a buffer that runs past its allocation are refused, so that a
// plan never sends a kernel to an address it cannot reach.
ar_result_t check_residency(const std::vector<Interval>& iv) {
    if (iv.empty()) return AR_SUCCESS;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(AR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    static const char* names[] = {"sendbufs", "recvbufs", "workspace"};
    for (const Interval& b : iv) {
        char what[32];
        if (b.role == 2)
            std::snprintf(what, sizeof(what), "workspace");
        else
            std::snprintf(what, sizeof(what), "%s[%d]", names[b.role], b.rank);
        void* p = reinterpret_cast<void*>(b.lo);
        hipPointerAttribute_t at{};
        e = hipPointerGetAttributes(&at, p);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // the launches read the last error: leave none behind
            return fail(AR_ERR_INVALID_ARGUMENT, "%s: the HIP runtime does not know this address (%s)", what,
                        hipGetErrorString(e));
        }
        if (at.type == hipMemoryTypeUnregistered || at.type == hipMemoryTypeHost)
            return fail(AR_ERR_INVALID_ARGUMENT, "%s is host memory, not device memory", what);
        if (at.type == hipMemoryTypeDevice && at.device != dev)
            return fail(AR_ERR_INVALID_ARGUMENT, "%s is memory of device %d, not of the current device %d", what,
                        at.device, dev);
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        e = hipMemGetAddressRange(&base, &size, p);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // extent unknown to the runtime: not checked
            continue;
        }
        const uintptr_t end = reinterpret_cast<uintptr_t>(base) + size;
        if (b.hi > end)
            return fail(AR_ERR_INVALID_ARGUMENT, "%s runs %llu bytes past the end of its allocation", what,
                        static_cast<unsigned long long>(b.hi - end));
    }
    return AR_SUCCESS;
}

struct Common {
    const void* const* send;
    void* const* recv;
    uint64_t count;
    ar_dtype_t dtype;
    ar_op_t op;
    int n;
    size_t esz;
};

ar_result_t check_common(const Common& k, bool has_op) {
    g_detail.clear();
    if (k.esz == 0) return fail(AR_ERR_INVALID_ARGUMENT, "unknown dtype %d", static_cast<int>(k.dtype));
    if (has_op && (k.op < AR_SUM || k.op > AR_AVG)) return fail(AR_ERR_INVALID_ARGUMENT, "unknown op %d", static_cast<int>(k.op));
    if (k.n < 1 || k.n > AR_MAX_RANKS) return fail(AR_ERR_INVALID_ARGUMENT, "nranks %d outside [1, %d]", k.n, AR_MAX_RANKS);
    if (k.send == nullptr || k.recv == nullptr) return fail(AR_ERR_INVALID_ARGUMENT, "null pointer array");
    if (k.count > (UINT64_MAX / AR_MAX_RANKS) / 16) return fail(AR_ERR_INVALID_ARGUMENT, "count %llu too large",
                                                               static_cast<unsigned long long>(k.count));
    return AR_SUCCESS;
}

// Bytes a buffer of `elems` elements spans; null is allowed only when empty.
ar_result_t check_ptr(const void* p, uint64_t elems, size_t esz, const char* what, int r) {
    if (elems == 0) return AR_SUCCESS;
    if (p == nullptr) return fail(AR_ERR_INVALID_ARGUMENT, "%s[%d] is null", what, r);
    if (reinterpret_cast<uintptr_t>(p) % esz != 0)
        return fail(AR_ERR_INVALID_ARGUMENT, "%s[%d] not aligned to its %zu-byte element", what, r, esz);
    return AR_SUCCESS;
}

// Streamed buffers share their address residue modulo `align` bytes.  The
// vector path needs 16; 256 lets every chunk body start and end on whole
// cache lines in all buffers at once.
struct Residue {
    int bytes;    // common residue modulo `align`, or -1 when not even 16 works
    int align;    // 256, 128, 64, 32 or 16
};

Residue common_residue(const std::vector<uintptr_t>& ptrs) {
    for (int align = 256; align >= 16; align /= 2) {
        const uintptr_t m = static_cast<uintptr_t>(align - 1);
        const uintptr_t r0 = ptrs.empty() ? 0 : (ptrs[0] & m);
        bool same = true;
        for (uintptr_t p : ptrs) same = same && ((p & m) == r0);
        if (same) return {static_cast<int>(r0), align};
    }
    return {-1, 16};
}

void fill_tables(KernelArgs& a, const Common& k) {
    for (int r = 0; r < k.n; ++r) {
        a.send[r] = static_cast<const char*>(k.send[r]);
        a.recv[r] = static_cast<char*>(k.recv[r]);
    }
    a.count = k.count;
    a.count_q = k.count / static_cast<uint64_t>(k.n);
    a.count_r = static_cast<uint32_t>(k.count % static_cast<uint64_t>(k.n));
    a.nranks = k.n;
    a.step = 0;
    a.shift = 0;
    a.ofs = 0;
    a.ws = nullptr;
}

// Grid for the tiles [tile_first, tile_end) of a launch.
ar_result_t grid_for(const KernelArgs& a, Launch& l, unsigned blocks_per_tile = 1) {
    int cus = 0;
    const ar_result_t rc = cu_count(&cus);
    if (rc != AR_SUCCESS) return rc;
    const uint64_t tiles = static_cast<uint64_t>(a.tile_end - a.tile_first) * blocks_per_tile;
    const unsigned bpc = blocks_per_cu();
    const uint64_t blocks = bpc == 0 ? tiles : std::min<uint64_t>(tiles, static_cast<uint64_t>(cus) * bpc);
    // the kernels stride over what one grid (at most 2^31 - 1 blocks) leaves
    l.blocks = static_cast<unsigned>(std::min<uint64_t>(std::max<uint64_t>(blocks, 1), 0x7fffffffu));
    return AR_SUCCESS;
}

// Tiles per chunk and grid size for a launch on the current device.  The
// buffer is cut into `parts` floor parts (0: one per rank, the ring's chunks).
ar_result_t plan(KernelArgs& a, Launch& l, const Common& k, Residue res, int parts = 0) {
    const int np = parts > 0 ? parts : k.n;
    l.vec = res.bytes >= 0;
    const uint64_t block = l.vec ? static_cast<uint64_t>(res.align) / k.esz : 1;   // A elements
    a.ofs = l.vec ? static_cast<int32_t>(res.bytes / static_cast<int>(k.esz)) : 0;
    int shift = 0;
    while ((1ull << shift) < block) ++shift;
    a.align_shift = shift;
    const uint64_t n = static_cast<uint64_t>(np);
    // the largest chunk body in units (16-byte vectors or elements), as the
    // kernels count it: whole aligned blocks of A elements inside [start, end)
    const uint64_t per_unit = l.vec ? 16 / k.esz : 1;
    const uint64_t ofs = static_cast<uint64_t>(a.ofs);
    uint64_t units = 0;
    for (int c = 0; c < np; ++c) {
        const uint64_t s = chunk_start(c, k.count, np), e = chunk_start(c + 1, k.count, np);
        const uint64_t fb = (s + ofs + block - 1) / block, eb = (e + ofs) / block;
        units = std::max(units, eb > fb ? (eb - fb) * block / per_unit : 0);
    }
    const uint64_t tile_units = static_cast<uint64_t>(arimpl::kThreads) * arimpl::kUnroll;
    const uint64_t tpc = std::max<uint64_t>(1, (units + tile_units - 1) / tile_units);
    const uint64_t tiles = n * tpc;
    if (tiles > 0x7fffffffu) return fail(AR_ERR_INVALID_ARGUMENT, "buffer too large for one launch");
    a.tiles_per_chunk = static_cast<uint32_t>(tpc);
    a.tile_first = 0;
    a.tile_end = static_cast<uint32_t>(tiles);
    return grid_for(a, l);
}

bool algo_known(ar_algo_t algo) {
    return algo >= AR_ALGO_FUSED && algo <= AR_ALGO_DOUBLE_BINARY_TREE_STEPS;
}

// The double binary tree, fused or level by level.
bool dbt_algo(ar_algo_t algo) {
    return algo == AR_ALGO_DOUBLE_BINARY_TREE || algo == AR_ALGO_DOUBLE_BINARY_TREE_STEPS;
}

// AllReduce-only algorithms: the tree orders, the persistent ring, the
// staged reduce-then-broadcast and the double binary tree.
bool allreduce_only_algo(ar_algo_t algo) {
    return (algo >= AR_ALGO_TREE && algo <= AR_ALGO_HALVING_DOUBLING_STEPS) || algo == AR_ALGO_RING_PERSISTENT ||
           algo == AR_ALGO_STAGED || dbt_algo(algo);
}

// The ring's own schedule, step by step: launched per step or pipelined in one launch.
bool ring_steps_algo(ar_algo_t algo) { return algo == AR_ALGO_RING || algo == AR_ALGO_RING_PIPELINED; }

// The AllReduce-only algorithms that bracket the reduction as a tree.
bool tree_algo(ar_algo_t algo) { return algo >= AR_ALGO_TREE && algo <= AR_ALGO_HALVING_DOUBLING_STEPS; }

// The tree algorithms that run stage by stage (and keep partials between stages).
bool tree_steps_algo(ar_algo_t algo) {
    return algo == AR_ALGO_TREE_STEPS || algo == AR_ALGO_RECURSIVE_DOUBLING || algo == AR_ALGO_HALVING_DOUBLING_STEPS ||
           algo == AR_ALGO_DOUBLE_BINARY_TREE_STEPS;
}

// The ones defined for a power-of-two number of ranks only.
bool power_of_two_algo(ar_algo_t algo) {
    return algo == AR_ALGO_RECURSIVE_DOUBLING || algo == AR_ALGO_HALVING_DOUBLING ||
           algo == AR_ALGO_HALVING_DOUBLING_STEPS;
}

int ceil_log2(int n) {
    int l = 0;
    while ((1 << l) < n) ++l;
    return l;
}

// r with its low `bits` bits in reverse order.
int bit_reverse(int r, int bits) {
    int v = 0;
    for (int b = 0; b < bits; ++b) v |= ((r >> b) & 1) << (bits - 1 - b);
    return v;
}

// When a one-pass AllReduce uses the small-message kernels (all ranks'
// values of a few positions staged in LDS) instead of the tiled ones: at most
// AR_SMALL_COUNT_MAX_DEFAULT elements per rank, and, in all ranks together,
// at most AR_SMALL_WORK_MAX elements for the ring's order and
// AR_SMALL_TREE_WORK_MAX bytes for the tree orders (binomial tree,
// halving/doubling, double binary tree).  A block takes kThreads / N
// positions, so the small kernels' cost grows with N * count where the tiled
// kernels' grows with count.  The ring's left fold adds N - 1 dependent steps
// per position, each with a conversion for bf16, so its bound counts
// elements; the trees' levels number only log2 N, and their bound counts
// bytes.  Measured on MI355X, per call in a graph, small / tiled: the bounds
// are the crossovers from 2 to 128 ranks (ring order: 32 x 2^16 f32 9.6 /
// 10.8 us, 64 x 2^16 f32 18.0 / 17.1, 64 x 2^16 bf16 23.4 / 19.4; tree: 64 x
// 2^16 bf16 19.9 / 22.8, 128 x 2^15 f32 42.3 / 35.4 and 32.7 / 36.3 on two
// machines, 128 x 2^14 f32 15.6 / 33.0).
#ifndef AR_SMALL_COUNT_MAX_DEFAULT
#define AR_SMALL_COUNT_MAX_DEFAULT (1ull << 16)
#endif
#ifndef AR_SMALL_WORK_MAX
#define AR_SMALL_WORK_MAX (1ull << 21)
#endif
#ifndef AR_SMALL_TREE_WORK_MAX
#define AR_SMALL_TREE_WORK_MAX (8ull << 20)
#endif

// Each bound read once per process from its environment variable, else the default.
uint64_t env_bound(const char* name, uint64_t fallback) {
    const char* e = std::getenv(name);
    if (e != nullptr && e[0] != '\0') return static_cast<uint64_t>(std::strtoull(e, nullptr, 10));
    return fallback;
}

// Elements per rank; AR_SMALL_COUNT_MAX overrides it, 0 turns every
// small-message kernel off.
uint64_t small_count_max() {
    static const uint64_t v = env_bound("AR_SMALL_COUNT_MAX", AR_SMALL_COUNT_MAX_DEFAULT);
    return v;
}

bool small_message(const Common& k) {
    static const uint64_t work = env_bound("AR_SMALL_WORK_MAX", AR_SMALL_WORK_MAX);
    return k.n > 1 && k.count <= small_count_max() && k.count * static_cast<uint64_t>(k.n) <= work;
}

bool small_tree_message(const Common& k) {
    static const uint64_t bytes = env_bound("AR_SMALL_TREE_MAX", AR_SMALL_TREE_WORK_MAX);
    return k.n > 1 && k.count <= small_count_max() && k.count * static_cast<uint64_t>(k.n) * k.esz <= bytes;
}

// One block per P = threads / N positions; the kernels stride over the rest.
void plan_small(KernelArgs& a, Launch& l, const Common& k) {
    const uint64_t per_block = static_cast<uint64_t>(arimpl::kThreads / k.n);
    l.vec = false;
    l.blocks = static_cast<unsigned>(std::max<uint64_t>(1, std::min<uint64_t>((k.count + per_block - 1) / per_block,
                                                                                0x7fffffffu)));
    a.tile_first = a.tile_end = a.tiles_per_chunk = 0;
}

// Total input bytes (N * S) up to which the fused AllReduce reads with
// cache-allocating loads; AR_CACHED_LOADS_MAX overrides it, 0 turns it off.
uint64_t cached_loads_max() {
    static const uint64_t v = [] {
        const char* e = std::getenv("AR_CACHED_LOADS_MAX");
        if (e != nullptr && e[0] != '\0') return static_cast<uint64_t>(std::strtoull(e, nullptr, 10));
        return static_cast<uint64_t>(AR_CACHED_LOADS_MAX_BYTES);
    }();
    return v;
}

// Tile order of a launch that streams every rank's buffer at once (the fused
// AllReduce, the staged reduce, the phases' reduce-scatter, the fused
// reduce-scatter, the fused tree-order AllReduces): one contiguous slab of
// tiles per XCD, else consecutive tiles to consecutive blocks.  Slabs from
// AR_TILE_XCD_MIN_RANKS ranks; the one-pass AllReduces of every order also
// from AR_FUSED_TILE_XCD_MIN_RANKS ranks, and the ring's at any rank count
// when it reads its inputs through the last-level cache (at most
// AR_CACHED_LOADS_MAX_BYTES in all) and they hold at least
// AR_FUSED_TILE_XCD_MIN_BYTES (the tree orders' kernels stream their inputs
// and gain nothing below 32 ranks: 8 x 8 MiB tree 34.2 / 35.7 us, 32 x 16
// MiB tree 244 / 222, double binary tree 230 / 220, 64 x 16 MiB 474 / 440 and
// 479 / 438).  Measured on MI355X, fused AllReduce, median of
// single calls (graph replay alike), plain / slabs, us: 8 x 8 MiB 31.4 / 29.0,
// 8 x 32 MiB 90.8 / 86.3, 16 x 4 MiB 37.8 / 33.6, 16 x 16 MiB 99.9 / 87.8,
// 32 x 8 MiB 115 / 96, 32 x 32 MiB 436 / 406, 32 x 128 MiB 1,678 / 1,624;
// outside those bounds 8 x 4 MiB 18.6 / 18.3, 16 x 1 MiB about 10 % slower
// in a graph, 8 x 128 MiB 381 / 403, 16 x 64 MiB 406 / 412; the one loss
// inside them 48 x 4 MiB 95.4 / 96.0.  The staged reduce and the phases'
// reduce-scatter stay within +-2.5 % at 8-48 ranks either way.  The
// AR_TILE_XCD environment variable sets one rank bound for every launch
// instead (0: never); it is read at every call, as AR_STAGE_BYTES is.
#ifndef AR_FUSED_TILE_XCD_MIN_RANKS
#define AR_FUSED_TILE_XCD_MIN_RANKS 32
#endif
#ifndef AR_FUSED_TILE_XCD_MIN_BYTES
#define AR_FUSED_TILE_XCD_MIN_BYTES (64ull << 20)
#endif

void tile_order(KernelArgs& a, Launch& l, const Common& k, bool fused_allreduce = false) {
    const char* e = std::getenv("AR_TILE_XCD");
    bool slabs;
    if (e != nullptr && e[0] != '\0') {
        const unsigned from = static_cast<unsigned>(std::strtoul(e, nullptr, 10));
        slabs = from != 0 && static_cast<unsigned>(k.n) >= from;
    } else if (fused_allreduce) {
        const uint64_t total = static_cast<uint64_t>(k.n) * k.count * k.esz;
        slabs = k.n >= AR_FUSED_TILE_XCD_MIN_RANKS || (l.cached && total >= AR_FUSED_TILE_XCD_MIN_BYTES);
    } else {
        slabs = k.n >= AR_TILE_XCD_MIN_RANKS;
    }
    a.xcd_slabs = (slabs && l.blocks >= 8) ? 1 : 0;
    // whole groups of eight blocks, one per XCD (the kernels stride within a slab)
    if (a.xcd_slabs) l.blocks = static_cast<unsigned>(std::min<uint64_t>((l.blocks + 7ull) / 8 * 8, 0x7ffffff8u));
}

// Bytes of rank 0's results per segment of AR_ALGO_STAGED: about
// AR_STAGE_READ_BYTES of inputs read per segment, between AR_STAGE_BYTES_MIN
// and AR_STAGE_BYTES_MAX of results.  The AR_STAGE_BYTES environment variable
// sets it outright; it is read at every call (plans keep what they were built
// with), so one process can exercise several segment sizes.
uint64_t stage_bytes(int nranks) {
    const char* e = std::getenv("AR_STAGE_BYTES");
    if (e != nullptr && e[0] != '\0') {
        const uint64_t b = static_cast<uint64_t>(std::strtoull(e, nullptr, 10));
        if (b > 0) return b;
    }
    const uint64_t b = AR_STAGE_READ_BYTES / static_cast<uint64_t>(nranks);
    return std::min<uint64_t>(AR_STAGE_BYTES_MAX, std::max<uint64_t>(AR_STAGE_BYTES_MIN, b));
}

// Grid of a launch that copies one value to many ranks (fused all-gather,
// staged broadcast): one block per unit row of a tile (kUnroll per tile)
// inside the measured band of total sizes, whole tiles per block outside it.
// The AR_HALF_TILES environment variable (read at every call) forces one form:
// 0 whole tiles, 1 unit rows.
ar_result_t copy_grid(const KernelArgs& a, Launch& l, const Common& k) {
    const char* e = std::getenv("AR_HALF_TILES");
    if (e != nullptr && (e[0] == '0' || e[0] == '1') && e[1] == '\0') {
        l.half = e[0] == '1';
    } else {
        const uint64_t total = k.count * k.esz * static_cast<uint64_t>(k.n);
        l.half = total >= AR_HALF_TILES_MIN_TOTAL && total < AR_HALF_TILES_MAX_TOTAL;
    }
    return grid_for(a, l, l.half ? arimpl::kUnroll : 1);
}

// The staged broadcast's form: one destination rank per block with a tile's
// blocks grouped on one XCD (form 3, k_staged_broadcast_xcd), unless
// AR_BCAST_FORM=0 (read at every call) asks for the tile forms of copy_grid
// (a whole or half tile to every rank per block).  The grid is
// 8 * ceil(tiles / 8) * (N-1) blocks, capped by AR_BLOCKS_PER_CU like the
// others (the kernel then strides).
ar_result_t broadcast_form(const KernelArgs& a, Launch& l, const Common& k) {
    const char* e = std::getenv("AR_BCAST_FORM");
    if ((e != nullptr && e[0] == '0' && e[1] == '\0') || k.n < 2) {
        l.form = 0;
        return AR_SUCCESS;
    }
    int cus = 0;
    const ar_result_t rc = cu_count(&cus);
    if (rc != AR_SUCCESS) return rc;
    const uint64_t tiles = a.tile_end - a.tile_first;
    uint64_t blocks = 8 * ((tiles + 7) / 8) * static_cast<uint64_t>(k.n - 1);
    const unsigned bpc = blocks_per_cu();
    if (bpc != 0) blocks = std::min<uint64_t>(blocks, static_cast<uint64_t>(cus) * bpc);
    l.form = 3;
    l.blocks = static_cast<unsigned>(std::min<uint64_t>(std::max<uint64_t>(blocks, 1), 0x7fffffffu));
    return AR_SUCCESS;
}

// The fused all-gather's form: one destination rank per block with a tile's
// blocks grouped on one XCD (form 3, k_gather_shards_xcd), unless
// AR_GATHER_FORM=0 (read at every call) asks for the tile forms of
// copy_grid.  Measured on MI355X, whole or half tiles to every rank per block
// against form 3, us: all-gather 8 x 256 MiB 395-400 / 347-359, 16 x 64 MiB
// 229-233 / 190, 64 x (2^26+7) 3,253-3,338 / 3,084-3,097, 8 x 16 MiB 44 / 41;
// the phases' AllReduce 8 x 256 MiB 742-745 / 721-722, 16 x 64 MiB 402-403 /
// 369-371.  The grid is 8 * ceil(tiles / 8) * N blocks, capped by
// AR_BLOCKS_PER_CU like the others (the kernel then strides).
ar_result_t gather_form(const KernelArgs& a, Launch& l, const Common& k) {
    const char* e = std::getenv("AR_GATHER_FORM");
    if (e != nullptr && e[0] == '0' && e[1] == '\0') {
        l.form = 0;
        return AR_SUCCESS;
    }
    int cus = 0;
    const ar_result_t rc = cu_count(&cus);
    if (rc != AR_SUCCESS) return rc;
    const uint64_t tiles = a.tile_end - a.tile_first;
    uint64_t blocks = 8 * ((tiles + 7) / 8) * static_cast<uint64_t>(k.n);
    const unsigned bpc = blocks_per_cu();
    if (bpc != 0) blocks = std::min<uint64_t>(blocks, static_cast<uint64_t>(cus) * bpc);
    l.form = 3;
    l.blocks = static_cast<unsigned>(std::min<uint64_t>(std::max<uint64_t>(blocks, 1), 0x7fffffffu));
    return AR_SUCCESS;
}

// Rank count from which AR_ALGO_AUTO runs AllReduce as two fused phases.
int phases_min_ranks() {
    static const int v = [] {
        const char* e = std::getenv("AR_PHASES_MIN_RANKS");
        if (e != nullptr && e[0] != '\0') return static_cast<int>(std::strtol(e, nullptr, 10));
        return AR_PHASES_MIN_RANKS;
    }();
    return v;
}

const char* kind_name(Kind kd) {
    switch (kd) {
        case Kind::kFusedAllReduce: return "fused_allreduce";
        case Kind::kFusedReduceScatter: return "fused_reduce_scatter";
        case Kind::kFusedAllGather: return "fused_all_gather";
        case Kind::kPlaceShards: return "place_shards";
        case Kind::kRingReduceStep: return "ring_reduce_step";
        case Kind::kRingReduceStepWs: return "ring_reduce_step_ws";
        case Kind::kRingCopyStep: return "ring_copy_step";
        case Kind::kFusedTree: return "fused_tree";
        case Kind::kTreeReduceStep: return "tree_reduce_step";
        case Kind::kTreeCopyStep: return "tree_copy_step";
        case Kind::kRingPersistent: return "ring_persistent";
        case Kind::kRingPipelined: return "ring_pipelined";
        case Kind::kRingPipelinedWs: return "ring_pipelined_ws";
        case Kind::kRingPipelinedGather: return "ring_pipelined_gather";
        case Kind::kSmallAllReduce: return "small_allreduce";
        case Kind::kSmallTree: return "small_tree";
        case Kind::kStagedReduce: return "staged_reduce";
        case Kind::kStagedBroadcast: return "staged_broadcast";
        case Kind::kFusedDbt: return "fused_dbt";
        case Kind::kDbtReduceStep: return "dbt_reduce_step";
        case Kind::kDbtCopyStep: return "dbt_copy_step";
        case Kind::kSmallDbt: return "small_dbt";
    }
    return "?";
}

struct Step {
    Launch l;
    KernelArgs a;
    unsigned planned_blocks = 0;   // the grid as planned (persistent plans)
};

ar_result_t launch_step(const Launch& l, const KernelArgs& a, hipStream_t stream) {
    const hipError_t e = arimpl::launch(l, a, stream);
    if (e == hipErrorStreamCaptureUnsupported && l.kind == Kind::kRingPersistent)
        return fail(AR_ERR_UNSUPPORTED, "the persistent ring cannot be captured into a graph");
    if (e != hipSuccess) return fail(AR_ERR_HIP, "%s launch: %s", kind_name(l.kind), hipGetErrorString(e));
    return AR_SUCCESS;
}

// Where planned launches go: straight onto a stream, or into a persistent plan.
class Sink {
public:
    explicit Sink(hipStream_t stream) : stream_(stream) {}
    Sink(std::vector<Step>* steps, ar_algo_t* algo) : steps_(steps), algo_(algo) {}

    // The algorithm a call resolved to (AR_ALGO_AUTO's choice), kept by plans.
    void resolved(ar_algo_t algo) {
        if (algo_ != nullptr) *algo_ = algo;
    }

    // Plans check where their buffers live; one-shot calls take them on trust.
    ar_result_t check_buffers(const std::vector<Interval>& iv) const {
        return steps_ != nullptr ? check_residency(iv) : AR_SUCCESS;
    }

    ar_result_t emit(Launch& l, Kind kind, const KernelArgs& a, const Common& k) {
        l.kind = kind;
        l.dtype = k.dtype;
        l.op = k.op;
        if (debug_enabled()) {
            std::fprintf(stderr,
                         "[ar] %s dtype=%s op=%d n=%d count=%llu step=%d shift=%d mode=%d last=%d vec=%d ofs=%d "
                         "align=2^%d tiles=[%u,%u) tiles/chunk=%u blocks=%u actors=%u cached=%d slabs=%d%s\n",
                         kind_name(kind), dtype_name(k.dtype), static_cast<int>(k.op), k.n,
                         static_cast<unsigned long long>(k.count), a.step, a.shift, a.mode, a.last, l.vec ? 1 : 0, a.ofs,
                         a.align_shift, a.tile_first, a.tile_end, a.tiles_per_chunk, l.blocks, l.actors,
                         l.cached ? 1 : 0, a.xcd_slabs, steps_ != nullptr ? " (planned)" : "");
        }
        if (steps_ != nullptr) {
            steps_->push_back(Step{l, a, l.blocks});
            return AR_SUCCESS;
        }
        return launch_step(l, a, stream_);
    }

private:
    hipStream_t stream_ = nullptr;
    std::vector<Step>* steps_ = nullptr;
    ar_algo_t* algo_ = nullptr;
};

// ---------------------------------------------------------------------------

// Workspace of the ring algorithm (launched per step or pipelined): one
// full-length buffer of partial sums for the reduce-scatter, and for the
// AllReduce of AR_BFLOAT16_ACC_F32; none with fewer than 3 ranks, where the
// only reduce step is also the last.  The
// staged tree AllReduces of AR_BFLOAT16_ACC_F32 keep one float32 slab of
// `count` elements per rank (each slab rounded up to 256 bytes).  The extra
// 1024 bytes cover placing the partials at the senders' residue: up to 255
// bytes to reach a 256-byte boundary, plus the residue itself in
// partial-sized elements (below 256 / element size elements of 4 bytes).
constexpr uint64_t kWorkspaceSlack = 1024;

uint64_t slab_bytes(uint64_t count) { return (count * 4 + 255) & ~static_cast<uint64_t>(255); }

uint64_t ring_workspace_bytes(ar_coll_t coll, uint64_t count, ar_dtype_t dt, int n, ar_algo_t algo) {
    if (count == 0) return 0;
    if (coll == AR_COLL_ALLREDUCE && tree_steps_algo(algo) && dt == AR_BFLOAT16_ACC_F32 && n >= 2)
        return static_cast<uint64_t>(n) * slab_bytes(count) + kWorkspaceSlack;
    if (!ring_steps_algo(algo) || n < 3) return 0;
    if (coll == AR_COLL_REDUCE_SCATTER || (coll == AR_COLL_ALLREDUCE && dt == AR_BFLOAT16_ACC_F32))
        return count * partial_size(dt) + kWorkspaceSlack;
    return 0;
}

// Check the caller's workspace and place the partials at the senders'
// residue (in partial-sized elements) so that they stream as aligned vectors.
ar_result_t use_workspace(KernelArgs& a, const Common& k, ar_coll_t coll, ar_algo_t algo, void* ws,
                          size_t ws_bytes, std::vector<Interval>* iv) {
    const uint64_t need = ring_workspace_bytes(coll, k.count, k.dtype, k.n, algo);
    if (need == 0) return AR_SUCCESS;
    if (ws == nullptr || ws_bytes < need)
        return fail(AR_ERR_INVALID_ARGUMENT, "this algorithm needs a workspace of %llu bytes here",
                    static_cast<unsigned long long>(need));
    const uintptr_t w = reinterpret_cast<uintptr_t>(ws);
    if (iv != nullptr) iv->push_back({w, w + need, true, 0, 2});
    const uintptr_t base = (w + 255u) & ~static_cast<uintptr_t>(255u);
    const uintptr_t shift = base - w + static_cast<uintptr_t>(a.ofs) * partial_size(k.dtype);
    const bool slabs = tree_steps_algo(algo);
    a.ws_stride = slabs ? slab_bytes(k.count) : 0;
    const uint64_t span = slabs ? static_cast<uint64_t>(k.n - 1) * a.ws_stride + k.count * 4
                                : k.count * partial_size(k.dtype);
    if (shift + span > need) return fail(AR_ERR_INTERNAL, "workspace placement");
    a.ws = reinterpret_cast<char*>(w + shift);
    return AR_SUCCESS;
}

// Ranks acting on one chunk in a stage of a tree-shaped schedule (the same
// count the kernels derive; each gets its own row of blocks).
unsigned stage_actors(int mode, int step, int n) {
    switch (mode) {
        case arimpl::kTreeReduce:
        case arimpl::kTreeBcast: {
            const int d = 1 << step;
            return n > d ? static_cast<unsigned>((n - d + 2 * d - 1) / (2 * d)) : 0u;
        }
        case arimpl::kRdExchange: return static_cast<unsigned>(n / 2);
        case arimpl::kHalvingReduce: return static_cast<unsigned>(n >> (step + 1));
        case arimpl::kDoublingGather: return 1u << step;
    }
    return 0u;
}

// AllReduce in a tree-shaped order.  The fused kernel folds the send table as
// a binomial tree; recursive halving's order is that tree over the ranks in
// bit-reversed order.  The staged forms emit one launch per stage.
ar_result_t tree_allreduce(const Common& k, ar_algo_t algo, void* ws, size_t ws_bytes,
                           const std::vector<uintptr_t>& ptrs, Sink& sink) {
    KernelArgs a{};
    Launch l{};
    fill_tables(a, k);
    ar_result_t rc = plan(a, l, k, common_residue(ptrs));
    if (rc != AR_SUCCESS) return rc;
    const int L = ceil_log2(k.n);
    if (algo == AR_ALGO_TREE || algo == AR_ALGO_HALVING_DOUBLING) {
        if (algo == AR_ALGO_HALVING_DOUBLING)
            for (int r = 0; r < k.n; ++r) a.send[r] = static_cast<const char*>(k.send[bit_reverse(r, L)]);
        l.depth = k.n < 16 ? 4 : (k.n < 64 ? 6 : 8);
        if (small_tree_message(k)) {
            plan_small(a, l, k);
            return sink.emit(l, Kind::kSmallTree, a, k);
        }
        // cache-allocating loads while the inputs fit in the last-level cache, as the ring's kernel
        l.cached = l.vec && static_cast<uint64_t>(k.n) * k.count * k.esz <= cached_loads_max();
        tile_order(a, l, k, true);
        return sink.emit(l, Kind::kFusedTree, a, k);
    }
    if ((rc = use_workspace(a, k, AR_COLL_ALLREDUCE, algo, ws, ws_bytes, nullptr)) != AR_SUCCESS) return rc;
    auto stage = [&](Kind kind, int mode, int step, bool last) {
        a.mode = mode;
        a.step = step;
        a.last = last ? 1 : 0;
        l.actors = stage_actors(mode, step, k.n);
        return sink.emit(l, kind, a, k);
    };
    switch (algo) {
        case AR_ALGO_TREE_STEPS:
            for (int s = 0; s < L; ++s)
                if ((rc = stage(Kind::kTreeReduceStep, arimpl::kTreeReduce, s, s == L - 1)) != AR_SUCCESS) return rc;
            for (int s = L - 1; s >= 0; --s)
                if ((rc = stage(Kind::kTreeCopyStep, arimpl::kTreeBcast, s, false)) != AR_SUCCESS) return rc;
            return AR_SUCCESS;
        case AR_ALGO_RECURSIVE_DOUBLING:
            for (int s = 0; s < L; ++s)
                if ((rc = stage(Kind::kTreeReduceStep, arimpl::kRdExchange, s, s == L - 1)) != AR_SUCCESS) return rc;
            return AR_SUCCESS;
        case AR_ALGO_HALVING_DOUBLING_STEPS:
            for (int s = 0; s < L; ++s)
                if ((rc = stage(Kind::kTreeReduceStep, arimpl::kHalvingReduce, s, s == L - 1)) != AR_SUCCESS) return rc;
            for (int s = 0; s < L; ++s)
                if ((rc = stage(Kind::kTreeCopyStep, arimpl::kDoublingGather, s, false)) != AR_SUCCESS) return rc;
            return AR_SUCCESS;
        default:
            return fail(AR_ERR_INTERNAL, "not a tree algorithm");
    }
}

int floor_log2(int n) {
    int l = 0;
    while ((2 << l) <= n) ++l;
    return l;
}

// Positions of height j (2^j times an odd number) among 1..n.
unsigned dbt_actors(int j, int n) { return static_cast<unsigned>(((n >> j) + 1) / 2); }

// AllReduce over the double binary tree: the buffer cut in two halves, half c
// reduced in binary tree c's bracketing.  The fused kernel evaluates both in
// one pass; the stage kernels climb the trees' floor(log2 N) levels, then
// descend them.
ar_result_t dbt_allreduce(const Common& k, ar_algo_t algo, void* ws, size_t ws_bytes,
                          const std::vector<uintptr_t>& ptrs, Sink& sink) {
    KernelArgs a{};
    Launch l{};
    fill_tables(a, k);
    ar_result_t rc = plan(a, l, k, common_residue(ptrs), 2);
    if (rc != AR_SUCCESS) return rc;
    a.count_q = k.count / 2;
    a.count_r = static_cast<uint32_t>(k.count % 2);
    if (algo == AR_ALGO_DOUBLE_BINARY_TREE) {
        l.depth = k.n < 16 ? 4 : 6;   // the deepest stack the trees need: 3 below 16 ranks, 6 up to 128
        if (small_tree_message(k)) {
            plan_small(a, l, k);
            return sink.emit(l, Kind::kSmallDbt, a, k);
        }
        // cache-allocating loads while the inputs fit in the last-level cache, as the ring's kernel
        l.cached = l.vec && static_cast<uint64_t>(k.n) * k.count * k.esz <= cached_loads_max();
        tile_order(a, l, k, true);
        return sink.emit(l, Kind::kFusedDbt, a, k);
    }
    if ((rc = use_workspace(a, k, AR_COLL_ALLREDUCE, algo, ws, ws_bytes, nullptr)) != AR_SUCCESS) return rc;
    const int levels = floor_log2(k.n);
    for (int j = 1; j <= levels; ++j) {
        a.step = j;
        a.last = j == levels ? 1 : 0;
        l.actors = dbt_actors(j, k.n);
        if ((rc = sink.emit(l, Kind::kDbtReduceStep, a, k)) != AR_SUCCESS) return rc;
    }
    for (int j = levels; j >= 1; --j) {
        a.step = j;
        a.last = 0;
        l.actors = dbt_actors(j, k.n);
        if ((rc = sink.emit(l, Kind::kDbtCopyStep, a, k)) != AR_SUCCESS) return rc;
    }
    return AR_SUCCESS;
}

ar_result_t allreduce_impl(const Common& k, ar_algo_t algo, void* ws, size_t ws_bytes, Sink& sink) {
    ar_result_t rc = check_common(k, true);
    if (rc != AR_SUCCESS) return rc;
    if (!algo_known(algo)) return fail(AR_ERR_INVALID_ARGUMENT, "unknown algo %d", static_cast<int>(algo));
    std::vector<Interval> iv;
    std::vector<uintptr_t> ptrs;
    const uint64_t bytes = k.count * k.esz;
    for (int r = 0; r < k.n; ++r) {
        if ((rc = check_ptr(k.send[r], k.count, k.esz, "sendbufs", r)) != AR_SUCCESS) return rc;
        if ((rc = check_ptr(k.recv[r], k.count, k.esz, "recvbufs", r)) != AR_SUCCESS) return rc;
        const uintptr_t s = reinterpret_cast<uintptr_t>(k.send[r]);
        const uintptr_t d = reinterpret_cast<uintptr_t>(k.recv[r]);
        if (bytes) {
            iv.push_back({s, s + bytes, false, r, 0});
            iv.push_back({d, d + bytes, true, r, 1});
        }
        ptrs.push_back(s);
        ptrs.push_back(d);
    }
    // AUTO (bounds in ar.h, from timings of the three forms): two fused phases
    // from AR_BIG_PHASES_MIN_RANKS ranks once all ranks together hold
    // AR_BIG_PHASES_MIN_TOTAL_BYTES, up to AR_BIG_PHASES_MAX_TOTAL_BYTES in all
    // and AR_BIG_PHASES_MAX_RANK_BYTES per rank; the staged
    // reduce-then-broadcast for large buffers over 6 ranks or more otherwise; the phases again from
    // AR_PHASES_MIN_RANKS ranks when every rank holds at least
    // AR_PHASES_MIN_BYTES and all together more than
    // AR_PHASES_ABOVE_TOTAL_BYTES; else the one fused kernel (and the
    // small-message kernel for the smallest messages)
    if (algo == AR_ALGO_AUTO) {
        const uint64_t per_rank = k.count * k.esz;
        const uint64_t total = per_rank * static_cast<uint64_t>(k.n);
        const bool narrow = k.esz == 2;   // 16-bit types: other bounds (measured)
        const uint64_t min_rank = narrow ? AR_STAGED_MIN_BYTES_16BIT : AR_STAGED_MIN_BYTES;
        const uint64_t min_total = narrow ? AR_STAGED_MIN_TOTAL_BYTES_16BIT : AR_STAGED_MIN_TOTAL_BYTES;
        const bool big_phases = k.n >= AR_BIG_PHASES_MIN_RANKS && total >= AR_BIG_PHASES_MIN_TOTAL_BYTES &&
                                total <= AR_BIG_PHASES_MAX_TOTAL_BYTES && per_rank <= AR_BIG_PHASES_MAX_RANK_BYTES;
        if (big_phases)
            algo = AR_ALGO_PHASES;
        else if (k.n >= AR_STAGED_MIN_RANKS && per_rank >= min_rank && total >= min_total)
            algo = AR_ALGO_STAGED;
        else if (k.n >= phases_min_ranks() && per_rank >= AR_PHASES_MIN_BYTES &&
                 total > AR_PHASES_ABOVE_TOTAL_BYTES && !small_message(k))
            algo = AR_ALGO_PHASES;
        else
            algo = AR_ALGO_FUSED;
    }
    sink.resolved(k.n == 1 ? AR_ALGO_FUSED : algo);
    if (algo == AR_ALGO_RING_PERSISTENT && k.dtype == AR_BFLOAT16_ACC_F32)
        return fail(AR_ERR_UNSUPPORTED, "the persistent ring has no form with float32 partials");
    if (power_of_two_algo(algo) && (k.n & (k.n - 1)) != 0)
        return fail(AR_ERR_UNSUPPORTED, "algo %d needs a power-of-two number of ranks, not %d",
                    static_cast<int>(algo), k.n);
    if (k.n == 1) algo = AR_ALGO_FUSED;           // a copy
    {
        KernelArgs probe{};
        if ((rc = use_workspace(probe, k, AR_COLL_ALLREDUCE, algo, ws, ws_bytes, &iv)) != AR_SUCCESS) return rc;
    }
    rc = check_overlaps(iv, [&](const Interval& s, const Interval& d) {
        return s.rank == d.rank && s.lo == d.lo;   // in place: send[r] == recv[r]
    });
    if (rc != AR_SUCCESS || (rc = sink.check_buffers(iv)) != AR_SUCCESS) return rc;
    if (k.count == 0) return AR_SUCCESS;

    if (tree_algo(algo)) return tree_allreduce(k, algo, ws, ws_bytes, ptrs, sink);
    if (dbt_algo(algo)) return dbt_allreduce(k, algo, ws, ws_bytes, ptrs, sink);
    KernelArgs a{};
    Launch l{};
    fill_tables(a, k);
    if (algo == AR_ALGO_PHASES) {
        // reduce-scatter: chunk c of the reduction into chunk c of recv[c] ...
        std::vector<uintptr_t> sends;
        for (int r = 0; r < k.n; ++r) {
            a.recv[r] = static_cast<char*>(k.recv[r]) + chunk_start(r, k.count, k.n) * k.esz;
            sends.push_back(reinterpret_cast<uintptr_t>(k.send[r]));
        }
        if ((rc = plan(a, l, k, common_residue(sends))) != AR_SUCCESS) return rc;
        // cache-allocating stores: the all-gather that follows rereads these chunks
        l.cached_store = true;
        tile_order(a, l, k);
        if ((rc = sink.emit(l, Kind::kFusedReduceScatter, a, k)) != AR_SUCCESS) return rc;
        // ... then all-gather in place: chunk c of recv[c] to every other rank
        KernelArgs g{};
        Launch lg{};
        fill_tables(g, k);
        std::vector<uintptr_t> recvs;
        for (int r = 0; r < k.n; ++r) {
            g.send[r] = static_cast<const char*>(k.recv[r]) + chunk_start(r, k.count, k.n) * k.esz;
            recvs.push_back(reinterpret_cast<uintptr_t>(k.recv[r]));
        }
        if ((rc = plan(g, lg, k, common_residue(recvs))) != AR_SUCCESS) return rc;
        if ((rc = gather_form(g, lg, k)) != AR_SUCCESS) return rc;
        return sink.emit(lg, Kind::kFusedAllGather, g, k);   // whole tiles: measured faster in place
    }
    if (algo == AR_ALGO_FUSED && small_message(k)) {
        plan_small(a, l, k);
        return sink.emit(l, Kind::kSmallAllReduce, a, k);
    }
    if ((rc = plan(a, l, k, common_residue(ptrs))) != AR_SUCCESS) return rc;
    if (algo == AR_ALGO_FUSED) {
        l.cached = l.vec && static_cast<uint64_t>(k.n) * k.count * k.esz <= cached_loads_max();
        tile_order(a, l, k, true);
        return sink.emit(l, Kind::kFusedAllReduce, a, k);
    }
    if (algo == AR_ALGO_STAGED) {
        // segments of whole tiles, each holding about stage_bytes() of rank 0's
        // results: reduce into rank 0, then broadcast from it
        // the nearest whole number of segments, tiles spread evenly over them (so
        // chunks rounded up to whole tiles do not leave a sliver of a segment)
        const uint32_t total = a.tile_end;
        const uint64_t tile_bytes = static_cast<uint64_t>(arimpl::kThreads) * arimpl::kUnroll * (l.vec ? 16 : k.esz);
        const uint64_t stage = stage_bytes(k.n);
        const uint64_t nseg = std::max<uint64_t>(1, (total * tile_bytes + stage / 2) / stage);
        const uint64_t per_seg = (total + nseg - 1) / nseg;
        for (uint64_t t0 = 0; t0 < total; t0 += per_seg) {
            a.tile_first = static_cast<uint32_t>(t0);
            a.tile_end = static_cast<uint32_t>(std::min<uint64_t>(total, t0 + per_seg));
            if ((rc = grid_for(a, l)) != AR_SUCCESS) return rc;
            tile_order(a, l, k);
            if ((rc = sink.emit(l, Kind::kStagedReduce, a, k)) != AR_SUCCESS) return rc;
            if ((rc = copy_grid(a, l, k)) != AR_SUCCESS) return rc;
            if ((rc = broadcast_form(a, l, k)) != AR_SUCCESS) return rc;
            if ((rc = sink.emit(l, Kind::kStagedBroadcast, a, k)) != AR_SUCCESS) return rc;
            l.form = 0;
            l.half = false;
        }
        return AR_SUCCESS;
    }
    if (algo == AR_ALGO_RING_PERSISTENT) return sink.emit(l, Kind::kRingPersistent, a, k);
    if (algo == AR_ALGO_RING_PIPELINED) {
        if (k.dtype != AR_BFLOAT16_ACC_F32) return sink.emit(l, Kind::kRingPipelined, a, k);
        // float32 partials travel through the workspace, as in the ring's launches
        if ((rc = use_workspace(a, k, AR_COLL_ALLREDUCE, algo, ws, ws_bytes, nullptr)) != AR_SUCCESS) return rc;
        a.mode = 1;
        return sink.emit(l, Kind::kRingPipelinedWs, a, k);
    }
    if (k.dtype == AR_BFLOAT16_ACC_F32) {
        // float32 partials travel through the workspace; the last step leaves
        // finished chunk c in chunk c of rank c-1's own buffer, as the ring does
        KernelArgs w = a;
        if ((rc = use_workspace(w, k, AR_COLL_ALLREDUCE, algo, ws, ws_bytes, nullptr)) != AR_SUCCESS) return rc;
        for (int c = 0; c < k.n; ++c)
            w.recv[c] = static_cast<char*>(k.recv[(c + k.n - 1) % k.n]) + chunk_start(c, k.count, k.n) * k.esz;
        for (int s = 0; s < k.n - 1; ++s) {
            w.step = s;
            if ((rc = sink.emit(l, Kind::kRingReduceStepWs, w, k)) != AR_SUCCESS) return rc;
        }
    } else {
        for (int s = 0; s < k.n - 1; ++s) {      // reduce-scatter steps
            a.step = s;
            if ((rc = sink.emit(l, Kind::kRingReduceStep, a, k)) != AR_SUCCESS) return rc;
        }
    }
    for (int s = 0; s < k.n - 1; ++s) {          // all-gather steps
        a.step = s;
        a.shift = 0;
        if ((rc = sink.emit(l, Kind::kRingCopyStep, a, k)) != AR_SUCCESS) return rc;
    }
    return AR_SUCCESS;
}

ar_result_t reduce_scatter_impl(const Common& k, ar_algo_t algo, void* ws, size_t ws_bytes, Sink& sink) {
    ar_result_t rc = check_common(k, true);
    if (rc != AR_SUCCESS) return rc;
    if (!algo_known(algo)) return fail(AR_ERR_INVALID_ARGUMENT, "unknown algo %d", static_cast<int>(algo));
    if (allreduce_only_algo(algo))
        return fail(AR_ERR_UNSUPPORTED, "algo %d is defined for AllReduce only", static_cast<int>(algo));
    if (!ring_steps_algo(algo)) algo = AR_ALGO_FUSED;
    sink.resolved(k.n == 1 ? AR_ALGO_FUSED : algo);
    std::vector<Interval> iv;
    std::vector<uintptr_t> ptrs;
    const uint64_t bytes = k.count * k.esz;
    for (int r = 0; r < k.n; ++r) {
        const uint64_t st = chunk_start(r, k.count, k.n);
        const uint64_t cl = chunk_start(r + 1, k.count, k.n) - st;
        if ((rc = check_ptr(k.send[r], k.count, k.esz, "sendbufs", r)) != AR_SUCCESS) return rc;
        if ((rc = check_ptr(k.recv[r], cl, k.esz, "recvbufs", r)) != AR_SUCCESS) return rc;
        const uintptr_t s = reinterpret_cast<uintptr_t>(k.send[r]);
        const uintptr_t d = reinterpret_cast<uintptr_t>(k.recv[r]);
        if (bytes) iv.push_back({s, s + bytes, false, r, 0});
        if (cl) iv.push_back({d, d + cl * k.esz, true, r, 1});
        ptrs.push_back(s);
    }
    {
        KernelArgs probe{};
        if ((rc = use_workspace(probe, k, AR_COLL_REDUCE_SCATTER, algo, ws, ws_bytes, &iv)) != AR_SUCCESS) return rc;
    }
    rc = check_overlaps(iv, [&](const Interval& s, const Interval& d) {
        // in place: recv[r] == send[r] + start(r) elements
        return s.rank == d.rank && d.lo == s.lo + chunk_start(d.rank, k.count, k.n) * k.esz;
    });
    if (rc != AR_SUCCESS || (rc = sink.check_buffers(iv)) != AR_SUCCESS) return rc;
    if (k.count == 0) return AR_SUCCESS;

    KernelArgs a{};
    Launch l{};
    fill_tables(a, k);
    const Residue residue = common_residue(ptrs);
    if ((rc = plan(a, l, k, residue)) != AR_SUCCESS) return rc;
    if (algo == AR_ALGO_FUSED || k.n == 1) {
        tile_order(a, l, k);
        return sink.emit(l, Kind::kFusedReduceScatter, a, k);
    }
    if ((rc = use_workspace(a, k, AR_COLL_REDUCE_SCATTER, algo, ws, ws_bytes, nullptr)) != AR_SUCCESS) return rc;
    if (algo == AR_ALGO_RING_PIPELINED) {
        a.mode = 0;
        return sink.emit(l, Kind::kRingPipelinedWs, a, k);
    }
    for (int s = 0; s < k.n - 1; ++s) {
        a.step = s;
        if ((rc = sink.emit(l, Kind::kRingReduceStepWs, a, k)) != AR_SUCCESS) return rc;
    }
    return AR_SUCCESS;
}

ar_result_t all_gather_impl(const Common& k, ar_algo_t algo, Sink& sink) {
    ar_result_t rc = check_common(k, false);
    if (rc != AR_SUCCESS) return rc;
    if (!algo_known(algo)) return fail(AR_ERR_INVALID_ARGUMENT, "unknown algo %d", static_cast<int>(algo));
    if (allreduce_only_algo(algo))
        return fail(AR_ERR_UNSUPPORTED, "algo %d is defined for AllReduce only", static_cast<int>(algo));
    if (!ring_steps_algo(algo)) algo = AR_ALGO_FUSED;
    sink.resolved(k.n == 1 ? AR_ALGO_FUSED : algo);
    std::vector<Interval> iv;
    std::vector<uintptr_t> ptrs;
    const uint64_t bytes = k.count * k.esz;
    for (int r = 0; r < k.n; ++r) {
        const uint64_t st = chunk_start(r, k.count, k.n);
        const uint64_t cl = chunk_start(r + 1, k.count, k.n) - st;
        if ((rc = check_ptr(k.send[r], cl, k.esz, "sendbufs", r)) != AR_SUCCESS) return rc;
        if ((rc = check_ptr(k.recv[r], k.count, k.esz, "recvbufs", r)) != AR_SUCCESS) return rc;
        const uintptr_t s = reinterpret_cast<uintptr_t>(k.send[r]);
        const uintptr_t d = reinterpret_cast<uintptr_t>(k.recv[r]);
        if (cl) iv.push_back({s, s + cl * k.esz, false, r, 0});
        if (bytes) iv.push_back({d, d + bytes, true, r, 1});
        ptrs.push_back(d);
    }
    rc = check_overlaps(iv, [&](const Interval& s, const Interval& d) {
        // in place: send[r] == recv[r] + start(r) elements
        return s.rank == d.rank && s.lo == d.lo + chunk_start(s.rank, k.count, k.n) * k.esz;
    });
    if (rc != AR_SUCCESS || (rc = sink.check_buffers(iv)) != AR_SUCCESS) return rc;
    if (k.count == 0) return AR_SUCCESS;

    KernelArgs a{};
    Launch l{};
    fill_tables(a, k);
    if ((rc = plan(a, l, k, common_residue(ptrs))) != AR_SUCCESS) return rc;
    if (algo == AR_ALGO_FUSED || k.n == 1) {
        if ((rc = copy_grid(a, l, k)) != AR_SUCCESS) return rc;
        if ((rc = gather_form(a, l, k)) != AR_SUCCESS) return rc;
        return sink.emit(l, Kind::kFusedAllGather, a, k);
    }
    if (algo == AR_ALGO_RING_PIPELINED) return sink.emit(l, Kind::kRingPipelinedGather, a, k);
    if ((rc = sink.emit(l, Kind::kPlaceShards, a, k)) != AR_SUCCESS) return rc;
    for (int s = 0; s < k.n - 1; ++s) {
        a.step = s;
        a.shift = 1;
        if ((rc = sink.emit(l, Kind::kRingCopyStep, a, k)) != AR_SUCCESS) return rc;
    }
    return AR_SUCCESS;
}

}  // namespace

void arimpl::set_error_detail(const char* text) { g_detail = text; }

// A persistent collective: the launches one call makes, validated and planned.
struct ar_plan_s {
    std::vector<Step> steps;
    ar_algo_t algo = AR_ALGO_AUTO;   // what the planned call resolved to
};

namespace {

// Persistent collectives: validate and plan once, enqueue many times.

template <typename Build>
ar_result_t make_plan(ar_plan_t* out, Build build) {
    g_detail.clear();
    if (out == nullptr) return fail(AR_ERR_INVALID_ARGUMENT, "null plan pointer");
    *out = nullptr;
    ar_plan_s* p = new (std::nothrow) ar_plan_s;
    if (p == nullptr) return fail(AR_ERR_INTERNAL, "out of host memory");
    Sink sink(&p->steps, &p->algo);
    const ar_result_t rc = build(sink);
    if (rc != AR_SUCCESS) {
        delete p;
        return rc;
    }
    *out = p;
    return AR_SUCCESS;
}

}  // namespace

extern "C" {

ar_result_t ar_allreduce(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                         ar_op_t op, int nranks, hipStream_t stream) {
    Sink sink(stream);
    return allreduce_impl({sendbufs, recvbufs, count, dtype, op, nranks, esize(dtype)}, AR_ALGO_AUTO, nullptr, 0,
                          sink);
}

ar_result_t ar_allreduce_ex(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                            ar_op_t op, int nranks, ar_algo_t algo, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    Sink sink(stream);
    return allreduce_impl({sendbufs, recvbufs, count, dtype, op, nranks, esize(dtype)}, algo, workspace,
                          workspace_bytes, sink);
}

ar_result_t ar_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                              ar_op_t op, int nranks, hipStream_t stream) {
    Sink sink(stream);
    return reduce_scatter_impl({sendbufs, recvbufs, count, dtype, op, nranks, esize(dtype)}, AR_ALGO_FUSED,
                               nullptr, 0, sink);
}

ar_result_t ar_reduce_scatter_ex(const void* const* sendbufs, void* const* recvbufs, size_t count,
                                 ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    Sink sink(stream);
    return reduce_scatter_impl({sendbufs, recvbufs, count, dtype, op, nranks, esize(dtype)}, algo, workspace,
                               workspace_bytes, sink);
}

ar_result_t ar_all_gather(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                          int nranks, hipStream_t stream) {
    Sink sink(stream);
    return all_gather_impl({sendbufs, recvbufs, count, dtype, AR_SUM, nranks, esize(dtype)}, AR_ALGO_FUSED, sink);
}

ar_result_t ar_all_gather_ex(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                             int nranks, ar_algo_t algo, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    (void)workspace;
    (void)workspace_bytes;
    Sink sink(stream);
    return all_gather_impl({sendbufs, recvbufs, count, dtype, AR_SUM, nranks, esize(dtype)}, algo, sink);
}

ar_result_t ar_allreduce_init(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                              ar_op_t op, int nranks, ar_algo_t algo, void* workspace, size_t workspace_bytes,
                              ar_plan_t* plan) {
    return make_plan(plan, [&](Sink& sink) {
        return allreduce_impl({sendbufs, recvbufs, count, dtype, op, nranks, esize(dtype)}, algo, workspace,
                              workspace_bytes, sink);
    });
}

ar_result_t ar_reduce_scatter_init(const void* const* sendbufs, void* const* recvbufs, size_t count,
                                   ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo, void* workspace,
                                   size_t workspace_bytes, ar_plan_t* plan) {
    return make_plan(plan, [&](Sink& sink) {
        return reduce_scatter_impl({sendbufs, recvbufs, count, dtype, op, nranks, esize(dtype)}, algo, workspace,
                                   workspace_bytes, sink);
    });
}

ar_result_t ar_all_gather_init(const void* const* sendbufs, void* const* recvbufs, size_t count, ar_dtype_t dtype,
                               int nranks, ar_algo_t algo, void* workspace, size_t workspace_bytes,
                               ar_plan_t* plan) {
    (void)workspace;
    (void)workspace_bytes;
    return make_plan(plan, [&](Sink& sink) {
        return all_gather_impl({sendbufs, recvbufs, count, dtype, AR_SUM, nranks, esize(dtype)}, algo, sink);
    });
}

ar_result_t ar_plan_start(ar_plan_t plan, hipStream_t stream) {
    if (plan == nullptr) return fail(AR_ERR_INVALID_ARGUMENT, "null plan");
    for (const Step& st : plan->steps) {
        const ar_result_t rc = launch_step(st.l, st.a, stream);
        if (rc != AR_SUCCESS) return rc;
    }
    return AR_SUCCESS;
}

int ar_plan_num_launches(ar_plan_t plan) {
    return plan == nullptr ? -1 : static_cast<int>(plan->steps.size());
}

int ar_plan_algo(ar_plan_t plan) {
    return plan == nullptr ? -1 : static_cast<int>(plan->algo);
}

ar_result_t ar_plan_limit_blocks(ar_plan_t plan, unsigned max_blocks) {
    g_detail.clear();
    if (plan == nullptr) return fail(AR_ERR_INVALID_ARGUMENT, "null plan");
    for (Step& st : plan->steps) {
        if (max_blocks == 0) {
            st.l.blocks = st.planned_blocks;
            continue;
        }
        const unsigned rows = st.l.actors > 0 ? st.l.actors : 1;   // the grid's y extent
        st.l.blocks = std::max(1u, std::min(st.planned_blocks, max_blocks / rows));
    }
    return AR_SUCCESS;
}

ar_result_t ar_plan_free(ar_plan_t plan) {
    delete plan;
    return AR_SUCCESS;
}

size_t ar_workspace_bytes(ar_coll_t coll, ar_algo_t algo, size_t count, ar_dtype_t dtype, int nranks) {
    const size_t e = esize(dtype);
    if (e == 0 || nranks < 1 || nranks > AR_MAX_RANKS || !algo_known(algo) ||
        count > (UINT64_MAX / AR_MAX_RANKS) / 16)
        return static_cast<size_t>(-1);
    switch (coll) {
        case AR_COLL_ALLREDUCE:
        case AR_COLL_ALL_GATHER:
        case AR_COLL_REDUCE_SCATTER:
            return static_cast<size_t>(ring_workspace_bytes(coll, count, dtype, nranks, algo));
    }
    return static_cast<size_t>(-1);
}

ar_result_t ar_chunk_range(int c, size_t count, int nranks, size_t* begin, size_t* end) {
    g_detail.clear();
    if (nranks < 1 || nranks > AR_MAX_RANKS) return fail(AR_ERR_INVALID_ARGUMENT, "nranks %d outside [1, %d]", nranks, AR_MAX_RANKS);
    if (c < 0 || c >= nranks) return fail(AR_ERR_INVALID_ARGUMENT, "chunk %d outside [0, %d)", c, nranks);
    if (begin == nullptr || end == nullptr) return fail(AR_ERR_INVALID_ARGUMENT, "null output pointer");
    if (count > (UINT64_MAX / AR_MAX_RANKS) / 16) return fail(AR_ERR_INVALID_ARGUMENT, "count too large");
    *begin = static_cast<size_t>(chunk_start(c, count, nranks));
    *end = static_cast<size_t>(chunk_start(c + 1, count, nranks));
    return AR_SUCCESS;
}

const char* ar_get_error_string(ar_result_t r) {
    switch (r) {
        case AR_SUCCESS: return "success";
        case AR_ERR_INVALID_ARGUMENT: return "invalid argument";
        case AR_ERR_UNSUPPORTED: return "unsupported";
        case AR_ERR_HIP: return "HIP runtime error";
        case AR_ERR_INTERNAL: return "internal error";
    }
    return "unknown result code";
}

const char* ar_get_last_error_detail(void) { return g_detail.c_str(); }

size_t ar_dtype_size(ar_dtype_t dtype) { return esize(dtype); }

}  // extern "C"
