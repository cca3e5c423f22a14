// HIP kernels (gfx950) for the ring AllReduce over N virtual ranks held in
// one GPU's HBM.
//
// The tiled kernels walk the buffer chunk by chunk, chunk(c) =
// [c*len/N, (c+1)*len/N) (tirogla.com "Ring all-reduce", section "Code"), so
// the chunk index c, and with it the ring rotation that decides which rank's
// buffer is read first, is the same for a whole block: the per-rank pointers
// are picked with scalar loads from the kernel arguments and the fold over
// ranks is a fixed sequence, never a register-indexed rotation.
//
// The work is a pure stream through HBM (one add per element per rank), so
// the tiled kernels use no LDS and no MFMA: each thread moves 16-byte
// vectors, `kUnroll` of them per rank per tile, issues a batch of up to
// `kBatch` ranks' loads before it folds them in ring order, and writes
// outputs with nontemporal stores (results that the next launch rereads with
// cache-allocating ones).  Chunk edges that are not 16-byte aligned
// (uneven chunks start anywhere) are done one element at a time by the first
// tile of the chunk.  Messages whose chunks are only a few elements long take
// k_small_allreduce instead, which stages every rank's values of a few
// positions in LDS.
//
// Arithmetic follows the ring's association order exactly: element i of
// chunk c is ((x_c (op) x_{c+1}) (op) x_{c+2}) ... (arjunsriva.com
// "AllReduce, All the Way Down", figure "Ring AllReduce · follow chunk 0"),
// one rounding per operation, no contraction (built with -ffp-contract=off),
// bf16 rounded to nearest-even after every operation.

#include "ar_device.h"

namespace arimpl {
namespace {

// ---------------------------------------------------------------------------
// fused kernels: one pass over HBM
// ---------------------------------------------------------------------------

// AllReduce: every rank's output gets the ring-order fold.  Reads N*S,
// writes N*S bytes.  In place (send[r] == recv[r]) is safe: each position is
// read by the thread that later writes it, and by no other.  NT_LOAD: the
// body's loads are nontemporal (inputs larger than the Infinity Cache) or
// cache-allocating (inputs that fit in it).
template <int DT, int OP, int VEC, bool NT_LOAD>
__global__ __launch_bounds__(kThreads) void k_fused_allreduce(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    AR_TILE_LOOP_BEGIN
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            store_elem_all<elem_size<DT>()>(a, n, i, fold_element<DT, OP>(a, c, i));
        }
    }
    typename Fold<DT, OP, VEC>::A acc[kUnroll];
    fold_units<DT, OP, VEC, NT_LOAD>(a, c, adj, tv0, live, acc);
    typename U::T res[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) res[u] = Fold<DT, OP, VEC>::done(acc[u], n);
    }
    for (int q = 0; q < n; ++q) {
        char* tb = U::tile(a.recv[q] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) U::store(tb, U::lane_off(u), res[u]);
        }
    }
    AR_TILE_LOOP_END
}

// Staged AllReduce: the data moves as a reduce onto rank 0 followed by a
// broadcast from it (bitfern.com "AllReduce Explained", section "Reduce
// Followed by Broadcast"), while every value keeps the ring's association
// order.  Reducing launch: the fused AllReduce's fold for the launch's tiles,
// stored to rank 0's receive buffer only.  The stores allocate in the caches
// (the one-pass kernels' outputs do not), so the broadcast launch that
// follows rereads the results from the Infinity Cache instead of HBM.  This
// launch is then almost all reads, and the broadcast almost all writes: HBM
// serves each direction faster alone than the two interleaved.
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_staged_reduce(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            store_elem<ESZ, false>(a.recv[0] + i * ESZ, fold_element<DT, OP>(a, c, i));
        }
    }
    typename Fold<DT, OP, VEC>::A acc[kUnroll];
    fold_units<DT, OP, VEC>(a, c, adj, tv0, live, acc);
    char* tb = U::tile(a.recv[0] - adj, tv0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) U::template store<false>(tb, U::lane_off(u), Fold<DT, OP, VEC>::done(acc[u], n));
    }
    AR_TILE_LOOP_END
}

// Staged AllReduce, broadcasting launch: rank 0's results for the same tiles
// (so the same elements, chunk edges included) copied to ranks 1..N-1.  Each
// block takes one of a tile's kUnroll units per thread, so a wave issues half
// the stores of a whole tile; HBM mostly takes the writes faster that way.
// With AR_BCAST_FORM=0 the host picks this form or k_staged_broadcast_tiles
// by measured shape; by default it takes k_staged_broadcast_xcd.
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_staged_broadcast(const KernelArgs a) {
    using U = Unit<DT, VEC, false>;   // cache-allocating loads: the results sit in the Infinity Cache
    constexpr int ESZ = elem_size<DT>();
    const int n = a.nranks;
    const uint32_t tpc = a.tiles_per_chunk;
    const int64_t adj = (VEC > 1) ? static_cast<int64_t>(a.ofs) * ESZ : 0;
    const char* src = a.recv[0];
    const uint64_t parts = static_cast<uint64_t>(a.tile_end - a.tile_first) * kUnroll;
    for (uint64_t w = blockIdx.x; w < parts; w += gridDim.x) {
        const uint32_t tile = a.tile_first + static_cast<uint32_t>(w / kUnroll);
        const int u = static_cast<int>(w % kUnroll);
        const int c = static_cast<int>(tile / tpc);
        const uint64_t t = tile - static_cast<uint32_t>(c) * tpc;
        const Span sp = chunk_span<VEC>(c, a);
        const uint64_t tv0 = sp.vb + t * (kThreads * kUnroll);
        if (VEC > 1 && t == 0 && u == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) {
                const uint32_t x = load_elem<ESZ>(src + i * ESZ);
                for (int q = 1; q < n; ++q) store_elem<ESZ>(a.recv[q] + i * ESZ, x);
            }
        }
        if (tv0 + U::lane_unit(u) < sp.ve) {
            const typename U::T x = U::load(U::tile(src - adj, tv0), U::lane_off(u));
            for (int q = 1; q < n; ++q) U::store(U::tile(a.recv[q] - adj, tv0), U::lane_off(u), x);
        }
    }
}

// The same broadcast with whole tiles per block (kUnroll unit rows): of the
// two tile forms, faster when all ranks' buffers hold less than 2 GiB or
// more than 8 GiB in all.
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_staged_broadcast_tiles(const KernelArgs a) {
    using U = Unit<DT, VEC, false>;   // cache-allocating loads: the results sit in the Infinity Cache
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    const char* src = a.recv[0];
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            const uint32_t x = load_elem<ESZ>(src + i * ESZ);
            for (int q = 1; q < n; ++q) store_elem<ESZ>(a.recv[q] + i * ESZ, x);
        }
    }
    typename U::T x[kUnroll];
    const char* sb = U::tile(src - adj, tv0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) x[u] = U::load(sb, U::lane_off(u));
    }
    for (int q = 1; q < n; ++q) {
        char* tb = U::tile(a.recv[q] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) U::store(tb, U::lane_off(u), x[u]);
        }
    }
    AR_TILE_LOOP_END
}

// Staged AllReduce, broadcasting launch, one destination rank per block with
// a tile's N-1 blocks on one XCD: workgroups go to MI355X's 8 XCDs in turn,
// so block b = x + 8 m, on XCD x, copies tile tile_first + 8 (m / (N-1)) + x
// of rank 0's results to rank 1 + m mod (N-1).  The source tile is fetched
// into that XCD's L2 once for its N-1 destinations, and neighbouring blocks
// on an XCD write the same tile of neighbouring ranks.  Measured on MI355X
// against whole or half tiles to every rank per block, staged AllReduce in
// us: 8 x 256 MiB 725 / 732, 16 x 64 MiB 378 / 402, 64 x 256 MiB 5,814 /
// 5,885; sending every destination's copy from its own XCD instead (each
// tile loaded N-1 times) was slower everywhere (8 x 256 MiB: 944 us).  The
// planned grid is 8 * ceil(tiles / 8) * (N-1) blocks; a capped grid strides
// over the same numbering (same results, the XCD grouping then approximate).
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_staged_broadcast_xcd(const KernelArgs a) {
    using U = Unit<DT, VEC, false>;   // cache-allocating loads: the results sit in the Infinity Cache
    constexpr int ESZ = elem_size<DT>();
    const int n = a.nranks;
    const uint32_t tpc = a.tiles_per_chunk;
    const int64_t adj = (VEC > 1) ? static_cast<int64_t>(a.ofs) * ESZ : 0;
    const char* src = a.recv[0];
    const uint64_t dests = static_cast<uint64_t>(n - 1);
    const uint64_t groups = (static_cast<uint64_t>(a.tile_end - a.tile_first) + 7) / 8;
    const uint64_t total = 8 * groups * dests;
    for (uint64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const uint64_t m = b / 8;
        const uint64_t tile64 = a.tile_first + 8 * (m / dests) + (b % 8);
        if (tile64 >= a.tile_end) continue;
        const uint32_t tile = static_cast<uint32_t>(tile64);
        const int q = 1 + static_cast<int>(m % dests);
        const int c = static_cast<int>(tile / tpc);
        const uint64_t t = tile - static_cast<uint32_t>(c) * tpc;
        const Span sp = chunk_span<VEC>(c, a);
        const uint64_t tv0 = sp.vb + t * (kThreads * kUnroll);
        if (VEC > 1 && t == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) store_elem<ESZ>(a.recv[q] + i * ESZ, load_elem<ESZ>(src + i * ESZ));
        }
        typename U::T x[kUnroll];
        const char* sb = U::tile(src - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (tv0 + U::lane_unit(u) < sp.ve) x[u] = U::load(sb, U::lane_off(u));
        }
        char* tb = U::tile(a.recv[q] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (tv0 + U::lane_unit(u) < sp.ve) U::store(tb, U::lane_off(u), x[u]);
        }
    }
}

// Reduce-scatter: the fold of chunk c goes to rank c's shard only.  Reads N*S,
// writes S bytes.  NT_STORE: nontemporal stores (a standalone reduce-scatter)
// or cache-allocating ones (the phases' AllReduce, whose all-gather rereads
// the chunks: 32 x 128 MiB float32 1,597 -> 1,512 us, measured on MI355X).
template <int DT, int OP, int VEC, bool NT_STORE>
__global__ __launch_bounds__(kThreads) void k_fused_reduce_scatter(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    AR_TILE_LOOP_BEGIN
    char* shard = a.recv[c];
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            store_elem<elem_size<DT>(), NT_STORE>(shard + (i - sp.s) * elem_size<DT>(), fold_element<DT, OP>(a, c, i));
        }
    }
    const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
    typename Fold<DT, OP, VEC>::A acc[kUnroll];
    fold_units<DT, OP, VEC>(a, c, adj, tv0, live, acc);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) {
            store_shard_unit<DT, VEC, NT_STORE>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u),
                                      Fold<DT, OP, VEC>::done(acc[u], n));
        }
    }
    AR_TILE_LOOP_END
}

// All-gather: shard c (on rank c) goes to position start(c) of every rank
// (ALL = true) or of rank c only (ALL = false, the ring all-gather's first
// placement).  A store to the address it was loaded from is skipped (in place).
template <int DT, int VEC, bool ALL>
__global__ __launch_bounds__(kThreads) void k_gather_shards(const KernelArgs a) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    const char* shard = a.send[c];
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            const uint32_t x = load_elem<ESZ>(shard + (i - sp.s) * ESZ);
            for (int q = ALL ? 0 : c; q < (ALL ? n : c + 1); ++q) {
                char* dst = a.recv[q] + i * ESZ;
                if (dst != shard + (i - sp.s) * ESZ) store_elem<ESZ>(dst, x);
            }
        }
    }
    const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
    typename U::T x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) x[u] = load_shard_unit<DT, VEC, AR_NT_LOADS_COPY>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u));
    }
    for (int q = ALL ? 0 : c; q < (ALL ? n : c + 1); ++q) {
        if (a.recv[q] + sp.s * ESZ == shard) continue;   // the shard already sits there
        char* tb = U::tile(a.recv[q] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) U::store(tb, U::lane_off(u), x[u]);
        }
    }
    AR_TILE_LOOP_END
}

// k_gather_shards with one of a tile's kUnroll unit rows per block (grid of
// kUnroll blocks per tile): each wave issues half the stores, which HBM
// mostly takes faster.  With AR_GATHER_FORM=0 the host picks this form or
// k_gather_shards by measured shape; by default it takes k_gather_shards_xcd.
template <int DT, int VEC, bool ALL>
__global__ __launch_bounds__(kThreads) void k_gather_shards_half(const KernelArgs a) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    constexpr int ESZ = elem_size<DT>();
    const int n = a.nranks;
    const uint32_t tpc = a.tiles_per_chunk;
    const int64_t adj = (VEC > 1) ? static_cast<int64_t>(a.ofs) * ESZ : 0;
    const uint64_t parts = static_cast<uint64_t>(a.tile_end - a.tile_first) * kUnroll;
    for (uint64_t w = blockIdx.x; w < parts; w += gridDim.x) {
        const uint32_t tile = a.tile_first + static_cast<uint32_t>(w / kUnroll);
        const int u = static_cast<int>(w % kUnroll);
        const int c = static_cast<int>(tile / tpc);
        const uint64_t t = tile - static_cast<uint32_t>(c) * tpc;
        const Span sp = chunk_span<VEC>(c, a);
        const uint64_t tv0 = sp.vb + t * (kThreads * kUnroll);
        const char* shard = a.send[c];
        if (VEC > 1 && t == 0 && u == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) {
                const uint32_t x = load_elem<ESZ>(shard + (i - sp.s) * ESZ);
                for (int q = ALL ? 0 : c; q < (ALL ? n : c + 1); ++q) {
                    char* dst = a.recv[q] + i * ESZ;
                    if (dst != shard + (i - sp.s) * ESZ) store_elem<ESZ>(dst, x);
                }
            }
        }
        if (tv0 + U::lane_unit(u) < sp.ve) {
            const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
            const typename U::T x =
                load_shard_unit<DT, VEC, AR_NT_LOADS_COPY>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u));
            for (int q = ALL ? 0 : c; q < (ALL ? n : c + 1); ++q) {
                if (a.recv[q] + sp.s * ESZ == shard) continue;   // the shard already sits there
                U::store(U::tile(a.recv[q] - adj, tv0), U::lane_off(u), x);
            }
        }
    }
}

// The fused all-gather with one destination rank per block and a tile's N
// blocks on one XCD (as k_staged_broadcast_xcd): block b = x + 8 m copies tile
// tile_first + 8 (m / N) + x of its chunk's shard to rank m mod N, skipping
// the rank the shard already sits in (in place).  Strides over the same
// numbering when the grid is capped.
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_gather_shards_xcd(const KernelArgs a) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    constexpr int ESZ = elem_size<DT>();
    const int n = a.nranks;
    const uint32_t tpc = a.tiles_per_chunk;
    const int64_t adj = (VEC > 1) ? static_cast<int64_t>(a.ofs) * ESZ : 0;
    const uint64_t dests = static_cast<uint64_t>(n);
    const uint64_t groups = (static_cast<uint64_t>(a.tile_end - a.tile_first) + 7) / 8;
    const uint64_t total = 8 * groups * dests;
    for (uint64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const uint64_t m = b / 8;
        const uint64_t tile64 = a.tile_first + 8 * (m / dests) + (b % 8);
        if (tile64 >= a.tile_end) continue;
        const uint32_t tile = static_cast<uint32_t>(tile64);
        const int q = static_cast<int>(m % dests);
        const int c = static_cast<int>(tile / tpc);
        const uint64_t t = tile - static_cast<uint32_t>(c) * tpc;
        const Span sp = chunk_span<VEC>(c, a);
        const uint64_t tv0 = sp.vb + t * (kThreads * kUnroll);
        const char* shard = a.send[c];
        if (a.recv[q] + sp.s * ESZ == shard) continue;   // the shard already sits there
        if (VEC > 1 && t == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i))
                store_elem<ESZ>(a.recv[q] + i * ESZ, load_elem<ESZ>(shard + (i - sp.s) * ESZ));
        }
        const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
        typename U::T x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (tv0 + U::lane_unit(u) < sp.ve)
                x[u] = load_shard_unit<DT, VEC, AR_NT_LOADS_COPY>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u));
        }
        char* tb = U::tile(a.recv[q] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (tv0 + U::lane_unit(u) < sp.ve) U::store(tb, U::lane_off(u), x[u]);
        }
    }
}

// AllReduce of a small message: the ring-order fold of P = kThreads / N
// positions per block, staged through LDS.  Position i belongs to chunk
// c = floor(((i+1)*N - 1) / len), whose fold starts at rank c.  The thread
// that loads rank r's value of a position stores it at slot (r - c) mod N of
// that position's row, so the row holds the ranks in the fold's order
// c, c+1, ..., N-1, 0, ..., c-1 and the fold reads it straight through (the
// chunk's division is done while the loads are in flight, and the fold's
// steps carry no index arithmetic).  Rows are N | 1 words apart: an odd
// stride puts the lanes of a wave in distinct LDS banks.  In place is safe:
// a block loads all its positions from every rank before it stores any.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void k_small_allreduce(const KernelArgs a) {
    constexpr int ESZ = elem_size<DT>();
    using F = Fold<DT, OP, 1>;
    // P rows of N | 1 words: at most kThreads + P <= 3 * kThreads / 2 for N >= 2
    __shared__ uint32_t vals[2 * kThreads];
    __shared__ uint32_t res[kThreads];
    const int n = a.nranks;
    const int P = kThreads / n;
    const int S = n | 1;
    const int t = static_cast<int>(threadIdx.x);
    const int r = t / P;             // the rank this thread loads and stores
    const int j = t - r * P;         // the position it loads and stores, within the block
    const SmallPtrs q = small_ptrs(a, P);
    for (uint64_t i0 = static_cast<uint64_t>(xcd_grouped_block()) * P; i0 < a.count;
         i0 += static_cast<uint64_t>(gridDim.x) * P) {
        const uint64_t i = i0 + static_cast<uint64_t>(j);
        if (r < n && i < a.count) {
            const uint32_t v = load_elem<ESZ>(q.src + i * ESZ);
            const int c = static_cast<int>(((i + 1) * static_cast<uint64_t>(n) - 1) / a.count);
            const int k = r >= c ? r - c : r - c + n;
            vals[j * S + k] = v;
        }
        __syncthreads();
        if (t < P && i0 + t < a.count) {
            const uint32_t* row = vals + t * S;
            typename F::A acc = F::first(row[0]);
            for (int k = 1; k < n; ++k) acc = F::add(acc, row[k]);
            res[t] = F::done(acc, n);
        }
        __syncthreads();
        if (r < n && i < a.count) store_elem<ESZ>(q.dst + i * ESZ, res[j]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// ring steps: one launch per step of the schedule on tirogla.com "Ring
// all-reduce" ("How it works").  In one launch every chunk c is handled by
// the one rank that receives it in this step.
// ---------------------------------------------------------------------------

// AllReduce, reduce-scatter step s: rank r receives chunk (r-s-1) mod N from
// rank r-1 and adds its own values, i.e. chunk c is reduced on rank
// r = c+s+1 from rank p = c+s.  recv[r][chunk c] = send[r] (op) P, with
// P = send[p] at s = 0 and the partial recv[p] afterwards; the last step
// (s = N-2) completes the chunk (avg divides by N).  Reads 2*S and writes S
// bytes.  No rank writes what another rank reads in the same step (rank r
// writes chunk r-s-1, rank r+1 reads chunk r-s of rank r).  Types whose
// partials are kept in the buffer type only.
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_reduce_step(const KernelArgs a) {
    ring_reduce_tiles<DT, OP, VEC>(a, a.step);
}

// Reduce-scatter ring step s with the partial sums in a workspace.  Chunk c
// is reduced on rank r = c+s+1: its own value (op) the incoming partial,
// which is send[c] at s = 0 and the workspace afterwards.  The last step
// (s = N-2, on rank c-1) completes the chunk and writes it through
// recv[c], a pointer to where chunk c's element start(c) belongs: the shard
// of rank c (reduce-scatter), or chunk c of rank c-1's own buffer (the
// AllReduce ring of AR_BFLOAT16_ACC_F32, whose partials travel as float32).
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_reduce_step_ws(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    using F = Fold<DT, OP, VEC>;
    using F1 = Fold<DT, OP, 1>;
    using P = Partials<DT, VEC>;
    using P1 = Partials<DT, 1>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    const int r = ring_rank(c, a.step + 1, n);
    const char* local = a.send[r];
    const bool first_step = (a.step == 0);
    const bool last = (a.step == n - 2);
    char* shard = a.recv[c];
    const char* ws_base = a.ws - static_cast<int64_t>(a.ofs) * P::kElemBytes;
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            typename F1::A in;
            if (first_step) {
                in = F1::first(load_elem<ESZ>(a.send[c] + i * ESZ));
            } else {
                in = P1::load(a.ws, i);   // the workspace is touched only after the first step
            }
            const typename F1::A v = F1::add_acc(F1::first(load_elem<ESZ>(local + i * ESZ)), in);
            if (last) {
                store_elem<ESZ>(shard + (i - sp.s) * ESZ, F1::done(v, n));
            } else {
                P1::store(a.ws, i, v);
            }
        }
    }
    const bool aligned = shard_aligned<DT>(shard, sp.s, a.ofs);
    typename U::T x[kUnroll];
    typename F::A y[kUnroll];
    const char* tl = U::tile(local - adj, tv0);
    const char* ts = U::tile(a.send[c] - adj, tv0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) {
            x[u] = U::load(tl, U::lane_off(u));
            if (first_step) {
                y[u] = F::first(U::load(ts, U::lane_off(u)));
            } else {
                y[u] = P::load(ws_base, tv0 + U::lane_unit(u));
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (!live[u]) continue;
        const typename F::A z = F::add_acc(F::first(x[u]), y[u]);
        if (last) {
            store_shard_unit<DT, VEC>(shard, sp.s, a.ofs, aligned, tv0 + U::lane_unit(u), F::done(z, n));
        } else {
            P::store(const_cast<char*>(ws_base), tv0 + U::lane_unit(u), z);
        }
    }
    AR_TILE_LOOP_END
}

// All-gather ring step s: chunk c is copied from rank r-1 to rank
// r = c+s+shift.  shift = 0 is the AllReduce's all-gather phase (rank r
// receives chunk (r-s) mod N); shift = 1 is the standalone all-gather (rank r
// receives chunk (r-s-1) mod N, ramchalamkr.github.io "Ring All-Gather").
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_ring_copy_step(const KernelArgs a) {
    ring_copy_tiles<DT, VEC>(a, a.step, a.shift);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int DT, int OP, int VEC>
hipError_t launch_reduce(const Launch& l, const KernelArgs& a, hipStream_t s) {
    const dim3 grid(l.blocks), block(kThreads);
    switch (l.kind) {
        case Kind::kFusedAllReduce:
            if constexpr (VEC > 1) {
                if (l.cached) {
                    hipLaunchKernelGGL((k_fused_allreduce<DT, OP, VEC, false>), grid, block, 0, s, a);
                    break;
                }
            }
            hipLaunchKernelGGL((k_fused_allreduce<DT, OP, VEC, static_cast<bool>(AR_NT_LOADS)>), grid, block, 0, s, a);
            break;
        case Kind::kFusedReduceScatter:
            if (l.cached_store)
                hipLaunchKernelGGL((k_fused_reduce_scatter<DT, OP, VEC, false>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((k_fused_reduce_scatter<DT, OP, VEC, true>), grid, block, 0, s, a);
            break;
        case Kind::kStagedReduce:
            hipLaunchKernelGGL((k_staged_reduce<DT, OP, VEC>), grid, block, 0, s, a);
            break;
        case Kind::kRingReduceStep:
            if constexpr (acc_f32<DT>()) {
                return hipErrorInvalidValue;   // float32 partials always take the workspace step
            } else {
                hipLaunchKernelGGL((k_ring_reduce_step<DT, OP, VEC>), grid, block, 0, s, a);
            }
            break;
        case Kind::kRingReduceStepWs:
            hipLaunchKernelGGL((k_ring_reduce_step_ws<DT, OP, VEC>), grid, block, 0, s, a);
            break;
        case Kind::kSmallAllReduce:
            hipLaunchKernelGGL((k_small_allreduce<DT, OP>), grid, block, 0, s, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Copies depend on the element size only: the 2-byte types move as bf16
// elements, the 4-byte ones as float32 elements (bit patterns unchanged).
template <int DT, int VEC>
hipError_t launch_copy(const Launch& l, const KernelArgs& a, hipStream_t s) {
    const dim3 grid(l.blocks), block(kThreads);
    switch (l.kind) {
        case Kind::kFusedAllGather:
            if (l.form == 3)
                hipLaunchKernelGGL((k_gather_shards_xcd<DT, VEC>), grid, block, 0, s, a);
            else if (l.half)
                hipLaunchKernelGGL((k_gather_shards_half<DT, VEC, true>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((k_gather_shards<DT, VEC, true>), grid, block, 0, s, a);
            break;
        case Kind::kPlaceShards:
            hipLaunchKernelGGL((k_gather_shards<DT, VEC, false>), grid, block, 0, s, a);
            break;
        case Kind::kRingCopyStep:
            hipLaunchKernelGGL((k_ring_copy_step<DT, VEC>), grid, block, 0, s, a);
            break;
        case Kind::kStagedBroadcast:
            if (l.form == 3)
                hipLaunchKernelGGL((k_staged_broadcast_xcd<DT, VEC>), grid, block, 0, s, a);
            else if (l.half)
                hipLaunchKernelGGL((k_staged_broadcast<DT, VEC>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((k_staged_broadcast_tiles<DT, VEC>), grid, block, 0, s, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DT, int OP>
hipError_t by_vec(const Launch& l, const KernelArgs& a, hipStream_t s) {
    constexpr int V = 16 / elem_size<DT>();
    return l.vec ? launch_reduce<DT, OP, V>(l, a, s) : launch_reduce<DT, OP, 1>(l, a, s);
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

template <int DT>
hipError_t copy_by_vec(const Launch& l, const KernelArgs& a, hipStream_t s) {
    constexpr int V = 16 / elem_size<DT>();
    return l.vec ? launch_copy<DT, V>(l, a, s) : launch_copy<DT, 1>(l, a, s);
}

}  // namespace

hipError_t launch(const Launch& l, const KernelArgs& a, hipStream_t stream) {
    if (l.kind == Kind::kFusedTree || l.kind == Kind::kTreeReduceStep || l.kind == Kind::kTreeCopyStep ||
        l.kind == Kind::kSmallTree)
        return launch_tree(l, a, stream);
    if (l.kind == Kind::kFusedDbt || l.kind == Kind::kSmallDbt || l.kind == Kind::kDbtReduceStep ||
        l.kind == Kind::kDbtCopyStep)
        return launch_dbt(l, a, stream);
    if (l.kind == Kind::kRingPersistent || l.kind == Kind::kRingPipelined || l.kind == Kind::kRingPipelinedWs ||
        l.kind == Kind::kRingPipelinedGather)
        return launch_persistent(l, a, stream);
    const bool copy = l.kind == Kind::kFusedAllGather || l.kind == Kind::kPlaceShards ||
                      l.kind == Kind::kRingCopyStep || l.kind == Kind::kStagedBroadcast;
    if (copy) {
        const bool two_bytes = l.dtype == AR_BFLOAT16 || l.dtype == AR_FLOAT16 || l.dtype == AR_BFLOAT16_ACC_F32;
        return two_bytes ? copy_by_vec<AR_BFLOAT16>(l, a, stream) : copy_by_vec<AR_FLOAT32>(l, a, stream);
    }
    switch (l.dtype) {
        case AR_FLOAT32: return by_op<AR_FLOAT32>(l, a, stream);
        case AR_BFLOAT16: return by_op<AR_BFLOAT16>(l, a, stream);
        case AR_INT32: return by_op<AR_INT32>(l, a, stream);
        case AR_FLOAT16: return by_op<AR_FLOAT16>(l, a, stream);
        case AR_BFLOAT16_ACC_F32: return by_op<AR_BFLOAT16_ACC_F32>(l, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace arimpl
