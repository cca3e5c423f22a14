// Internal interface between the host entry points (ar_api.hip) and the
// kernel sources (ar_kernels.hip, which dispatches to ar_tree_kernels.hip,
// ar_dbt_kernels.hip and ar_persistent_kernels.hip).  Not installed;
// include/ar.h is the public ABI.
#pragma once

#include <cstdint>

#include "ar.h"

namespace arimpl {

constexpr int kThreads = 256;   // threads per block: four 64-wide wavefronts

// What one launch does.
enum class Kind : int {
    kFusedAllReduce = 0,   // reduce element i over all ranks, store to every rank
    kFusedReduceScatter,   // reduce element i over all ranks, store to the owner's shard
    kFusedAllGather,       // copy shard c to position start(c) of every rank
    kPlaceShards,          // copy shard c to position start(c) of rank c only
    kRingReduceStep,       // AllReduce ring, reduce-scatter step `step`
    kRingReduceStepWs,     // reduce-scatter ring, step `step`, partials in the workspace
    kRingCopyStep,         // all-gather ring step `step` (rank mapping shifted by `shift`)
    kFusedTree,            // reduce element i over all ranks in the binomial-tree bracketing of the
                           // send table's order, store to every rank
    kTreeReduceStep,       // one reducing stage of a tree-shaped schedule (`mode`, `step`)
    kTreeCopyStep,         // one distributing stage of a tree-shaped schedule (`mode`, `step`)
    kRingPersistent,       // all 2(N-1) ring steps in one cooperative launch
    kRingPipelined,        // all 2(N-1) ring steps in one launch, slice by slice
    kRingPipelinedWs,      // the same with the reduce-scatter partials in the workspace (`mode` 0:
                           // reduce-scatter into the shards; 1: AllReduce, then the all-gather steps)
    kRingPipelinedGather,  // the all-gather ring in one launch, slice by slice
    kSmallAllReduce,       // the fused AllReduce of a small message, staged through LDS
    kSmallTree,            // kFusedTree for a small message, staged through LDS
    kStagedReduce,         // kFusedAllReduce for tiles [tile_first, tile_end), stored to rank 0 only
    kStagedBroadcast,      // copy rank 0's result for tiles [tile_first, tile_end) to every other rank
    kFusedDbt,             // reduce each half of the buffer in its binary tree's bracketing (the
                           // double binary tree), store to every rank
    kDbtReduceStep,        // one reducing level of the double binary tree (`step` = height)
    kDbtCopyStep,          // one distributing level of the double binary tree (`step` = height)
    kSmallDbt,             // kFusedDbt for a small message, staged through LDS
};

// Stages of the tree-shaped schedules; at stage `step` the partner distance is d.
enum TreeMode : int {
    kTreeReduce = 0,       // binomial reduction, d = 2^step: rank r (r mod 2d == 0) adds rank r+d
    kTreeBcast = 1,        // binomial distribution, d = 2^step: rank r (r mod 2d == 0) sends to r+d
    kRdExchange = 2,       // recursive doubling, d = 2^step: ranks r and r^d both get r (op) r^d
    kHalvingReduce = 3,    // recursive halving, d = N / 2^(step+1): of each pair sharing chunk c,
                           // the rank whose bit d matches c's adds its partner's partial
    kDoublingGather = 4,   // recursive doubling all-gather, d = 2^step: chunk c goes to the ranks
                           // that lack it from their partner r^d
};

// Kernel arguments, passed by value.  Pointers are the callers' device
// addresses.  On the vector path every streamed full-length buffer p has the
// same residue `ofs` elements modulo A = 2^align_shift elements (A * element
// size is 256 bytes when the buffers allow it, and at least 16), so its
// 16-byte vector v starts at (p - ofs elements) + 16*v and holds elements
// [v*V - ofs, (v+1)*V - ofs), V = 16 / element size.  Each chunk's body of
// vectors starts and ends on an A-element boundary in every buffer, so whole
// cache lines are written; the few elements before and after it are done one
// at a time.
struct KernelArgs {
    const char* send[AR_MAX_RANKS];
    char* recv[AR_MAX_RANKS];
    char* ws;                  // workspace for kRingReduceStepWs (already residue-adjusted)
    uint64_t count;            // elements per rank (full length)
    uint64_t count_q;          // count / nranks
    uint32_t count_r;          // count % nranks: start(c) = c*count_q + (c*count_r)/nranks
    uint32_t tiles_per_chunk;  // grid tiles that cover one chunk's body
    uint32_t tile_first;       // this launch covers tiles [tile_first, tile_end) of N * tiles_per_chunk
    uint32_t tile_end;
    int32_t nranks;
    int32_t step;              // ring step s
    int32_t shift;             // kRingCopyStep: acting rank = (c + step + shift) mod N
    int32_t ofs;               // common element residue of the streamed buffers modulo the body alignment
    int32_t align_shift;       // log2 of the body alignment in elements (vector path)
    int32_t mode;              // kTree*Step: a TreeMode
    int32_t last;              // kTreeReduceStep: nonzero on the stage that completes the values
    uint64_t ws_stride;        // kTreeReduceStep with float32 partials: bytes between ranks' partials
    int32_t xcd_slabs;         // tiled kernels: nonzero walks the tiles in one contiguous slab per XCD
};

struct Launch {
    Kind kind;
    ar_dtype_t dtype;
    ar_op_t op;
    bool vec;                  // 16-byte vector path (all streamed buffers share a residue)
    bool cached;               // one-pass AllReduces (ring and tree orders) on the vector path: cache-allocating loads
    bool half;                 // kFusedAllGather, kStagedBroadcast: one unit row of a tile per block
    int form;                  // kStagedBroadcast, kFusedAllGather: 3 one destination per block, a
                               // tile's blocks grouped on one XCD; 0 the tile forms above
    bool cached_store;         // kFusedReduceScatter: cache-allocating stores of the shards (the
                               // phases' AllReduce, whose all-gather rereads them)
    unsigned blocks;
    int depth;                 // kFusedTree: partial slots, 2^depth > N (4, 6 or 8); kFusedDbt: stack
                               // slots (4 below 16 ranks, else 6)
    unsigned actors;           // kTree*Step, kDbt*Step: actors per chunk in the stage (the grid's y extent)
};

// Vectors of 16 bytes each thread handles per rank per tile.
#ifndef AR_TILE_UNROLL
#define AR_TILE_UNROLL 2
#endif
constexpr int kUnroll = AR_TILE_UNROLL;

// Inputs of at most this many bytes in total (N * S) are read by the fused
// AllReduce with cache-allocating loads instead of nontemporal ones: they fit
// in MI355X's 256 MB Infinity Cache, so a call that reads the same buffers
// again finds them there.  Measured on MI355X at 8 ranks, float32, per call
// in a replayed graph: 2^20 per rank 9.7 -> 9.0 us, 2^22 45.8 -> 43.0 us,
// 2^23 (256 MiB of inputs) 92 -> 80 us; from 512 MiB on, nontemporal loads
// win (2^24 per rank: 186.5 against 197 us).
#ifndef AR_CACHED_LOADS_MAX_BYTES
#define AR_CACHED_LOADS_MAX_BYTES (256ull << 20)
#endif

// AR_ALGO_STAGED: rank 0's results per segment (one reducing and one
// broadcasting launch each) are about AR_STAGE_READ_BYTES / N bytes, kept
// between AR_STAGE_BYTES_MIN and AR_STAGE_BYTES_MAX.  The broadcast rereads
// them, so they should stay in MI355X's 256 MB Infinity Cache between the two
// launches.  Measured on MI355X, float32, 256 MiB per rank, median us per
// call, 32 MiB / 128 MiB segments: 8 ranks 740 / 736, 16 ranks 1,513 /
// 1,519, 32 ranks 2,979 / 3,002, 64 ranks 5,944 / 6,028, 128 ranks 11,701 /
// 11,728.
#ifndef AR_STAGE_READ_BYTES
#define AR_STAGE_READ_BYTES (2048ull << 20)
#endif
#ifndef AR_STAGE_BYTES_MIN
#define AR_STAGE_BYTES_MIN (32ull << 20)
#endif
#ifndef AR_STAGE_BYTES_MAX
#define AR_STAGE_BYTES_MAX (128ull << 20)
#endif

// Rank count from which the launches that stream every rank's buffer at once
// walk their tiles in one contiguous slab per XCD (tile_walk); 0 never.
// Measured on MI355X, the same buffers in one process, plain / slabs, us:
// 64 x 16 MiB float32 fused 427 / 395, staged 386 / 370, phases 378 / 364;
// 128 x 64 MiB fused 3,351 / 3,285, staged 2,986 / 2,934; 64 x 256 MiB
// phases 6,412 / 6,096, fused and staged within 1 %; 32 x 256 MiB within
// 1.5 % (staged slower); 8 x 256 MiB fused 741 / 790 (slower).  The
// standalone fused reduce-scatter: 64 x 16 MiB 187.7 / 180.7, 128 x 64 MiB
// 1,395 / 1,380, 64 x (2^26+7) 2,910 / 2,909, 32 x 256 MiB 1,551 / 1,566.
// The fused AllReduce takes slabs more widely (its rule is kept with the
// host's dispatch).
#ifndef AR_TILE_XCD_MIN_RANKS
#define AR_TILE_XCD_MIN_RANKS 64
#endif

// The copy launches that write one value to many ranks (the fused all-gather
// and the staged AllReduce's broadcast) give each block one of a tile's
// kUnroll unit rows when the ranks' buffers hold between
// AR_HALF_TILES_MIN_TOTAL and AR_HALF_TILES_MAX_TOTAL bytes in all (N * S);
// outside that band whole tiles per block are faster.  This applies to the
// tile forms only (AR_BCAST_FORM=0, AR_GATHER_FORM=0); by default both copies
// give each block one destination rank, a tile's blocks grouped on one XCD.  Measured on MI355X,
// float32, same box, staged AllReduce whole / half tiles in us: inside the
// band 8 x 256 MiB 736 / 723, 16 x 256 MiB 1,509 / 1,461, 64 x 64 MiB
// 1,559 / 1,527, 32 x 128 MiB 1,519 / 1,495; below it 8 x 4 MiB 19.1 / 21.3,
// 16 x 64 MiB 396 / 415, 64 x 16 MiB 419 / 473; above it 32 x 256 MiB
// 2,984 / 3,046, 64 x 256 MiB 5,928 / 6,341.  The all-gather follows the
// same band (64 x 16 MiB 235 / 284 us; 16 x 256 MiB 785 / 736 us).
#ifndef AR_HALF_TILES_MIN_TOTAL
#define AR_HALF_TILES_MIN_TOTAL (2048ull << 20)
#endif
#ifndef AR_HALF_TILES_MAX_TOTAL
#define AR_HALF_TILES_MAX_TOTAL (8192ull << 20)
#endif

// Replace the calling thread's error text (what ar_get_last_error_detail
// returns) for a failure found outside ar_api.hip.
void set_error_detail(const char* text);

// Enqueue one kernel; returns the HIP error of the launch.
hipError_t launch(const Launch& l, const KernelArgs& a, hipStream_t stream);

// The kernels of the tree-shaped schedules (ar_tree_kernels.hip); `launch`
// forwards the kFusedTree, kSmallTree, kTreeReduceStep and kTreeCopyStep
// kinds here.
hipError_t launch_tree(const Launch& l, const KernelArgs& a, hipStream_t stream);

// The double binary tree (ar_dbt_kernels.hip); `launch` forwards the
// kFusedDbt, kSmallDbt, kDbtReduceStep and kDbtCopyStep kinds here.  Their tile loop
// cuts the buffer in two parts (count_q = count / 2, count_r = count % 2).
hipError_t launch_dbt(const Launch& l, const KernelArgs& a, hipStream_t stream);

// The ring in one launch (ar_persistent_kernels.hip).  kRingPersistent: a
// cooperative launch on at most as many blocks as the device holds at once;
// refuses (hipErrorStreamCaptureUnsupported) while `stream` is capturing.
// kRingPipelined, kRingPipelinedWs, kRingPipelinedGather: ordinary launches,
// one block per slice.
hipError_t launch_persistent(const Launch& l, const KernelArgs& a, hipStream_t stream);

}  // namespace arimpl
