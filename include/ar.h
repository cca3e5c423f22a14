/*
 * ar.h — ring AllReduce over N virtual ranks resident in one GPU's HBM.
 *
 * C ABI of libar.so.  Calls keep no state from one to the next (tirogla.com
 * "Ring all-reduce", section "How it works", the line that states the
 * collective's inputs, outputs and state), and every call is asynchronous:
 * it validates its arguments on the host, enqueues kernels on `stream` and
 * returns.  The arguments follow the collective's statement
 * on arjunsriva.com "AllReduce, All the Way Down", section "The Contract"
 * (send buffer, receive buffer, count, datatype, reduction, participants,
 * stream), with the communicator replaced by the number of virtual ranks and
 * one send and one receive pointer per rank.
 *
 * Virtual rank r owns the device buffers sendbufs[r] and recvbufs[r].
 * `count` is always the FULL per-rank length `len` in elements.  The ring
 * cuts it into N chunks, chunk(c) = [c*len/N, (c+1)*len/N) with floor
 * division (tirogla.com "Ring all-reduce", section "Code"); chunks may be
 * uneven and, when len < N, empty.  cl(c) below is the length of chunk c.
 *
 * Result ("ring association order").  Element i of chunk c is reduced as it
 * travels the ring from rank c: ((x_c (op) x_{c+1}) (op) x_{c+2}) ... with
 * ranks taken mod N and the result rounded to the buffer type after every
 * operation (arjunsriva.com, figure "Ring AllReduce · follow chunk 0";
 * tirogla.com "Ring all-reduce", "How it works").  The ring-order algorithms below give
 * these bits exactly, and every rank receives identical bits.
 *
 * Pointers.  `sendbufs` and `recvbufs` are HOST arrays of `nranks` DEVICE
 * pointers; the arrays are read during the call only and may be freed when
 * it returns.  The device buffers are owned by the caller and must stay
 * valid until the work enqueued on `stream` completes.  The one-shot calls
 * take the pointers on trust (asking the runtime about every buffer would
 * cost as much as a small collective): a host pointer, or a count beyond a
 * buffer's allocation, makes their kernels fault.  The *_init calls below
 * check where the buffers live, once.  Buffers need only be
 * aligned to their element size; when all the buffers a kernel streams share
 * the same address residue modulo 16 bytes the kernels move 16-byte vectors,
 * otherwise one element at a time (same results, lower bandwidth).
 *
 * Aliasing.  In place is allowed: AllReduce with sendbufs[r] == recvbufs[r];
 * reduce-scatter with recvbufs[r] == sendbufs[r] + start(r) elements;
 * all-gather with sendbufs[r] == recvbufs[r] + start(r) elements.  Receive
 * buffers that overlap each other, or that overlap a send buffer in any
 * other way, are rejected with AR_ERR_INVALID_ARGUMENT.
 *
 * Errors.  All validation happens before anything is enqueued; a call that
 * returns an error has launched nothing.  count == 0 is a successful no-op.
 * A HIP launch failure returns AR_ERR_HIP.  ar_get_last_error_detail()
 * describes the most recent failure of the calling thread.
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of virtual ranks one call accepts (the pointer tables travel
 * in the kernel arguments). */
#define AR_MAX_RANKS 128

typedef enum {
    AR_SUCCESS = 0,
    AR_ERR_INVALID_ARGUMENT = 1,
    AR_ERR_UNSUPPORTED = 2,
    AR_ERR_HIP = 3,
    AR_ERR_INTERNAL = 4
} ar_result_t;

/* Element types.  AR_BFLOAT16 and AR_FLOAT16 results are rounded to the
 * 16-bit type (nearest, ties to even) after every ring step, as a ring that
 * keeps 16-bit buffers does.  AR_BFLOAT16_ACC_F32 has bf16 buffers but keeps
 * the partial sums in float32 and rounds to bf16 once, when a chunk is
 * complete (tirogla.com "Ring all-reduce", implementation notes: reduce in
 * fp32, or at least bf16 with fp32 accumulation). */
typedef enum {
    AR_FLOAT32 = 0,
    AR_BFLOAT16 = 1,
    AR_INT32 = 2,
    AR_FLOAT16 = 3,
    AR_BFLOAT16_ACC_F32 = 4
} ar_dtype_t;

/* Reduction operators (sum, product, minimum, maximum, average: bitfern.com
 * "AllReduce Explained", section "What Is AllReduce?").  int32 sum and
 * product wrap modulo 2^32.  Float min/max are IEEE 754-2019 minimum and
 * maximum: a NaN operand gives NaN, and -0 < +0.  AR_AVG is the ring's sum
 * divided by nranks once, when a chunk is complete ("2.1 Collective
 * communication primitives in detail", section 3.4: sum, then divide by N):
 * a float quotient rounded once to the buffer type, or an int32 quotient
 * truncated toward zero from the wrapped sum. */
typedef enum {
    AR_SUM = 0,
    AR_PROD = 1,
    AR_MIN = 2,
    AR_MAX = 3,
    AR_AVG = 4
} ar_op_t;

/* AR_ALGO_FUSED: one kernel reads element i from all N ranks, reduces it in
 *   ring order and writes every output (N*S bytes read, N*S written for
 *   AllReduce: the minimum).  Inputs of at most 256 MiB in total (N*S) are
 *   read with cache-allocating loads, so that a repeated call finds them in
 *   the device's 256 MB last-level cache; larger ones stream past it.  The
 *   choice affects speed only, never the result.
 * AR_ALGO_RING: the ring's steps one by one, one kernel launch per step:
 *   N-1 reduce-scatter steps then N-1 all-gather steps, each rank adding the
 *   chunk received from rank r-1 (tirogla.com "Ring all-reduce", "How it
 *   works").
 * AR_ALGO_PHASES: AllReduce as reduce-scatter followed by all-gather ("2.1
 *   Collective communication primitives in detail", section 3.8), each phase
 *   one fused pass: the reduced chunk c lands in chunk c of recvbufs[c]
 *   (cache-allocating stores), then is copied to every other rank, each
 *   destination by its own workgroup, a tile's workgroups on one XCD.  The
 *   copy rereads S bytes, partly from the last-level cache, beyond the fused
 *   kernel's 2N*S, but the read-heavy and the write-heavy halves run apart,
 *   which MI355X HBM serves faster for large buffers.
 * AR_ALGO_AUTO: for AllReduce, by shape (rules below): AR_ALGO_PHASES or
 *   AR_ALGO_STAGED for large buffers, AR_ALGO_PHASES at many ranks,
 *   AR_ALGO_FUSED otherwise; the fused kernel for the single phases.
 * These four give the same bits: the ring's association order.
 *
 * The remaining algorithms are AllReduce only (AR_ERR_UNSUPPORTED for
 * reduce-scatter and all-gather) and bracket the reduction differently from
 * the ring, so their float results differ from the ring's in the last bits:
 * AR_ALGO_TREE: the binomial tree of bitfern.com "AllReduce Explained"
 *   (section "Tree AllReduce": reduce toward a root, then send the result
 *   back down): rank r (r mod 2d = 0) adds the partial of rank r+d for
 *   d = 1, 2, 4, ..., so element i is ((x0 x1)(x2 x3))((x4 x5)(x6 x7))...
 *   for any N.  One fused pass (2*N*S bytes).
 * AR_ALGO_TREE_STEPS: the same tree stage by stage: ceil(log2 N) reducing
 *   launches toward rank 0, then as many distributing launches.
 * AR_ALGO_RECURSIVE_DOUBLING: the same bracketing reached by exchanges
 *   (same section, "Recursive Doubling"): log2 N launches, in launch k rank
 *   r and rank r XOR 2^k both get r (op) r XOR 2^k.  N a power of two.
 * AR_ALGO_HALVING_DOUBLING: Rabenseifner's order (tirogla.com "Ring
 *   all-reduce", "How it works", cost model: recursive-halving
 *   reduce-scatter, recursive-doubling all-gather): partners at distance
 *   N/2 first, so element i is ((x0 x4)(x2 x6))((x1 x5)(x3 x7)) at N = 8.
 *   One fused pass.  N a power of two.
 * AR_ALGO_HALVING_DOUBLING_STEPS: the same schedule stage by stage: log2 N
 *   recursive-halving launches (chunk c finishes on rank c), then log2 N
 *   recursive-doubling launches.  N a power of two.
 * A power-of-two algorithm with another N fails with AR_ERR_UNSUPPORTED.
 *
 * AR_ALGO_RING_PERSISTENT: the ring's 2(N-1) steps (the same work and the
 *   same bits as AR_ALGO_RING) in one cooperative launch, with a grid-wide
 *   barrier where AR_ALGO_RING has a kernel boundary.  AllReduce only; not
 *   for AR_BFLOAT16_ACC_F32 (AR_ERR_UNSUPPORTED).  It cannot be enqueued
 *   while the stream is being captured into a graph (AR_ERR_UNSUPPORTED),
 *   and, since its blocks must all be resident at once, it should not
 *   overlap other kernels on the device.
 * AR_ALGO_RING_PIPELINED: the ring's steps in one ordinary launch, slices
 *   of the chunks pipelined through the ring ("AllReduce, All the Way Down":
 *   the tensor divided into chunks that are pipelined).  One workgroup
 *   carries one slice of one chunk through every step in order, loading the
 *   sender's partial and storing its own, so the steps need no barrier.  The
 *   same bits as AR_ALGO_RING, for all three collectives and every dtype,
 *   with the same workspace as AR_ALGO_RING; can be captured into a graph.
 * AR_ALGO_STAGED: AllReduce moved as a reduce followed by a broadcast
 *   (bitfern.com "AllReduce Explained", section "Reduce Followed by
 *   Broadcast"; "2.1 Collective communication primitives in detail",
 *   section 3.3, the note that AllReduce is Reduce plus Broadcast), with the
 *   ring's association order kept, cut into segments of rank 0's results.
 *   Per segment, one launch folds every position in ring order and stores
 *   the result to recvbufs[0] only, then one launch copies it to the other
 *   ranks, each destination by its own workgroup, a tile's workgroups on one
 *   XCD (AR_BCAST_FORM=0: whole or half tiles to every rank per
 *   workgroup).  The results are reread from the device's 256 MB last-level
 *   cache, so HBM still moves N*S read and N*S written; the reading and the
 *   writing launches run apart, which MI355X HBM serves faster than the two
 *   interleaved.  The same bits as AR_ALGO_FUSED.  AllReduce only; 2
 *   launches per segment.  A segment holds about 2 GiB / N of results,
 *   between 32 and 128 MiB; the AR_STAGE_BYTES environment variable sets it
 *   in bytes instead.
 * AR_ALGO_DOUBLE_BINARY_TREE: the double binary tree (tirogla.com "Ring
 *   all-reduce", "How it works", cost model: about 2 log2 N latency terms
 *   and 2 S/B; NCCL's choice for small messages at large N), built as
 *   Sanders, Speck and Traff's two trees ("Two-tree algorithms for full
 *   bandwidth broadcast, reduction and scan", 2009): the buffer's floor
 *   halves [0, count/2) and [count/2, count) are reduced in two binary trees
 *   over the ranks, no rank an inner node of both.  Tree 0 is the in-order
 *   tree over positions 1..N holding ranks 0..N-1 (position p's height is its
 *   trailing zero bits; an inner node p of height h has children
 *   p - 2^(h-1) and p + 2^j for the largest j < h with p + 2^j <= N); tree 1
 *   is the same with every rank moved on by one.  A node combines
 *   ((left (op) own) (op) right): at N = 8 half 0 is
 *   ((((((x0 x1) x2) x3) ((x4 x5) x6)) x7) and half 1 the same over ranks
 *   1, 2, ..., 7, 0.  One fused pass (2*N*S bytes), any N.
 * AR_ALGO_DOUBLE_BINARY_TREE_STEPS: the same trees level by level:
 *   floor(log2 N) reducing launches up both trees at once, then as many
 *   distributing launches down them.  AR_BFLOAT16_ACC_F32 keeps its float32
 *   partials in a workspace, one count-element slab per rank. */
typedef enum {
    AR_ALGO_FUSED = 0,
    AR_ALGO_RING = 1,
    AR_ALGO_PHASES = 2,
    AR_ALGO_AUTO = 3,
    AR_ALGO_TREE = 4,
    AR_ALGO_TREE_STEPS = 5,
    AR_ALGO_RECURSIVE_DOUBLING = 6,
    AR_ALGO_HALVING_DOUBLING = 7,
    AR_ALGO_HALVING_DOUBLING_STEPS = 8,
    AR_ALGO_RING_PERSISTENT = 9,
    AR_ALGO_RING_PIPELINED = 10,
    AR_ALGO_STAGED = 11,
    AR_ALGO_DOUBLE_BINARY_TREE = 12,
    AR_ALGO_DOUBLE_BINARY_TREE_STEPS = 13
} ar_algo_t;

/* AR_ALGO_AUTO's choice for an AllReduce, from side-by-side timings of the
 * three forms on MI355X, fused / phases / staged, in microseconds, float32
 * unless noted.  Two regimes were measured:
 * (a) steady state (bench.py --form-sweep; median of three processes, each
 *     after many calls):
 *   8 x 256 MiB 753 / 718 / 722; 8 x 128 MiB 372 / 359 / 368; 8 x 64 MiB
 *   188 / 184 / 196; 8 x 32 MiB 83 / 96 / 97; 16 x 256 MiB 1,587 / 1,417 /
 *   1,470; 16 x 64 MiB 392 / 362 / 362; 16 x 16 MiB 87 / 95 / 94; 32 x 32 MiB
 *   421 / 374 / 387; 64 x 64 MiB 1,677 / 1,549 / 1,564; 64 x 16 MiB 415 / 398
 *   / 400; 128 x 64 MiB 3,367 / 2,981 / 3,012; 6 x 256 MiB 547 / 561 / 536;
 *   4 x 256 MiB 362 / 370 / 363; 2 x 512 MiB 382 / 484 / 429; bf16 8 x 128
 *   MiB 403 / 368 / 365, 8 x 64 MiB 201 / 190 / 186, 16 x 64 MiB 410 / 356 /
 *   365; int32 16 x 64 MiB 389 / 359 / 354.
 * (b) a fresh process, after 2 s idle, mean of calls 6 to 25: the two
 *     phases' in-place gather runs 3-8 % slow over its first twenty or so
 *     calls; the other forms do not:
 *   8 x 256 MiB 753 / 751 / 732; 8 x 64 MiB 197 / 204 / 193; 16 x 64 MiB 405
 *   / 395 / 381; 32 x 32 MiB 448 / 407 / 398; 16 x 256 MiB 1,575 / 1,420 /
 *   1,438; 64 x 64 MiB 1,694 / 1,522 / 1,546; bf16 8 x 128 MiB 396 / 413 /
 *   385, 16 x 64 MiB 415 / 403 / 389, 16 x 32 MiB 220 / 216 / 205, 32 x 32
 *   MiB 452 / 409 / 413; phases / staged only, two processes each: 32 x 256
 *   MiB 2,873 and 2,862 / 2,910 and 2,921; 16 x 512 MiB 3,518 and 3,536 /
 *   3,178 and 3,168; 48 x 256 MiB 4,646 and 4,927 / 4,449 and 4,483; 64 x
 *   256 MiB 6,279 and 6,087 / 5,981 and 6,098; 128 x 128 MiB 6,202 and
 *   6,118 / 6,056 and 6,046.
 * The rules follow (b) where the two disagree, in order:
 *   1. AR_ALGO_PHASES from AR_BIG_PHASES_MIN_RANKS ranks with at least
 *      AR_BIG_PHASES_MIN_TOTAL_BYTES and at most
 *      AR_BIG_PHASES_MAX_TOTAL_BYTES over all ranks, and at most
 *      AR_BIG_PHASES_MAX_RANK_BYTES per rank (beyond those the staged form
 *      leads by 2-10 %, within them the phases by 1-2 %);
 *   2. AR_ALGO_STAGED from AR_STAGED_MIN_RANKS ranks with at least
 *      AR_STAGED_MIN_BYTES per rank and AR_STAGED_MIN_TOTAL_BYTES in all
 *      (16-bit types: the _16BIT bounds);
 *   3. AR_ALGO_PHASES from AR_PHASES_MIN_RANKS ranks with at least
 *      AR_PHASES_MIN_BYTES per rank and more than
 *      AR_PHASES_ABOVE_TOTAL_BYTES in all (up to that size the fused kernel
 *      reads its inputs through the last-level cache and leads: fused /
 *      phases, median of single calls, us: 24 x 8 MiB 76 / 85, 32 x 8 MiB
 *      97 / 109, 48 x 5 MiB 104 / 118, 64 x 4 MiB 122 / 125; above it 24 x
 *      12 MiB 130 / 119, 32 x 12 MiB 174 / 153, 64 x 6 MiB 175 / 158);
 *   4. AR_ALGO_FUSED.
 * Every choice gives the same bits. */
#define AR_BIG_PHASES_MIN_RANKS 16
#define AR_BIG_PHASES_MIN_TOTAL_BYTES (4ull << 30)
#define AR_BIG_PHASES_MAX_TOTAL_BYTES (8ull << 30)
#define AR_BIG_PHASES_MAX_RANK_BYTES (256ull << 20)
#define AR_STAGED_MIN_RANKS 6
#define AR_STAGED_MIN_BYTES (32ull << 20)
#define AR_STAGED_MIN_TOTAL_BYTES (1024ull << 20)
#define AR_STAGED_MIN_BYTES_16BIT (32ull << 20)
#define AR_STAGED_MIN_TOTAL_BYTES_16BIT (512ull << 20)
/* Rank count from which AR_ALGO_AUTO runs an AllReduce as two fused phases
 * (measured crossover on MI355X; the AR_PHASES_MIN_RANKS environment variable
 * overrides it). */
#define AR_PHASES_MIN_RANKS 24
/* Bytes per rank from which AR_ALGO_AUTO may take the two phases (measured
 * on MI355X: below it the single fused kernel is faster at every rank count). */
#define AR_PHASES_MIN_BYTES (4u << 20)
/* Bytes in all that rule 3 requires the inputs to exceed: the fused kernel's
 * cache-allocating loads reach up to here. */
#define AR_PHASES_ABOVE_TOTAL_BYTES (256ull << 20)

/* Environment variables.  They tune speed only; no setting changes a
 * result's bits.
 *   AR_STAGE_BYTES       AR_ALGO_STAGED: bytes of results per segment (read
 *                        at every call; a plan keeps what it was built with)
 *   AR_BCAST_FORM        0: the staged broadcast with whole or half tiles
 *                        to every rank per workgroup instead of one
 *                        destination per workgroup (read at every call)
 *   AR_GATHER_FORM       0: the same for the fused all-gather (read at
 *                        every call)
 *   AR_HALF_TILES        0 or 1: with AR_BCAST_FORM=0 or AR_GATHER_FORM=0,
 *                        whole tiles or half tiles per workgroup (read at
 *                        every call; unset: chosen by size)
 *   AR_TILE_XCD          rank count from which the fused AllReduce, the
 *                        staged reduce and the fused reduce-scatter walk
 *                        their tiles in one contiguous slab per XCD (fewer
 *                        pages for each XCD to translate; unset: 64, and
 *                        for the fused AllReduce 32, or any rank count when
 *                        its inputs hold 64-256 MiB in all; 0: never; read
 *                        at every call)
 *   AR_PHASES_MIN_RANKS  AR_ALGO_AUTO's rank bound for AR_ALGO_PHASES
 *   AR_SMALL_COUNT_MAX   elements per rank up to which the one-pass kernels
 *                        stage a few positions of every rank in LDS
 *                        (default 2^16; 0: never)
 *   AR_SMALL_WORK_MAX    bound on N * count for the same kernels, ring order
 *                        (default 2^21 elements)
 *   AR_SMALL_TREE_MAX    bound on N * S, in bytes, for the tree orders'
 *                        small-message kernels (default 8 MiB)
 *   AR_CACHED_LOADS_MAX  input bytes (N*S) up to which the fused AllReduce
 *                        reads with cache-allocating loads; 0: never
 *   AR_BLOCKS_PER_CU     cap the tiled kernels' grids at this many workgroups
 *                        per compute unit (they stride over the rest); 0:
 *                        one workgroup per tile
 *   AR_DEBUG             nonzero: print every planned launch to stderr
 * All but the first five are read once per process. */

typedef enum {
    AR_COLL_ALLREDUCE = 0,
    AR_COLL_REDUCE_SCATTER = 1,
    AR_COLL_ALL_GATHER = 2
} ar_coll_t;

/* AllReduce (tirogla.com "Ring all-reduce"; "2.1 Collective communication
 * primitives in detail", section 3.4): every recvbufs[r] (count elements)
 * receives the reduction of all sendbufs[*] (count elements each).
 * Algorithm AR_ALGO_AUTO. */
ar_result_t ar_allreduce(const void* const* sendbufs, void* const* recvbufs, size_t count,
                         ar_dtype_t dtype, ar_op_t op, int nranks, hipStream_t stream);

/* Reduce-scatter ("2.1 Collective communication primitives in detail",
 * section 3.5: rank i keeps reduced shard i): sendbufs[r] holds count
 * elements; recvbufs[r] receives the cl(r) elements of chunk r of the
 * reduction, packed.  The association order is AllReduce's, so
 * all-gather after reduce-scatter reproduces AllReduce bit for bit.  Fused
 * algorithm (AR_ALGO_PHASES and AR_ALGO_AUTO mean the same here). */
ar_result_t ar_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, size_t count,
                              ar_dtype_t dtype, ar_op_t op, int nranks, hipStream_t stream);

/* All-gather (ramchalamkr.github.io "NCCL Primitives Deep Dive", section
 * "Ring All-Gather"; "2.1 ...", section 3.6): sendbufs[r] holds shard r,
 * cl(r) elements; every recvbufs[r] (count elements) receives all shards
 * concatenated in rank order.  No arithmetic.  Fused algorithm
 * (AR_ALGO_PHASES and AR_ALGO_AUTO mean the same here). */
ar_result_t ar_all_gather(const void* const* sendbufs, void* const* recvbufs, size_t count,
                          ar_dtype_t dtype, int nranks, hipStream_t stream);

/* The same three collectives with the algorithm chosen by the caller.
 * Reduce-scatter and all-gather take AR_ALGO_RING (one launch per step) and
 * AR_ALGO_RING_PIPELINED (the steps in one launch); AR_ALGO_FUSED,
 * AR_ALGO_PHASES and AR_ALGO_AUTO all mean their fused kernel; the tree
 * orders and AR_ALGO_RING_PERSISTENT are AllReduce only (AR_ERR_UNSUPPORTED).
 * `workspace` is device memory of at least ar_workspace_bytes(...) bytes
 * owned by the caller (NULL when that size is 0); it must not overlap any
 * buffer and must stay valid until the stream work completes.  Only the ring
 * algorithms (AR_ALGO_RING and AR_ALGO_RING_PIPELINED) need one, for
 * nranks >= 3: the reduce-scatter keeps the partial
 * sums in flight between steps in it, since its receive buffers are only one
 * shard long, and so does the AllReduce of AR_BFLOAT16_ACC_F32, whose float32
 * partials do not fit the bf16 buffers.  Other ring AllReduces and the ring
 * all-gather work in recvbufs.  The staged tree algorithms
 * (AR_ALGO_TREE_STEPS, AR_ALGO_RECURSIVE_DOUBLING,
 * AR_ALGO_HALVING_DOUBLING_STEPS, AR_ALGO_DOUBLE_BINARY_TREE_STEPS) keep
 * their partials in recvbufs too,
 * except for AR_BFLOAT16_ACC_F32, whose float32 partials take one
 * count-element float32 slab per rank in the workspace (nranks >= 2). */
ar_result_t ar_allreduce_ex(const void* const* sendbufs, void* const* recvbufs, size_t count,
                            ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
ar_result_t ar_reduce_scatter_ex(const void* const* sendbufs, void* const* recvbufs, size_t count,
                                 ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
ar_result_t ar_all_gather_ex(const void* const* sendbufs, void* const* recvbufs, size_t count,
                             ar_dtype_t dtype, int nranks, ar_algo_t algo,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Reduce-scatter that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same call, rules, errors and results as
 * ar_reduce_scatter_ex with `algo`, except that the workspace the ring
 * algorithms need (ar_workspace_bytes) is not passed in: it is a fixed array
 * of AR_NOALLOC_SCRATCH_BYTES in device memory inside the library.  Each
 * device holds its own copy from the first call on it until the process ends;
 * that first call looks its address up (hipGetSymbolAddress), so make it
 * outside a graph capture.  A call whose workspace would exceed
 * AR_NOALLOC_SCRATCH_BYTES fails with AR_ERR_INVALID_ARGUMENT and launches
 * nothing (float32 ring: up to 16M - 256 elements per rank).  Nothing in the
 * array needs to start at zero, and each call overwrites what it uses, but
 * every call on one device shares the one array: calls whose work overlaps
 * on the same GPU (other streams, or concurrent host threads) race and give
 * wrong results.  Algorithms that need no workspace touch the array not at
 * all.  No call here allocates device memory. */
#define AR_NOALLOC_SCRATCH_BYTES (64ull << 20)
ar_result_t ar_reduce_scatter_noalloc(const void* const* sendbufs, void* const* recvbufs, size_t count,
                                      ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo,
                                      hipStream_t stream);

/* Persistent collectives, in the manner of MPI's persistent AllReduce request
 * (bitfern.com "AllReduce Explained", section "MPI_Allreduce"): *_init
 * validates the arguments and plans the launches once, with the same
 * arguments, rules and errors as the matching *_ex call, and one check more:
 * it asks the HIP runtime where each buffer lives (hipPointerGetAttributes,
 * hipMemGetAddressRange) and refuses with AR_ERR_INVALID_ARGUMENT plain or
 * pinned host memory, another device's memory and a buffer (or workspace)
 * that runs past the end of its allocation; ar_plan_start then
 * only enqueues the planned kernels on `stream`, as often as wanted, so a hot
 * loop or a HIP graph capture pays no validation.  The plan keeps the device
 * pointers it was given: the buffers (and workspace) must stay valid, and
 * hold the inputs, whenever the plan is started.  Starts whose work overlaps
 * on the GPU write the same outputs and race.  *_init allocates the plan in
 * host memory and sets *plan (NULL on error); ar_plan_free releases it
 * (NULL is accepted).  A plan may be started from several threads.  A plan
 * belongs to the device that was current at *_init, where its buffers live
 * and for whose compute units its grids were sized: start it on a stream of
 * that device. */
typedef struct ar_plan_s* ar_plan_t;

ar_result_t ar_allreduce_init(const void* const* sendbufs, void* const* recvbufs, size_t count,
                              ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo,
                              void* workspace, size_t workspace_bytes, ar_plan_t* plan);
ar_result_t ar_reduce_scatter_init(const void* const* sendbufs, void* const* recvbufs, size_t count,
                                   ar_dtype_t dtype, ar_op_t op, int nranks, ar_algo_t algo,
                                   void* workspace, size_t workspace_bytes, ar_plan_t* plan);
ar_result_t ar_all_gather_init(const void* const* sendbufs, void* const* recvbufs, size_t count,
                               ar_dtype_t dtype, int nranks, ar_algo_t algo,
                               void* workspace, size_t workspace_bytes, ar_plan_t* plan);
ar_result_t ar_plan_start(ar_plan_t plan, hipStream_t stream);
/* Kernel launches one start enqueues (0 for count == 0), or -1 for NULL. */
int ar_plan_num_launches(ar_plan_t plan);
/* The algorithm (an ar_algo_t) the planned call runs: AR_ALGO_AUTO's choice
 * for the plan's shape, AR_ALGO_FUSED for the fused forms of reduce-scatter
 * and all-gather and for a single rank; -1 for NULL. */
int ar_plan_algo(ar_plan_t plan);
/* Cap the workgroups of every launch of the plan at `max_blocks` (each
 * launch keeps at least one block per acting rank of its stage); the
 * kernels then stride over their tiles, with the same results.  0 restores
 * the planned grids (one block per tile).  This bounds the compute units a
 * collective occupies while it overlaps other work: arjunsriva.com "AllReduce,
 * All the Way Down" (section on communication sharing the machine with the
 * model) notes that an overlapped collective still takes SMs and HBM
 * bandwidth from the computation beside it.  Not safe to call while another
 * thread starts the same plan. */
ar_result_t ar_plan_limit_blocks(ar_plan_t plan, unsigned max_blocks);
ar_result_t ar_plan_free(ar_plan_t plan);

/* Workspace in bytes that a call with these arguments needs (0: none).
 * Returns (size_t)-1 for invalid arguments.  The leading `coll` names the
 * collective: the size depends on it (only the ring reduce-scatter, whose
 * receive buffers are one shard long, and the float32-partial variants keep
 * partial sums in a workspace), so this takes one argument more than a
 * per-algorithm size would. */
size_t ar_workspace_bytes(ar_coll_t coll, ar_algo_t algo, size_t count, ar_dtype_t dtype, int nranks);

/* Bounds of chunk c: *begin = c*count/nranks, *end = (c+1)*count/nranks
 * (floor division in 64-bit integers; tirogla.com "Ring all-reduce",
 * section "Code").  Host only; touches no device. */
ar_result_t ar_chunk_range(int c, size_t count, int nranks, size_t* begin, size_t* end);

/* Static text for a result code. */
const char* ar_get_error_string(ar_result_t r);

/* Description of the calling thread's most recent failed call ("" if none).
 * The text stays valid until that thread's next call into the library. */
const char* ar_get_last_error_detail(void);

/* Size in bytes of one element of `dtype`, 0 if unknown. */
size_t ar_dtype_size(ar_dtype_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* AR_H */
