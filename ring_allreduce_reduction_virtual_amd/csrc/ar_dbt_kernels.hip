// HIP kernels (gfx950) for AllReduce over two binary trees, the double binary
// tree, over N virtual ranks held in one GPU's HBM.
//
// The pages give the double binary tree's cost (tirogla.com "Ring
// all-reduce", section "How it works": about 2 log2 N latency terms and
// 2 S/B) and its use (small and medium messages at large N), not its
// construction.  That comes from Sanders, Speck and Träff, "Two-tree
// algorithms for full bandwidth broadcast, reduction and scan" (2009): two
// binary trees over the same ranks, no rank an inner node of both, each
// carrying half of the buffer.  Here:
//
//   * the halves are the buffer's floor split in two, [0, len/2) and
//     [len/2, len): parts 0 and 1 of the tile loop;
//   * tree 0 is the in-order binary tree over positions 1..N (position p
//     holds rank p-1): p's height is its count of trailing zero bits, the
//     root is the largest power of two <= N, an inner node p of height h has
//     the left child p - 2^(h-1) and the right child p + 2^j for the largest
//     j < h with p + 2^j <= N (none when p = N); tree 1 is tree 0 with every
//     rank moved on by one (position p holds rank p mod N).  Inner positions
//     are even, so inner ranks are odd in tree 0 and even in tree 1;
//   * an inner node combines ((left partial (op) own value) (op) right partial).
//
// The fused kernel evaluates that bracketing in one pass (reads N*S, writes
// N*S): it feeds the ranks in position order to a stack machine whose stack
// holds the inner nodes still waiting for their right subtree (at most 6 for
// N <= 128).  Positions are uniform over a block, so every push, pop and
// climb is a scalar branch and the stack stays in registers.
//
// The stage kernels run the schedule as the ranks would exchange messages:
// reducing stage j (j = 1..H, H = floor(log2 N)) has every node of height j
// of both trees combine its children's partials; distributing stage j
// (j = H..1) has every node of height j copy the finished half to its
// children.  2H launches in all.  Partials live in the ranks' receive
// buffers (their own half of them), or, for AR_BFLOAT16_ACC_F32, in float32
// in one workspace slab per rank.

#include "ar_device.h"

namespace arimpl {
namespace {

// Tile loop over the two halves: tile -> (half c, tile t within the half).
#define AR_HALF_LOOP_BEGIN                                                                   \
    const int n = a.nranks;                                                                  \
    const uint32_t tpc = a.tiles_per_chunk;                                                  \
    const int64_t adj = (VEC > 1) ? static_cast<int64_t>(a.ofs) * elem_size<DT>() : 0;       \
    const TileWalk walk = tile_walk(a);                                                      \
    for (uint32_t tile = walk.first; tile < walk.end; tile += walk.step) {                   \
        const int c = static_cast<int>(tile / tpc);                                          \
        const uint64_t t = tile - static_cast<uint32_t>(c) * tpc;                            \
        const Span sp = part_span<VEC>(c, 2, a);                                             \
        const uint64_t tv0 = sp.vb + t * (kThreads * kUnroll);                               \
        bool live[kUnroll];                                                                  \
        _Pragma("unroll") for (int u = 0; u < kUnroll; ++u)                                  \
            live[u] = tv0 + U::lane_unit(u) < sp.ve;

// Rank at position p (1..n) of tree `tree` (0 or 1).
__device__ __forceinline__ int dbt_rank(uint32_t p, int tree, int n) {
    const int r = static_cast<int>(p) - 1 + tree;
    return r >= n ? r - n : r;
}

// Parent position of q in the tree over positions 1..n, 0 for the root:
// q = k 2^h with k odd is a left child of q + 2^h when k = 1 mod 4 and that
// position exists, otherwise the right child of q - 2^h.
__device__ __forceinline__ uint32_t dbt_parent(uint32_t q, uint32_t n) {
    const uint32_t h = static_cast<uint32_t>(__builtin_ctz(q));
    const uint32_t step = 1u << h;
    if (((q >> h) & 3u) == 1u && q + step <= n) return q + step;
    return q > step ? q - step : 0u;
}

// Right child of an inner position p of height h (0 when it has none).
__device__ __forceinline__ uint32_t dbt_right(uint32_t p, int h, uint32_t n) {
    for (int j = h - 1; j >= 0; --j) {
        if (p + (1u << j) <= n) return p + (1u << j);
    }
    return 0u;
}

// The in-order evaluation of a tree's bracketing as the ranks are fed in
// position order.  `cur` is the value of the last completed subtree; the
// stack holds A_p = (left subtree (op) own value) of the inner nodes whose
// right subtree is still being fed, the innermost in slot 0.  Push and pop
// shift every slot by one, so no slot is ever indexed by a variable and the
// stack stays in registers (an indexed register array would go to scratch).
template <int DT, int OP, int VEC, int D>
struct InOrder {
    using F = Fold<DT, OP, VEC>;
    using A = typename F::A;
    A slot[D][kUnroll];
    A cur[kUnroll];

    __device__ __forceinline__ void push() {
#pragma unroll
        for (int j = D - 1; j > 0; --j) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) slot[j][u] = slot[j - 1][u];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) slot[0][u] = cur[u];
    }
    // cur = (top of the stack) (op) cur
    __device__ __forceinline__ void pop_join(const bool (&live)[kUnroll]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) cur[u] = F::add_acc(slot[0][u], cur[u]);
        }
#pragma unroll
        for (int j = 0; j + 1 < D; ++j) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) slot[j][u] = slot[j + 1][u];
        }
    }
    // Position p's value x (in working precision).
    __device__ __forceinline__ void feed(uint32_t p, uint32_t n, const A (&x)[kUnroll], const bool (&live)[kUnroll]) {
        const int h = __builtin_ctz(p);
        if (h == 0) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) cur[u] = x[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) cur[u] = F::add_acc(cur[u], x[u]);   // left subtree (op) own value
            }
            if (p < n) {                                           // a right subtree follows
                push();
                return;
            }
        }
        // the subtree rooted at q = p is complete: join while it is a right child
        uint32_t q = p;
        for (;;) {
            const uint32_t par = dbt_parent(q, n);
            if (par == 0u || par > q) break;
            pop_join(live);
            q = par;
        }
    }
};

// Ranks whose loads are in flight together; fewer when float32 partials fill
// the deepest stack (D = 6 slots, for 16 to 128 ranks), whose registers they
// share.
template <int DT, int D>
constexpr int dbt_batch() {
    return (D >= 6 && acc_f32<DT>()) ? 4 : 8;
}

// One element i of half c, folded the same way (chunk edges), completed.
template <int DT, int OP, int D>
__device__ __forceinline__ uint32_t dbt_element(const KernelArgs& a, int c, uint64_t i) {
    constexpr int ESZ = elem_size<DT>();
    using F = Fold<DT, OP, 1>;
    const int n = a.nranks;
    const bool live[kUnroll] = {true};
    InOrder<DT, OP, 1, D> m;
    for (int k = 0; k < n; k += kEdgeBatch) {
        uint32_t v[kEdgeBatch];
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (k + j < n) v[j] = load_elem<ESZ>(a.send[dbt_rank(static_cast<uint32_t>(k + j + 1), c, n)] + i * ESZ);
        }
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (k + j < n) {
                typename F::A x[kUnroll];
                x[0] = F::first(v[j]);
                m.feed(static_cast<uint32_t>(k + j + 1), static_cast<uint32_t>(n), x, live);
            }
        }
    }
    return F::done(m.cur[0], n);
}

// AllReduce over the two trees in one pass: half c folded in tree c's
// bracketing, stored to every rank.  In place (send[r] == recv[r]) is safe:
// each position is read by the thread that later writes it, and by no other.
template <int DT, int OP, int VEC, int D, bool NT_LOAD>
__global__ __launch_bounds__(kThreads) void k_fused_dbt(const KernelArgs a) {
    using U = Unit<DT, VEC, NT_LOAD>;
    using F = Fold<DT, OP, VEC>;
    constexpr int B = dbt_batch<DT, D>();
    AR_HALF_LOOP_BEGIN
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) store_elem_all<elem_size<DT>()>(a, n, i, dbt_element<DT, OP, D>(a, c, i));
    }
    InOrder<DT, OP, VEC, D> m;
    for (int k = 0; k < n; k += B) {
        typename U::T x[B][kUnroll];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (k + j < n) {
                const char* tb = U::tile(a.send[dbt_rank(static_cast<uint32_t>(k + j + 1), c, n)] - adj, tv0);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (live[u]) x[j][u] = U::load(tb, U::lane_off(u));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (k + j < n) {
                typename F::A w[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (live[u]) w[u] = F::first(x[j][u]);
                }
                m.feed(static_cast<uint32_t>(k + j + 1), static_cast<uint32_t>(n), w, live);
            }
        }
    }
    typename U::T res[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) res[u] = F::done(m.cur[u], n);
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

// The two trees' bracketings for a small message: P = kThreads / N positions
// per block staged through LDS (see small_stage), then evaluated level by
// level: thread (p - 1) P + j holds tree position p of column j, and at
// level h = 1 .. H = floor(log2 N) every position of height h combines
// ((left child (op) own value) (op) right child) from the values of the
// levels below, kept in LDS, with a barrier between levels.  Those are the
// in-order machine's operations on the same operands, so the bits are the
// same, in H dependent steps instead of N.  A column's half, and with it the
// rank at each position, follows from its element index.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void k_small_dbt(const KernelArgs a) {
    constexpr int ESZ = elem_size<DT>();
    using F = Fold<DT, OP, 1>;
    using A = typename F::A;
    __shared__ uint32_t vals[kThreads];
    __shared__ A acc[kThreads];
    __shared__ uint32_t res[kThreads];
    const int n = a.nranks;
    const int P = kThreads / n;
    const int t = static_cast<int>(threadIdx.x);
    const uint32_t p = static_cast<uint32_t>(t / P) + 1u;       // this thread's tree position
    const int col = t - (t / P) * P;                             // its column
    const bool node = p <= static_cast<uint32_t>(n);
    const int hp = node ? __builtin_ctz(p) : -1;
    int levels = 0;
    while ((2u << levels) <= static_cast<uint32_t>(n)) ++levels;  // floor(log2 N): the root's height
    const uint32_t root = 1u << levels;
    const SmallPtrs q = small_ptrs(a, P);
    for (uint64_t i0 = static_cast<uint64_t>(xcd_grouped_block()) * P; i0 < a.count;
         i0 += static_cast<uint64_t>(gridDim.x) * P) {
        small_stage<ESZ>(a, q, vals, P, i0);
        __syncthreads();
        const bool active = node && i0 + col < a.count;
        A own{};
        if (active) {
            const int c = (i0 + col) >= a.count_q ? 1 : 0;      // half 1 starts at count / 2
            own = F::first(vals[dbt_rank(p, c, n) * P + col]);
            if (hp == 0) acc[t] = own;                           // a leaf's value is its own
        }
        __syncthreads();
        for (int h = 1; h <= levels; ++h) {
            if (active && hp == h) {
                A v = F::add_acc(acc[(p - (1u << (h - 1)) - 1u) * P + col], own);
                const uint32_t rp = dbt_right(p, h, static_cast<uint32_t>(n));
                if (rp != 0u) v = F::add_acc(v, acc[(rp - 1u) * P + col]);
                acc[t] = v;
            }
            __syncthreads();
        }
        if (t < P && i0 + t < a.count) res[t] = F::done(acc[(root - 1u) * P + t], n);
        __syncthreads();
        small_store<ESZ>(a, q, res, P, i0);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// stages: one launch per tree level
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ const char* dbt_partial(const KernelArgs& a, int r) {
    if constexpr (acc_f32<DT>()) {
        return a.ws + static_cast<uint64_t>(r) * a.ws_stride;
    } else {
        return a.recv[r];
    }
}

// Reducing stage j = a.step (1..H): actor blockIdx.y is position
// p = 2^j (2 blockIdx.y + 1) of both trees; in half c, rank(p) computes
// ((left (op) own) (op) right) from its children's partials (a leaf's is its
// send buffer).  The stage that reaches the root (`last`) finishes the value
// into the root's receive buffer; the others keep partials.  Hazard-free: a
// partial written in stage j is read only by the node's parent, in a later
// stage, and an inner node's send half is read by that node alone.
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_dbt_reduce_step(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    using F = Fold<DT, OP, VEC>;
    using F1 = Fold<DT, OP, 1>;
    using P = Partials<DT, VEC>;
    using P1 = Partials<DT, 1>;
    constexpr int ESZ = elem_size<DT>();
    const int64_t pofs = acc_f32<DT>() ? static_cast<int64_t>(a.ofs) * 4 : static_cast<int64_t>(a.ofs) * ESZ;
    const int j = a.step;
    const uint32_t p = (2u * blockIdx.y + 1u) << j;
    if (p > static_cast<uint32_t>(a.nranks)) return;
    AR_HALF_LOOP_BEGIN
    const bool last = a.last != 0;
    {
        const uint32_t lp = p - (1u << (j - 1));
        const uint32_t rp = dbt_right(p, j, static_cast<uint32_t>(n));
        const int me = dbt_rank(p, c, n);
        const int lr = dbt_rank(lp, c, n);
        const int rr = rp != 0u ? dbt_rank(rp, c, n) : me;
        const bool lsend = j == 1;                                   // the left child is a leaf
        const bool rsend = rp != 0u && __builtin_ctz(rp) == 0;      // so is the right one
        if (VEC > 1 && t == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) {
                typename F1::A v = lsend ? F1::first(load_elem<ESZ>(a.send[lr] + i * ESZ))
                                         : P1::load(dbt_partial<DT>(a, lr), i);
                v = F1::add_acc(v, F1::first(load_elem<ESZ>(a.send[me] + i * ESZ)));
                if (rp != 0u) {
                    v = F1::add_acc(v, rsend ? F1::first(load_elem<ESZ>(a.send[rr] + i * ESZ))
                                             : P1::load(dbt_partial<DT>(a, rr), i));
                }
                if (last) {
                    store_elem<ESZ>(a.recv[me] + i * ESZ, F1::done(v, n));
                } else {
                    P1::store(const_cast<char*>(dbt_partial<DT>(a, me)), i, v);
                }
            }
        }
        typename F::A v[kUnroll], w[kUnroll];
        const char* tl = U::tile(a.send[lr] - adj, tv0);
        const char* tm = U::tile(a.send[me] - adj, tv0);
        const char* tr = U::tile(a.send[rr] - adj, tv0);
        const char* pl = dbt_partial<DT>(a, lr) - pofs;
        const char* pr = dbt_partial<DT>(a, rr) - pofs;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!live[u]) continue;
            v[u] = lsend ? F::first(U::load(tl, U::lane_off(u))) : P::load(pl, tv0 + U::lane_unit(u));
            w[u] = F::first(U::load(tm, U::lane_off(u)));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) v[u] = F::add_acc(v[u], w[u]);
        }
        if (rp != 0u) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) w[u] = rsend ? F::first(U::load(tr, U::lane_off(u))) : P::load(pr, tv0 + U::lane_unit(u));
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) v[u] = F::add_acc(v[u], w[u]);
            }
        }
        if (last) {
            char* to = U::tile(a.recv[me] - adj, tv0);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) U::store(to, U::lane_off(u), F::done(v[u], n));
            }
        } else {
            char* po = const_cast<char*>(dbt_partial<DT>(a, me)) - pofs;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) P::store(po, tv0 + U::lane_unit(u), v[u]);
            }
        }
    }
    AR_TILE_LOOP_END
}

// Distributing stage j = a.step (H..1): position p = 2^j (2 blockIdx.y + 1)
// copies its finished half to its children.  No rank is both a source and a
// destination of one half in one stage (sources have height j, destinations
// lower).
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_dbt_copy_step(const KernelArgs a) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    constexpr int ESZ = elem_size<DT>();
    const int j = a.step;
    const uint32_t p = (2u * blockIdx.y + 1u) << j;
    if (p > static_cast<uint32_t>(a.nranks)) return;
    AR_HALF_LOOP_BEGIN
    {
        const uint32_t lp = p - (1u << (j - 1));
        const uint32_t rp = dbt_right(p, j, static_cast<uint32_t>(n));
        const char* src = a.recv[dbt_rank(p, c, n)];
        char* d0 = a.recv[dbt_rank(lp, c, n)];
        char* d1 = rp != 0u ? a.recv[dbt_rank(rp, c, n)] : nullptr;
        if (VEC > 1 && t == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) {
                const uint32_t x = load_elem<ESZ>(src + i * ESZ);
                store_elem<ESZ>(d0 + i * ESZ, x);
                if (d1 != nullptr) store_elem<ESZ>(d1 + i * ESZ, x);
            }
        }
        typename U::T x[kUnroll];
        const char* ts = U::tile(src - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) x[u] = U::load(ts, U::lane_off(u));
        }
        char* t0 = U::tile(d0 - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) U::store(t0, U::lane_off(u), x[u]);
        }
        if (d1 != nullptr) {
            char* t1 = U::tile(d1 - adj, tv0);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (live[u]) U::store(t1, U::lane_off(u), x[u]);
            }
        }
    }
    AR_TILE_LOOP_END
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int DT, int OP, int VEC>
hipError_t launch_reduce(const Launch& l, const KernelArgs& a, hipStream_t s) {
    const dim3 grid(l.blocks, l.actors > 0 ? l.actors : 1), block(kThreads);
    switch (l.kind) {
        case Kind::kFusedDbt:
            if constexpr (VEC > 1) {
                if (l.cached) {   // inputs that fit in the last-level cache: cache-allocating loads
                    switch (l.depth) {
                        case 4: hipLaunchKernelGGL((k_fused_dbt<DT, OP, VEC, 4, false>), grid, block, 0, s, a); break;
                        case 6: hipLaunchKernelGGL((k_fused_dbt<DT, OP, VEC, 6, false>), grid, block, 0, s, a); break;
                        default: return hipErrorInvalidValue;
                    }
                    break;
                }
            }
            switch (l.depth) {
                case 4: hipLaunchKernelGGL((k_fused_dbt<DT, OP, VEC, 4, AR_NT_LOADS>), grid, block, 0, s, a); break;
                case 6: hipLaunchKernelGGL((k_fused_dbt<DT, OP, VEC, 6, AR_NT_LOADS>), grid, block, 0, s, a); break;
                default: return hipErrorInvalidValue;
            }
            break;
        case Kind::kDbtReduceStep:
            hipLaunchKernelGGL((k_dbt_reduce_step<DT, OP, VEC>), grid, block, 0, s, a);
            break;
        case Kind::kSmallDbt:
            if constexpr (VEC == 1) {
                hipLaunchKernelGGL((k_small_dbt<DT, OP>), grid, block, 0, s, a);
            } else {
                return hipErrorInvalidValue;
            }
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

// Copies depend on the element size only (bit patterns are moved unchanged).
template <int DT>
hipError_t copy_by_vec(const Launch& l, const KernelArgs& a, hipStream_t s) {
    constexpr int V = 16 / elem_size<DT>();
    const dim3 grid(l.blocks, l.actors > 0 ? l.actors : 1), block(kThreads);
    if (l.vec) {
        hipLaunchKernelGGL((k_dbt_copy_step<DT, V>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((k_dbt_copy_step<DT, 1>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dbt(const Launch& l, const KernelArgs& a, hipStream_t stream) {
    if (l.kind == Kind::kDbtCopyStep) {
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
