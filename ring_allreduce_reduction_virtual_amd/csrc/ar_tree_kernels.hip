// HIP kernels (gfx950) for AllReduce in tree-shaped orders over N virtual
// ranks held in one GPU's HBM.
//
// The schedules are those of bitfern.com "AllReduce Explained: Algorithms,
// Performance, and Distributed Training" (section "Common AllReduce
// Algorithms": "Tree AllReduce", "Recursive Doubling") and Rabenseifner's
// recursive-halving reduce-scatter plus recursive-doubling all-gather
// (tirogla.com "Ring all-reduce", section "How it works", cost model).  Each
// one brackets the N-term reduction of an element the same way for every
// element and every rank:
//
//   binomial tree / recursive doubling   ((x0 x1) (x2 x3)) ((x4 x5) (x6 x7)) ...
//   recursive halving                    ((x0 x4) (x2 x6)) ((x1 x5) (x3 x7)) ...
//
// The second is the first applied to the ranks in bit-reversed order, so one
// fused kernel computes both: it folds the send table in the order the host
// gives it with a binary counter of partials (leaf k merges with the partial
// in slot j for every set bit j of k, lowest first; the slots left at the end,
// one per set bit of N, join from the lowest up), which is exactly the
// binomial tree's bracketing for any N.  One pass: reads N*S, writes N*S.
//
// The step kernels run the schedules stage by stage, one launch per stage,
// as the virtual ranks would exchange messages: they keep the pages' stage
// counts (2 ceil(log2 N) for the tree, log2 N for recursive doubling,
// 2 log2 N for halving/doubling) and with them each schedule's launch
// latency.  Partials between stages live in the ranks' own receive buffers,
// or, for AR_BFLOAT16_ACC_F32, in float32 in a workspace with one slab per
// rank.

#include "ar_device.h"

namespace arimpl {
namespace {

// ---------------------------------------------------------------------------
// fused: the binomial-tree bracketing in one pass
// ---------------------------------------------------------------------------

// Ranks whose loads are in flight together; fewer for the widest partial
// slots, whose registers they share.
#ifndef AR_TREE_BATCH
#define AR_TREE_BATCH 8
#endif
template <int DT, int D>
constexpr int tree_batch() {
    return (D >= 8 && acc_f32<DT>()) ? 4 : AR_TREE_BATCH;
}

// Add leaf k (x) to the counter of partials: slot j holds the complete
// subtree of 2^j leaves when bit j of k is set.  The bits of k are uniform
// over the block, so the branches are scalar.
template <int DT, int OP, int VEC, int D>
__device__ __forceinline__ void tree_push(typename Fold<DT, OP, VEC>::A (&slot)[D][kUnroll], uint32_t k,
                                          typename Fold<DT, OP, VEC>::A (&x)[kUnroll],
                                          const bool (&live)[kUnroll]) {
    using F = Fold<DT, OP, VEC>;
    bool placed = false;
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (!placed) {
            if ((k >> j) & 1u) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (live[u]) x[u] = F::add_acc(slot[j][u], x[u]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (live[u]) slot[j][u] = x[u];
                }
                placed = true;
            }
        }
    }
}

// The slots left after N leaves (one per set bit of N) joined from the
// smallest subtree up: the last rank's partial is the innermost right operand.
template <int DT, int OP, int VEC, int D>
__device__ __forceinline__ typename Fold<DT, OP, VEC>::A tree_result(
    const typename Fold<DT, OP, VEC>::A (&slot)[D][kUnroll], uint32_t n, int u) {
    using F = Fold<DT, OP, VEC>;
    typename F::A res = slot[0][u];
    bool have = false;
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if ((n >> j) & 1u) {
            res = have ? F::add_acc(slot[j][u], res) : slot[j][u];
            have = true;
        }
    }
    return res;
}

// One element i folded the same way (chunk edges), completed.
template <int DT, int OP, int D>
__device__ __forceinline__ uint32_t tree_element(const KernelArgs& a, uint64_t i) {
    constexpr int ESZ = elem_size<DT>();
    using F = Fold<DT, OP, 1>;
    typename F::A slot[D][kUnroll];
    const bool live[kUnroll] = {true};
    for (int k = 0; k < a.nranks; k += kEdgeBatch) {
        uint32_t v[kEdgeBatch];
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (k + j < a.nranks) v[j] = load_elem<ESZ>(a.send[k + j] + i * ESZ);
        }
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (k + j < a.nranks) {
                typename F::A x[kUnroll];
                x[0] = F::first(v[j]);
                tree_push<DT, OP, 1, D>(slot, static_cast<uint32_t>(k + j), x, live);
            }
        }
    }
    return F::done(tree_result<DT, OP, 1, D>(slot, static_cast<uint32_t>(a.nranks), 0), a.nranks);
}

// AllReduce in the binomial-tree bracketing of the send table's order (the
// host passes the ranks in bit-reversed order for recursive halving).  In
// place (send[r] == recv[r]) is safe: each position is read by the thread
// that later writes it, and by no other.
template <int DT, int OP, int VEC, int D, bool NT_LOAD>
__global__ __launch_bounds__(kThreads) void k_fused_tree(const KernelArgs a) {
    using U = Unit<DT, VEC, NT_LOAD>;
    using F = Fold<DT, OP, VEC>;
    constexpr int B = tree_batch<DT, D>();
    AR_TILE_LOOP_BEGIN
    (void)c;
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            store_elem_all<elem_size<DT>()>(a, n, i, tree_element<DT, OP, D>(a, i));
        }
    }
    typename F::A slot[D][kUnroll];
    for (int k = 0; k < n; k += B) {
        typename U::T x[B][kUnroll];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (k + j < n) {
                const char* tb = U::tile(a.send[k + j] - adj, tv0);
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
                tree_push<DT, OP, VEC, D>(slot, static_cast<uint32_t>(k + j), w, live);
            }
        }
    }
    typename U::T res[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) res[u] = F::done(tree_result<DT, OP, VEC, D>(slot, static_cast<uint32_t>(n), u), n);
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

// The binomial-tree bracketing for a small message: P = kThreads / N
// positions per block staged through LDS (see small_stage), then reduced
// stage by stage: thread r P + j holds leaf r (the send table's r-th rank) of
// column j, and at stage k every r with r mod 2^(k+1) = 0 adds the partial of
// r + 2^k when that leaf exists, (own (op) received), a barrier between
// stages.  That is the binary counter's bracketing with the same operand
// order, so the bits are the same, in ceil(log2 N) dependent steps instead
// of N.
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void k_small_tree(const KernelArgs a) {
    constexpr int ESZ = elem_size<DT>();
    using F = Fold<DT, OP, 1>;
    using A = typename F::A;
    __shared__ uint32_t vals[kThreads];
    __shared__ A acc[kThreads];
    __shared__ uint32_t res[kThreads];
    const int n = a.nranks;
    const int P = kThreads / n;
    const int t = static_cast<int>(threadIdx.x);
    const int r = t / P;                                         // this thread's leaf
    const int col = t - r * P;                                   // its column
    const SmallPtrs q = small_ptrs(a, P);
    for (uint64_t i0 = static_cast<uint64_t>(xcd_grouped_block()) * P; i0 < a.count;
         i0 += static_cast<uint64_t>(gridDim.x) * P) {
        small_stage<ESZ>(a, q, vals, P, i0);
        __syncthreads();
        const bool active = r < n && i0 + col < a.count;
        if (active) acc[t] = F::first(vals[t]);
        __syncthreads();
        for (int d = 1; d < n; d <<= 1) {
            if (active && (r & (2 * d - 1)) == 0 && r + d < n) acc[t] = F::add_acc(acc[t], acc[t + d * P]);
            __syncthreads();
        }
        if (t < P && i0 + t < a.count) res[t] = F::done(acc[t], n);
        __syncthreads();
        small_store<ESZ>(a, q, res, P, i0);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// stages: one launch per stage of a schedule
// ---------------------------------------------------------------------------

// Who acts on chunk c in a stage: rank `out` gets `left (op) right`
// (reducing stages; `out2`, when not negative, gets the same value) or a copy
// of `left`'s values (distributing stages).
struct Actor {
    int out, left, right, out2;
};

__device__ __forceinline__ int stage_actors(int mode, int step, int n) {
    switch (mode) {
        case kTreeReduce:
        case kTreeBcast: {
            const int d = 1 << step;   // ranks r = 0, 2d, 4d, ... with r + d < n
            return n > d ? (n - d + 2 * d - 1) / (2 * d) : 0;
        }
        case kRdExchange: return n / 2;
        case kHalvingReduce: return n >> (step + 1);
        case kDoublingGather: return 1 << step;
    }
    return 0;
}

__device__ __forceinline__ Actor stage_actor(int mode, int step, int n, int c, int j) {
    switch (mode) {
        case kTreeReduce: {
            const int d = 1 << step, r = j * 2 * d;
            return {r, r, r + d, -1};
        }
        case kTreeBcast: {
            const int d = 1 << step, r = j * 2 * d;
            return {r + d, r, -1, -1};
        }
        case kRdExchange: {
            // pair j: the rank with bit d clear, and its partner
            const int d = 1 << step, r = ((j & ~(d - 1)) << 1) | (j & (d - 1));
            return {r, r, r | d, r | d};
        }
        case kHalvingReduce: {
            // the ranks that keep chunk c agree with c on bits d and above
            const int d = n >> (step + 1), r = (c & ~(d - 1)) | j;
            return {r, r, r ^ d, -1};
        }
        case kDoublingGather: {
            // receivers agree with c on bits 2d and above and differ at bit d
            const int d = 1 << step, r = (c & ~(2 * d - 1)) | (~c & d) | j;
            return {r, r ^ d, -1, -1};
        }
    }
    return {0, 0, 0, -1};
}

// Whether rank x's operand in this reducing stage is its send buffer (it
// has received nothing yet) or its partial.  Binomial reduction: a rank
// first receives in stage 0 when it is even and rank x+1 exists.
__device__ __forceinline__ bool operand_is_send(const KernelArgs& a, int x) {
    if (a.step == 0) return true;
    if (a.mode == kTreeReduce) return (x & 1) != 0 || x + 1 >= a.nranks;
    return false;
}

template <int DT>
__device__ __forceinline__ const char* partial_of(const KernelArgs& a, int x) {
    if constexpr (acc_f32<DT>()) {
        return a.ws + static_cast<uint64_t>(x) * a.ws_stride;
    } else {
        return a.recv[x];
    }
}

// A reducing stage: actor blockIdx.y of chunk c computes out = left (op) right; the
// stage that completes the values (`last`) finishes them (avg divides by N,
// float32 partials round to bf16) into the receive buffer.  Hazard-free:
// in every mode no rank's partial is written in a stage where another rank
// reads it (the readers' partners are never outputs of the same chunk).
template <int DT, int OP, int VEC>
__global__ __launch_bounds__(kThreads) void k_tree_reduce_step(const KernelArgs a) {
    using U = Unit<DT, VEC>;
    using F = Fold<DT, OP, VEC>;
    using F1 = Fold<DT, OP, 1>;
    using P = Partials<DT, VEC>;
    using P1 = Partials<DT, 1>;
    constexpr int ESZ = elem_size<DT>();
    const int64_t pofs = acc_f32<DT>() ? static_cast<int64_t>(a.ofs) * 4 : static_cast<int64_t>(a.ofs) * ESZ;
    const int j = static_cast<int>(blockIdx.y);
    if (j >= stage_actors(a.mode, a.step, a.nranks)) return;
    AR_TILE_LOOP_BEGIN
    const bool last = a.last != 0;
    {
        const Actor ac = stage_actor(a.mode, a.step, n, c, j);
        const bool ls = operand_is_send(a, ac.left), rs = operand_is_send(a, ac.right);
        if (VEC > 1 && t == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) {
                const typename F1::A x = ls ? F1::first(load_elem<ESZ>(a.send[ac.left] + i * ESZ))
                                            : P1::load(partial_of<DT>(a, ac.left), i);
                const typename F1::A y = rs ? F1::first(load_elem<ESZ>(a.send[ac.right] + i * ESZ))
                                            : P1::load(partial_of<DT>(a, ac.right), i);
                const typename F1::A z = F1::add_acc(x, y);
                if (last) {
                    const uint32_t v = F1::done(z, n);
                    store_elem<ESZ>(a.recv[ac.out] + i * ESZ, v);
                    if (ac.out2 >= 0) store_elem<ESZ>(a.recv[ac.out2] + i * ESZ, v);
                } else {
                    P1::store(const_cast<char*>(partial_of<DT>(a, ac.out)), i, z);
                    if (ac.out2 >= 0) P1::store(const_cast<char*>(partial_of<DT>(a, ac.out2)), i, z);
                }
            }
        }
        typename F::A x[kUnroll], y[kUnroll];
        const char* tl = U::tile(a.send[ac.left] - adj, tv0);
        const char* tr = U::tile(a.send[ac.right] - adj, tv0);
        const char* pl = partial_of<DT>(a, ac.left) - pofs;
        const char* pr = partial_of<DT>(a, ac.right) - pofs;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!live[u]) continue;
            if (ls) {
                x[u] = F::first(U::load(tl, U::lane_off(u)));
            } else {
                x[u] = P::load(pl, tv0 + U::lane_unit(u));
            }
            if (rs) {
                y[u] = F::first(U::load(tr, U::lane_off(u)));
            } else {
                y[u] = P::load(pr, tv0 + U::lane_unit(u));
            }
        }
        if (last) {
            char* to = U::tile(a.recv[ac.out] - adj, tv0);
            char* to2 = ac.out2 >= 0 ? U::tile(a.recv[ac.out2] - adj, tv0) : nullptr;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (!live[u]) continue;
                const typename U::T v = F::done(F::add_acc(x[u], y[u]), n);
                U::store(to, U::lane_off(u), v);
                if (to2 != nullptr) U::store(to2, U::lane_off(u), v);
            }
        } else {
            char* po = const_cast<char*>(partial_of<DT>(a, ac.out)) - pofs;
            char* po2 = ac.out2 >= 0 ? const_cast<char*>(partial_of<DT>(a, ac.out2)) - pofs : nullptr;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (!live[u]) continue;
                const typename F::A z = F::add_acc(x[u], y[u]);
                P::store(po, tv0 + U::lane_unit(u), z);
                if (po2 != nullptr) P::store(po2, tv0 + U::lane_unit(u), z);
            }
        }
    }
    AR_TILE_LOOP_END
}

// A distributing stage: actor blockIdx.y of chunk c copies recv[left] to recv[out].
// No rank is both a source and a destination of chunk c in one stage.
template <int DT, int VEC>
__global__ __launch_bounds__(kThreads) void k_tree_copy_step(const KernelArgs a) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    constexpr int ESZ = elem_size<DT>();
    const int j = static_cast<int>(blockIdx.y);
    if (j >= stage_actors(a.mode, a.step, a.nranks)) return;
    AR_TILE_LOOP_BEGIN
    {
        const Actor ac = stage_actor(a.mode, a.step, n, c, j);
        const char* src = a.recv[ac.left];
        char* dst = a.recv[ac.out];
        if (VEC > 1 && t == 0) {
            uint64_t i;
            if (edge_element(sp, threadIdx.x, &i)) store_elem<ESZ>(dst + i * ESZ, load_elem<ESZ>(src + i * ESZ));
        }
        typename U::T x[kUnroll];
        const char* ts = U::tile(src - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) x[u] = U::load(ts, U::lane_off(u));
        }
        char* td = U::tile(dst - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) U::store(td, U::lane_off(u), x[u]);
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
        case Kind::kFusedTree:
            if constexpr (VEC > 1) {
                if (l.cached) {   // inputs that fit in the last-level cache: cache-allocating loads
                    switch (l.depth) {
                        case 4: hipLaunchKernelGGL((k_fused_tree<DT, OP, VEC, 4, false>), grid, block, 0, s, a); break;
                        case 6: hipLaunchKernelGGL((k_fused_tree<DT, OP, VEC, 6, false>), grid, block, 0, s, a); break;
                        case 8: hipLaunchKernelGGL((k_fused_tree<DT, OP, VEC, 8, false>), grid, block, 0, s, a); break;
                        default: return hipErrorInvalidValue;
                    }
                    break;
                }
            }
            switch (l.depth) {
                case 4: hipLaunchKernelGGL((k_fused_tree<DT, OP, VEC, 4, AR_NT_LOADS>), grid, block, 0, s, a); break;
                case 6: hipLaunchKernelGGL((k_fused_tree<DT, OP, VEC, 6, AR_NT_LOADS>), grid, block, 0, s, a); break;
                case 8: hipLaunchKernelGGL((k_fused_tree<DT, OP, VEC, 8, AR_NT_LOADS>), grid, block, 0, s, a); break;
                default: return hipErrorInvalidValue;
            }
            break;
        case Kind::kTreeReduceStep:
            hipLaunchKernelGGL((k_tree_reduce_step<DT, OP, VEC>), grid, block, 0, s, a);
            break;
        case Kind::kSmallTree:
            if constexpr (VEC == 1) {
                hipLaunchKernelGGL((k_small_tree<DT, OP>), grid, block, 0, s, a);
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
        hipLaunchKernelGGL((k_tree_copy_step<DT, V>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((k_tree_copy_step<DT, 1>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tree(const Launch& l, const KernelArgs& a, hipStream_t stream) {
    if (l.kind == Kind::kTreeCopyStep) {
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
