// Device-side building blocks shared by the kernel sources (ar_kernels.hip:
// the ring schedules; ar_tree_kernels.hip: the tree-shaped orders;
// ar_dbt_kernels.hip: the double binary tree; ar_persistent_kernels.hip: the
// ring in one launch): element arithmetic,
// 16-byte vector access, the fold over ranks, the chunk geometry with its
// tile loop, the ring's step bodies, and the LDS staging of small messages.
// Everything here is inline device code in an unnamed namespace, so each
// kernel source gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "ar_internal.h"

namespace arimpl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Ranks whose loads are in flight together before they are folded.
#ifndef AR_RANK_BATCH
#define AR_RANK_BATCH 8
#endif
constexpr int kBatch = AR_RANK_BATCH;

// Ranks whose loads are in flight together when one element is folded on
// its own (chunk edges).  Each batch costs a memory round trip, and when
// chunks are only a few elements long (small messages over many ranks) the
// edges are all there is.
constexpr int kEdgeBatch = 8;

// Nontemporal hints: the reducing kernels stream their N input buffers once
// (AR_NT_LOADS), the copies read a shard that several ranks' stores follow
// (AR_NT_LOADS_COPY), and every output is written once (AR_NT_STORES).
#ifndef AR_NT_LOADS
#define AR_NT_LOADS 1
#endif
#ifndef AR_NT_LOADS_COPY
#define AR_NT_LOADS_COPY 0
#endif
#ifndef AR_NT_STORES
#define AR_NT_STORES 1
#endif

// Element types: float32 and int32 (4 bytes); bf16, IEEE binary16 and bf16
// with float32 partial sums (2 bytes).
template <int DT>
constexpr int elem_size() { return (DT == AR_FLOAT32 || DT == AR_INT32) ? 4 : 2; }

// AR_BFLOAT16_ACC_F32 keeps its partial sums in float32 and rounds to bf16
// once, when a chunk is complete; every other type keeps its partials in the
// buffer type, rounded after each operation.
template <int DT>
constexpr bool acc_f32() { return DT == AR_BFLOAT16_ACC_F32; }

// avg combines like sum; its one division by N happens when a chunk is complete.
constexpr int combine_op(int op) { return op == AR_AVG ? AR_SUM : op; }

// ---------------------------------------------------------------------------
// element arithmetic
// ---------------------------------------------------------------------------

typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// IEEE binary32 operations, round to nearest even.  min/max are IEEE
// 754-2019 minimum/maximum: NaN if either operand is NaN, and for equal
// operands the sign bits decide (-0 below +0).
template <int OP>
__device__ __forceinline__ float f32_apply(float a, float b) {
    if constexpr (OP == AR_SUM) {
        return a + b;
    } else if constexpr (OP == AR_PROD) {
        return a * b;
    } else if constexpr (OP == AR_MIN) {
        const float lo = (a < b) ? a : b;
        const float tie = as_f(as_u(a) | as_u(b));
        const float r = (a == b) ? tie : lo;
        return (a != a || b != b) ? as_f(0x7fc00000u) : r;
    } else {
        const float hi = (a > b) ? a : b;
        const float tie = as_f(as_u(a) & as_u(b));
        const float r = (a == b) ? tie : hi;
        return (a != a || b != b) ? as_f(0x7fc00000u) : r;
    }
}

// int32: sum and product wrap modulo 2^32 (unsigned arithmetic).
template <int OP>
__device__ __forceinline__ uint32_t i32_apply(uint32_t a, uint32_t b) {
    if constexpr (OP == AR_SUM) {
        return a + b;
    } else if constexpr (OP == AR_PROD) {
        return a * b;
    } else if constexpr (OP == AR_MIN) {
        return (static_cast<int32_t>(a) < static_cast<int32_t>(b)) ? a : b;
    } else {
        return (static_cast<int32_t>(a) > static_cast<int32_t>(b)) ? a : b;
    }
}

// bf16 bits are the upper half of the float32 with the same value.
__device__ __forceinline__ float bf16_widen(uint32_t h) { return as_f(h << 16); }

// float32 -> bf16, nearest with ties to even.  AR_BF16_HW_CVT (default 1)
// uses gfx950's conversion instruction (v_cvt_pk_bf16_f32, two values per
// instruction, in the default round-to-nearest-even mode, subnormals kept);
// 0 uses the integer formula: adding 0x7FFF plus the last kept bit carries
// into the upper half exactly when the dropped half is above one half ulp, or
// equal to it with an odd last bit.  Either way NaN -> a quiet NaN.
#ifndef AR_BF16_HW_CVT
#define AR_BF16_HW_CVT 1
#endif
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_round(float f) {
    if constexpr (AR_BF16_HW_CVT) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
    } else {
        const uint32_t u = as_u(f);
        const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
        const uint32_t quiet = (u >> 16) | 0x40u;
        return ((u & 0x7fffffffu) > 0x7f800000u) ? quiet : rounded;
    }
}

// Two values rounded to bf16 and packed: lo in bits 0-15, hi in bits 16-31.
__device__ __forceinline__ uint32_t bf16_round2(float lo, float hi) {
    if constexpr (AR_BF16_HW_CVT) {
        const f32x2_t v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    } else {
        return bf16_round(lo) | (bf16_round(hi) << 16);
    }
}

// IEEE binary16 <-> float32 with the hardware conversions (exact widening;
// narrowing to nearest even, subnormals kept, overflow to infinity).
__device__ __forceinline__ float f16_widen(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
__device__ __forceinline__ uint32_t f16_round(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// One operation of the ring on values held in the buffer type.
template <int DT, int OP>
struct Red {
    static constexpr int kOp = combine_op(OP);

    // one element held in the low bits of a 32-bit value
    static __device__ __forceinline__ uint32_t elem(uint32_t a, uint32_t b) {
        if constexpr (DT == AR_FLOAT32) {
            return as_u(f32_apply<kOp>(as_f(a), as_f(b)));
        } else if constexpr (DT == AR_INT32) {
            return i32_apply<kOp>(a, b);
        } else if constexpr (DT == AR_FLOAT16) {
            return f16_round(f32_apply<kOp>(f16_widen(a & 0xffffu), f16_widen(b & 0xffffu)));
        } else {
            return bf16_round(f32_apply<kOp>(bf16_widen(a & 0xffffu), bf16_widen(b & 0xffffu)));
        }
    }
    // one 32-bit word: one 4-byte element or two 2-byte elements
    static __device__ __forceinline__ uint32_t word(uint32_t a, uint32_t b) {
        if constexpr (DT == AR_BFLOAT16 || DT == AR_BFLOAT16_ACC_F32) {
            return bf16_round2(f32_apply<kOp>(bf16_widen(a & 0xffffu), bf16_widen(b & 0xffffu)),
                               f32_apply<kOp>(bf16_widen(a >> 16), bf16_widen(b >> 16)));
        } else if constexpr (elem_size<DT>() == 2) {
            return elem(a, b) | (elem(a >> 16, b >> 16) << 16);
        } else {
            return elem(a, b);
        }
    }
    static __device__ __forceinline__ u32x4 vec(u32x4 a, u32x4 b) {
        u32x4 r;
        r.x = word(a.x, b.x);
        r.y = word(a.y, b.y);
        r.z = word(a.z, b.z);
        r.w = word(a.w, b.w);
        return r;
    }

    // avg: the one division by N of a complete sum, rounded to the buffer
    // type (int32: truncating toward zero)
    static __device__ __forceinline__ uint32_t avg_elem(uint32_t v, int n) {
        if constexpr (DT == AR_FLOAT32) {
            return as_u(as_f(v) / static_cast<float>(n));
        } else if constexpr (DT == AR_INT32) {
            return static_cast<uint32_t>(static_cast<int32_t>(v) / n);
        } else if constexpr (DT == AR_FLOAT16) {
            return f16_round(f16_widen(v & 0xffffu) / static_cast<float>(n));
        } else {
            return bf16_round(bf16_widen(v & 0xffffu) / static_cast<float>(n));
        }
    }
    static __device__ __forceinline__ uint32_t avg_word(uint32_t v, int n) {
        if constexpr (elem_size<DT>() == 2) {
            return avg_elem(v, n) | (avg_elem(v >> 16, n) << 16);
        } else {
            return avg_elem(v, n);
        }
    }
    static __device__ __forceinline__ u32x4 avg_vec(u32x4 v, int n) {
        u32x4 r;
        r.x = avg_word(v.x, n);
        r.y = avg_word(v.y, n);
        r.z = avg_word(v.z, n);
        r.w = avg_word(v.w, n);
        return r;
    }
};

// ---------------------------------------------------------------------------
// memory access
// ---------------------------------------------------------------------------

template <int ESZ>
__device__ __forceinline__ uint32_t load_elem(const char* p) {
    if constexpr (ESZ == 2) {
        return *reinterpret_cast<const uint16_t*>(p);
    } else {
        return *reinterpret_cast<const uint32_t*>(p);
    }
}

template <int ESZ, bool NT = AR_NT_STORES>
__device__ __forceinline__ void store_elem(char* p, uint32_t v) {
    if constexpr (ESZ == 2) {
        if constexpr (NT) {
            __builtin_nontemporal_store(static_cast<uint16_t>(v), reinterpret_cast<uint16_t*>(p));
        } else {
            *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v);
        }
    } else {
        if constexpr (NT) {
            __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
        } else {
            *reinterpret_cast<uint32_t*>(p) = v;
        }
    }
}

template <bool NT = AR_NT_LOADS>
__device__ __forceinline__ u32x4 load16(const char* p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    } else {
        return *reinterpret_cast<const u32x4*>(p);
    }
}

template <bool NT = AR_NT_STORES>
__device__ __forceinline__ void store16(char* p, u32x4 v) {
    if constexpr (NT) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    } else {
        *reinterpret_cast<u32x4*>(p) = v;
    }
}

// Element e (0 <= e < 16/ESZ) of a 16-byte vector.
template <int ESZ>
__device__ __forceinline__ uint32_t vec_elem(u32x4 v, int e) {
    const uint32_t w = (ESZ == 2) ? v[e >> 1] : v[e];
    if constexpr (ESZ == 2) {
        return (e & 1) ? (w >> 16) : (w & 0xffffu);
    } else {
        return w;
    }
}

// A unit is what one thread moves per rank per access: a 16-byte vector on
// the vector path (VEC > 1 elements) or one element (VEC == 1).  A block
// addresses each buffer through the start of its tile (`tile`, uniform over
// the block) plus the thread's byte offset inside the tile (`lane_off`).
template <int DT, int VEC, bool NT_LOAD = AR_NT_LOADS>
struct Unit {
    static constexpr int kEsz = elem_size<DT>();
    static constexpr int kBytes = (VEC > 1) ? 16 : kEsz;
    using T = std::conditional_t<(VEC > 1), u32x4, uint32_t>;

    // `p` is the buffer address minus the common residue (vector path); tv0
    // the tile's first unit.
    static __device__ __forceinline__ const char* tile(const char* p, uint64_t tv0) { return p + tv0 * kBytes; }
    static __device__ __forceinline__ char* tile(char* p, uint64_t tv0) { return p + tv0 * kBytes; }
    // The thread's u-th unit inside the tile: one 16-byte access per lane per
    // instruction, so each wave instruction covers 1 KiB contiguous.
    static __device__ __forceinline__ uint32_t lane_unit(int u) {
        return threadIdx.x + static_cast<uint32_t>(u) * kThreads;
    }
    static __device__ __forceinline__ uint32_t lane_off(int u) { return lane_unit(u) * kBytes; }
    static __device__ __forceinline__ T load(const char* tb, uint32_t off) {
        if constexpr (VEC > 1) {
            return load16<NT_LOAD>(tb + off);
        } else {
            return load_elem<kEsz>(tb + off);
        }
    }
    // NT: nontemporal store (the default for outputs, written once) or a
    // cache-allocating one (a result that a later launch reads back)
    template <bool NT = AR_NT_STORES>
    static __device__ __forceinline__ void store(char* tb, uint32_t off, T x) {
        if constexpr (VEC > 1) {
            store16<NT>(tb + off, x);
        } else {
            store_elem<kEsz, NT>(tb + off, x);
        }
    }
    template <int OP>
    static __device__ __forceinline__ T combine(T a, T b) {
        if constexpr (VEC > 1) {
            return Red<DT, OP>::vec(a, b);
        } else {
            return Red<DT, OP>::elem(a, b);
        }
    }
};

// The fold of one unit across ranks: the chunk owner's value starts it
// (`first`), every later rank's value is combined in (`add`), and `done`
// completes it (avg divides by N once; float32 partials of
// AR_BFLOAT16_ACC_F32 are rounded to bf16).  A is the type partials are kept
// in: the buffer type, or float32 for AR_BFLOAT16_ACC_F32.
template <int DT, int OP, int VEC>
struct Fold {
    using U = Unit<DT, VEC>;
    using T = typename U::T;
    using A = std::conditional_t<acc_f32<DT>(), std::conditional_t<(VEC > 1), f32x8, float>, T>;
    static constexpr int kOp = combine_op(OP);

    static __device__ __forceinline__ A widen(T x) {
        if constexpr (!acc_f32<DT>()) {
            return x;
        } else if constexpr (VEC > 1) {
            f32x8 r;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r[2 * k] = bf16_widen(x[k] & 0xffffu);
                r[2 * k + 1] = bf16_widen(x[k] >> 16);
            }
            return r;
        } else {
            return bf16_widen(x & 0xffffu);
        }
    }
    static __device__ __forceinline__ A first(T x) { return widen(x); }
    static __device__ __forceinline__ A add(A acc, T x) {
        if constexpr (!acc_f32<DT>()) {
            return U::template combine<OP>(acc, x);
        } else if constexpr (VEC > 1) {
            const f32x8 w = widen(x);
            f32x8 r;
#pragma unroll
            for (int k = 0; k < 8; ++k) r[k] = f32_apply<kOp>(acc[k], w[k]);
            return r;
        } else {
            return f32_apply<kOp>(acc, widen(x));
        }
    }
    // two partials (ring step: the local value and the incoming partial)
    static __device__ __forceinline__ A add_acc(A acc, A y) {
        if constexpr (!acc_f32<DT>()) {
            return U::template combine<OP>(acc, y);
        } else if constexpr (VEC > 1) {
            f32x8 r;
#pragma unroll
            for (int k = 0; k < 8; ++k) r[k] = f32_apply<kOp>(acc[k], y[k]);
            return r;
        } else {
            return f32_apply<kOp>(acc, y);
        }
    }
    static __device__ __forceinline__ T done(A acc, int n) {
        if constexpr (!acc_f32<DT>()) {
            if constexpr (OP == AR_AVG) {
                if constexpr (VEC > 1) {
                    return Red<DT, OP>::avg_vec(acc, n);
                } else {
                    return Red<DT, OP>::avg_elem(acc, n);
                }
            } else {
                return acc;
            }
        } else if constexpr (VEC > 1) {
            u32x4 r;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float lo = acc[2 * k], hi = acc[2 * k + 1];
                if constexpr (OP == AR_AVG) {
                    lo = lo / static_cast<float>(n);
                    hi = hi / static_cast<float>(n);
                }
                r[k] = bf16_round2(lo, hi);
            }
            return r;
        } else {
            float v = acc;
            if constexpr (OP == AR_AVG) v = v / static_cast<float>(n);
            return bf16_round(v);
        }
    }
};

// ---------------------------------------------------------------------------
// chunk geometry
// ---------------------------------------------------------------------------

struct Span {
    uint64_t s, e;    // element bounds of the chunk
    uint64_t vb, ve;  // units of the chunk body: vectors (VEC > 1) or elements
    uint64_t hb, he;  // head elements [hb, he) done one by one (VEC > 1 only)
    uint64_t tb, te;  // tail elements [tb, te)
};

// Part c of `parts` floor parts of the buffer: [c*count/parts, (c+1)*count/parts),
// with a.count_q = count / parts and a.count_r = count % parts.
template <int VEC>
__device__ __forceinline__ Span part_span(int c, int parts, const KernelArgs& a) {
    Span sp;
    // c*count/n = c*(count/n) + c*(count%n)/n; the last product is below 128^2,
    // so only a 32-bit division is left
    const uint32_t n = static_cast<uint32_t>(parts);
    const uint32_t cu = static_cast<uint32_t>(c);
    sp.s = static_cast<uint64_t>(cu) * a.count_q + (cu * a.count_r) / n;
    sp.e = static_cast<uint64_t>(cu + 1) * a.count_q + ((cu + 1) * a.count_r) / n;
    if constexpr (VEC > 1) {
        // the body: whole aligned blocks of A = 2^align_shift elements, as vectors
        const uint64_t ofs = static_cast<uint64_t>(a.ofs);
        const uint32_t sh = static_cast<uint32_t>(a.align_shift);
        const uint64_t first_block = (sp.s + ofs + (1ull << sh) - 1) >> sh;
        const uint64_t end_block = (sp.e + ofs) >> sh;
        sp.vb = (first_block << sh) / VEC;
        sp.ve = (end_block << sh) / VEC;
        if (sp.ve < sp.vb) sp.ve = sp.vb;
        const uint64_t body_first = sp.vb * VEC - ofs;   // first element of the body (>= s)
        const uint64_t body_end = sp.ve * VEC - ofs;     // one past its last element
        // head [s, min(body_first, e)); tail from the body's end (or the head's end
        // when the body is empty) up to e; both stay inside [s, e) also for
        // empty and short chunks
        sp.hb = sp.s;
        sp.he = body_first < sp.e ? body_first : sp.e;
        sp.tb = body_end > sp.he ? body_end : sp.he;
        if (sp.tb > sp.e) sp.tb = sp.e;
        sp.te = sp.e;
    } else {
        sp.vb = sp.s;
        sp.ve = sp.e;
        sp.hb = sp.he = sp.tb = sp.te = sp.s;
    }
    return sp;
}

// Chunk c of the ring's plan: one part per rank.
template <int VEC>
__device__ __forceinline__ Span chunk_span(int c, const KernelArgs& a) {
    return part_span<VEC>(c, a.nranks, a);
}

// Element handled by thread j among the chunk's edge elements, or false.
__device__ __forceinline__ bool edge_element(const Span& sp, unsigned j, uint64_t* i) {
    const uint64_t nh = sp.he - sp.hb;
    const uint64_t nt = sp.te - sp.tb;
    if (j < nh) {
        *i = sp.hb + j;
        return true;
    }
    if (j < nh + nt) {
        *i = sp.tb + (j - nh);
        return true;
    }
    return false;
}

__device__ __forceinline__ int ring_rank(int c, int k, int n) {
    // (c + k) mod n for 0 <= c < n, 0 <= k < 2n
    int r = c + k;
    r = (r >= n) ? r - n : r;
    return (r >= n) ? r - n : r;
}

// ---------------------------------------------------------------------------
// the ring-order fold of one chunk position across all ranks
// ---------------------------------------------------------------------------

// acc[u] = ((x_c (op) x_{c+1}) (op) ...) at the thread's units of the tile
// that starts at unit tv0, for live u.  NT_LOAD picks nontemporal or
// cache-allocating loads.
template <int DT, int OP, int VEC, bool NT_LOAD = AR_NT_LOADS>
__device__ __forceinline__ void fold_units(const KernelArgs& a, int c, int64_t adj, uint64_t tv0,
                                           const bool (&live)[kUnroll],
                                           typename Fold<DT, OP, VEC>::A (&acc)[kUnroll]) {
    using U = Unit<DT, VEC, NT_LOAD>;
    using F = Fold<DT, OP, VEC>;
    const int n = a.nranks;
    {
        const char* tb = U::tile(a.send[c] - adj, tv0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (live[u]) acc[u] = F::first(U::load(tb, U::lane_off(u)));
        }
    }
    for (int k = 1; k < n; k += kBatch) {
        typename U::T x[kBatch][kUnroll];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (k + j < n) {
                const char* tb = U::tile(a.send[ring_rank(c, k + j, n)] - adj, tv0);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (live[u]) x[j][u] = U::load(tb, U::lane_off(u));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (k + j < n) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (live[u]) acc[u] = F::add(acc[u], x[j][u]);
                }
            }
        }
    }
}

// Same fold for one element i (chunk edges), completed.
template <int DT, int OP>
__device__ __forceinline__ uint32_t fold_element(const KernelArgs& a, int c, uint64_t i) {
    constexpr int ESZ = elem_size<DT>();
    using F = Fold<DT, OP, 1>;
    const int n = a.nranks;
    typename F::A acc = F::first(load_elem<ESZ>(a.send[c] + i * ESZ));
    for (int k = 1; k < n; k += kEdgeBatch) {
        uint32_t x[kEdgeBatch];
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (k + j < n) x[j] = load_elem<ESZ>(a.send[ring_rank(c, k + j, n)] + i * ESZ);
        }
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (k + j < n) acc = F::add(acc, x[j]);
        }
    }
    return F::done(acc, n);
}

// Store one element i to every rank's receive buffer (chunk edges).  The
// receive pointers come from the kernel arguments kEdgeBatch at a time, so
// their loads overlap instead of each store waiting for its own pointer
// (which dominates when chunks are tiny).  The tiles' stores keep a plain
// loop: batching their pointers costs registers, and occupancy, there.
template <int ESZ>
__device__ __forceinline__ void store_elem_all(const KernelArgs& a, int n, uint64_t i, uint32_t v) {
    for (int q0 = 0; q0 < n; q0 += kEdgeBatch) {
        char* p[kEdgeBatch];
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (q0 + j < n) p[j] = a.recv[q0 + j];
        }
#pragma unroll
        for (int j = 0; j < kEdgeBatch; ++j) {
            if (q0 + j < n) store_elem<ESZ>(p[j] + i * ESZ, v);
        }
    }
}

// Store unit v of a result into a shard that starts at element `s` of the
// full buffer (reduce-scatter output).  `aligned` says whether the shard's
// 16-byte vectors line up with the source's.
template <int DT, int VEC, bool NT = AR_NT_STORES>
__device__ __forceinline__ void store_shard_unit(char* shard, uint64_t s, int32_t ofs, bool aligned,
                                                 uint64_t v, typename Unit<DT, VEC>::T x) {
    constexpr int ESZ = elem_size<DT>();
    if constexpr (VEC > 1) {
        const uint64_t first = v * VEC - static_cast<uint64_t>(ofs);   // element index in the full buffer
        if (aligned) {
            store16<NT>(shard + (first - s) * ESZ, x);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) store_elem<ESZ, NT>(shard + (first + e - s) * ESZ, vec_elem<ESZ>(x, e));
        }
    } else {
        store_elem<ESZ, NT>(shard + (v - s) * ESZ, x);
    }
}

// Load unit v of the full-buffer position space from a shard starting at `s`.
template <int DT, int VEC, bool NT_LOAD>
__device__ __forceinline__ typename Unit<DT, VEC>::T load_shard_unit(const char* shard, uint64_t s, int32_t ofs,
                                                                     bool aligned, uint64_t v) {
    constexpr int ESZ = elem_size<DT>();
    if constexpr (VEC > 1) {
        const uint64_t first = v * VEC - static_cast<uint64_t>(ofs);
        if (aligned) return load16<NT_LOAD>(shard + (first - s) * ESZ);
        u32x4 r = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const uint32_t x = load_elem<ESZ>(shard + (first + e - s) * ESZ);
            if constexpr (ESZ == 2) {
                r[e >> 1] |= (e & 1) ? (x << 16) : x;
            } else {
                r[e] = x;
            }
        }
        return r;
    } else {
        return load_elem<ESZ>(shard + (v - s) * ESZ);
    }
}

template <int DT>
__device__ __forceinline__ bool shard_aligned(const void* shard, uint64_t s, int32_t ofs) {
    constexpr int ESZ = elem_size<DT>();
    const uint64_t q = reinterpret_cast<uint64_t>(shard) - (s + static_cast<uint64_t>(ofs)) * ESZ;
    return (q & 15u) == 0;
}

// The tiles a block walks: consecutive tiles to consecutive blocks (the
// default), or, when the launch sets xcd_slabs, the launch's tiles cut into
// eight contiguous slabs, slab x walked by the blocks the dispatcher deals to
// XCD x (blocks x, x + 8, x + 16, ...).  Each XCD then touches one eighth of
// the address range that all the blocks in flight touch, and with it one
// eighth of the pages its address translation caches must hold.  Measured on
// MI355X it pays from 64 ranks (up to 8 % at 64 x 16 MiB), for the fused
// AllReduce also from 32 ranks and whenever its inputs sit in the last-level
// cache; streaming 128-256 MiB per rank from HBM at 8-16 ranks, the plain
// order is faster.  The host gives
// such a launch a grid of a multiple of eight blocks; blocks past the last
// whole group of eight walk nothing.
struct TileWalk {
    uint32_t first, end, step;
};

__device__ __forceinline__ TileWalk tile_walk(const KernelArgs& a) {
    const uint32_t per = gridDim.x >> 3;   // blocks per XCD
    if (a.xcd_slabs == 0 || per == 0) return {a.tile_first + blockIdx.x, a.tile_end, gridDim.x};
    const uint32_t x = blockIdx.x & 7u, m = blockIdx.x >> 3;
    const uint64_t span = a.tile_end - a.tile_first;
    const uint32_t s0 = a.tile_first + static_cast<uint32_t>(span * x / 8);
    const uint32_t s1 = a.tile_first + static_cast<uint32_t>(span * (x + 1) / 8);
    if (m >= per) return {s1, s1, 1u};
    return {s0 + m, s1, per};
}

// Tile loop: tile -> (chunk c, tile t within the chunk); consecutive tiles
// walk one chunk after another (measured faster on MI355X than cycling over
// the chunks).  A launch covers tiles [tile_first, tile_end) in the order of
// tile_walk; the host keeps N * tiles_per_chunk below 2^31.
#define AR_TILE_LOOP_BEGIN                                                                   \
    const int n = a.nranks;                                                                  \
    const uint32_t tpc = a.tiles_per_chunk;                                                  \
    const int64_t adj = (VEC > 1) ? static_cast<int64_t>(a.ofs) * elem_size<DT>() : 0;       \
    const TileWalk walk = tile_walk(a);                                                      \
    for (uint32_t tile = walk.first; tile < walk.end; tile += walk.step) {                   \
        const int c = static_cast<int>(tile / tpc);                                          \
        const uint64_t t = tile - static_cast<uint32_t>(c) * tpc;                            \
        const Span sp = chunk_span<VEC>(c, a);                                               \
        const uint64_t tv0 = sp.vb + t * (kThreads * kUnroll);                               \
        bool live[kUnroll];                                                                  \
        _Pragma("unroll") for (int u = 0; u < kUnroll; ++u)                                  \
            live[u] = tv0 + U::lane_unit(u) < sp.ve;

#define AR_TILE_LOOP_END }

// Partial sums kept between the steps of a schedule: the buffer type, or
// float32 (4 bytes per element, 32 bytes per unit of eight bf16) for
// AR_BFLOAT16_ACC_F32.  `base` is the workspace minus the common residue in
// partial-sized elements, so unit v sits at base + v * kBytes.
template <int DT, int VEC>
struct Partials {
    static constexpr bool kF32 = acc_f32<DT>();
    static constexpr int kElemBytes = kF32 ? 4 : elem_size<DT>();
    static constexpr int kBytes = kF32 ? (VEC > 1 ? 32 : 4) : Unit<DT, VEC>::kBytes;
    using A = typename Fold<DT, AR_SUM, VEC>::A;

    static __device__ __forceinline__ A load(const char* base, uint64_t v) {
        const char* p = base + v * kBytes;
        if constexpr (!kF32) {
            return Unit<DT, VEC, false>::load(p, 0);
        } else if constexpr (VEC > 1) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
            f32x8 r;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r[k] = as_f(lo[k]);
                r[k + 4] = as_f(hi[k]);
            }
            return r;
        } else {
            return *reinterpret_cast<const float*>(p);
        }
    }
    static __device__ __forceinline__ void store(char* base, uint64_t v, A x) {
        char* p = base + v * kBytes;
        if constexpr (!kF32 && VEC > 1) {
            *reinterpret_cast<u32x4*>(p) = x;
        } else if constexpr (!kF32) {
            // one element of the buffer type, held in the low bits of x
            if constexpr (elem_size<DT>() == 2) {
                *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(x);
            } else {
                *reinterpret_cast<uint32_t*>(p) = x;
            }
        } else if constexpr (VEC > 1) {
            u32x4 lo, hi;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lo[k] = as_u(x[k]);
                hi[k] = as_u(x[k + 4]);
            }
            *reinterpret_cast<u32x4*>(p) = lo;
            *reinterpret_cast<u32x4*>(p + 16) = hi;
        } else {
            *reinterpret_cast<float*>(p) = x;
        }
    }
};


// ---------------------------------------------------------------------------
// the ring's steps over every chunk (tirogla.com "Ring all-reduce", "How it
// works"): the bodies of the one-launch-per-step kernels, and of the
// persistent ring that runs all steps in one launch
// ---------------------------------------------------------------------------

// Reduce-scatter step `step` of the AllReduce ring: chunk c is reduced on
// rank r = c+step+1 from rank p = c+step (see k_ring_reduce_step).
template <int DT, int OP, int VEC>
__device__ __forceinline__ void ring_reduce_tiles(const KernelArgs& a, int step) {
    static_assert(!acc_f32<DT>(), "float32 partials need the workspace step");
    using U = Unit<DT, VEC>;
    using F = Fold<DT, OP, VEC>;
    using F1 = Fold<DT, OP, 1>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    const int r = ring_rank(c, step + 1, n);
    const int p = ring_rank(c, step, n);
    const char* local = a.send[r];
    const char* incoming = (step == 0) ? a.send[p] : a.recv[p];
    char* out = a.recv[r];
    const bool last = (step == n - 2);
    if (VEC > 1 && t == 0) {
        uint64_t i;
        if (edge_element(sp, threadIdx.x, &i)) {
            uint32_t v = F1::add(load_elem<ESZ>(local + i * ESZ), load_elem<ESZ>(incoming + i * ESZ));
            if (last) v = F1::done(v, n);
            store_elem<ESZ>(out + i * ESZ, v);
        }
    }
    typename U::T x[kUnroll], y[kUnroll];
    const char* tl = U::tile(local - adj, tv0);
    const char* ti = U::tile(incoming - adj, tv0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (live[u]) {
            x[u] = U::load(tl, U::lane_off(u));
            y[u] = U::load(ti, U::lane_off(u));
        }
    }
    char* to = U::tile(out - adj, tv0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (!live[u]) continue;
        typename U::T z = F::add(x[u], y[u]);
        if (last) z = F::done(z, n);
        U::store(to, U::lane_off(u), z);
    }
    AR_TILE_LOOP_END
}

// All-gather step `step`: chunk c is copied from rank r-1 to rank
// r = c+step+shift (see k_ring_copy_step).
template <int DT, int VEC>
__device__ __forceinline__ void ring_copy_tiles(const KernelArgs& a, int step, int shift) {
    using U = Unit<DT, VEC, AR_NT_LOADS_COPY>;
    constexpr int ESZ = elem_size<DT>();
    AR_TILE_LOOP_BEGIN
    const int r = ring_rank(c, step + shift, n);
    const int p = ring_rank(r, n - 1, n);
    const char* src = a.recv[p];
    char* dst = a.recv[r];
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
    AR_TILE_LOOP_END
}

// ---------------------------------------------------------------------------
// small messages: all ranks' values of a few positions staged in LDS
// ---------------------------------------------------------------------------

// When chunks are only a few elements long, the tiled kernels leave most
// threads idle and fold each edge element rank by rank, a memory round trip
// per batch of ranks.  The small-message kernels instead give a block
// P = kThreads / N consecutive positions [i0, i0 + P): thread t = r*P + j
// loads rank r's element i0 + j (one load per thread, all in flight at once)
// into LDS, the positions are reduced from LDS (the ring's left fold by one
// thread per position; the tree orders level by level across threads), and
// every thread stores one result to one rank.  Per-lane rank pointers are read from the kernel
// argument segment through its address, so the table is never copied.
__device__ __forceinline__ const KernelArgs* kernarg_table() {
#if defined(__HIP_DEVICE_COMPILE__)
    return reinterpret_cast<const KernelArgs*>(__builtin_amdgcn_kernarg_segment_ptr());
#else
    return nullptr;   // the host pass never runs device code
#endif
}

// The small-message kernels: thread t of a block loads and stores rank t / P
// at position t mod P of the block's P positions.  Its two rank pointers are
// read from the argument table once, ahead of the loads and stores that need
// them.
struct SmallPtrs {
    const char* src;
    char* dst;
};

__device__ __forceinline__ SmallPtrs small_ptrs(const KernelArgs& a, int P) {
    const int r = static_cast<int>(threadIdx.x) / P;
    if (r >= a.nranks) return {nullptr, nullptr};
    return {kernarg_table()->send[r], kernarg_table()->recv[r]};
}

// The block's place in a small-message launch when each XCD takes one
// contiguous run of blocks: the dispatcher deals block b to XCD b mod 8, and
// b is mapped to x * q + min(x, rem) + b / 8 for x = b mod 8, q = G / 8,
// rem = G mod 8 (a one-to-one map of [0, G)).  Neighbouring positions share
// cache lines; so mapped, each line is loaded through one XCD's L2 instead
// of all eight (measured on MI355X, ring order, per call in a graph: 128
// ranks x 4 KiB 6.9 -> 4.2 us, 64 ranks x 64 KiB 11.8 -> 6.7 us; 2 to 16
// ranks within +-5 %).
__device__ __forceinline__ uint32_t xcd_grouped_block() {
    const uint32_t g = gridDim.x, b = blockIdx.x;
    const uint32_t x = b & 7u, q = g >> 3, rem = g & 7u;
    return x * q + (x < rem ? x : rem) + (b >> 3);
}

template <int ESZ>
__device__ __forceinline__ void small_stage(const KernelArgs& a, const SmallPtrs& q, uint32_t* vals, int P,
                                            uint64_t i0) {
    const int t = static_cast<int>(threadIdx.x);
    const int r = t / P;
    const uint64_t i = i0 + static_cast<uint64_t>(t - r * P);
    if (r < a.nranks && i < a.count) vals[t] = load_elem<ESZ>(q.src + i * ESZ);
}

template <int ESZ>
__device__ __forceinline__ void small_store(const KernelArgs& a, const SmallPtrs& q, const uint32_t* res, int P,
                                            uint64_t i0) {
    const int t = static_cast<int>(threadIdx.x);
    const int r = t / P;
    const int j = t - r * P;
    const uint64_t i = i0 + static_cast<uint64_t>(j);
    if (r < a.nranks && i < a.count) store_elem<ESZ>(q.dst + i * ESZ, res[j]);
}

}  // namespace
}  // namespace arimpl
