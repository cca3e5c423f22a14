"""Pins for the tree-shaped schedules of the oracle (oracle/orders.py).

What fixes them, without any implementation to compare against:

* the bracketing each schedule computes is identified by brute force: among
  all (2N-3)!! bracketings of an N-term sum, exactly one agrees with the
  schedule on inputs whose exponents spread so widely that different
  bracketings round differently, and it is the tree written out by hand from
  the pages' descriptions (binomial tree: neighbours first; recursive
  doubling: distance 1, 2, 4, ...; recursive halving: distance N/2 first);
* exact closed forms (integer sums, int32 wrap-around, min/max, products)
  catch a dropped or repeated term;
* the float32 forward error of a tree of height h is at most
  gamma_h * sum|x| against the exact sum (pairwise summation's bound),
  tighter than the ring's (N-1) * u * sum|x|;
* stage counts and bytes against the pages' cost statements: a tree takes a
  logarithmic number of stages, recursive doubling log2 N rounds, and
  Rabenseifner's algorithm 2 log2 N stages with the ring's 2(N-1)/N * S
  bytes per rank.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle.explore import bracketings, canonical, evaluate, ring_tree
from oracle.orders import (
    ORDERS,
    binomial_tree,
    halving_doubling_allreduce,
    halving_tree,
    order_allreduce,
    order_bracketing,
    recursive_doubling_allreduce,
    tree_allreduce,
    tree_order_fold,
    tree_order_fold_columns,
)
from oracle.ring import bf16_bits_to_f32, f32_to_bf16_bits, ring_order_fold, same_bits

# the bracketings typed out by hand from the pages' descriptions
TREE = {
    1: 0,
    2: (0, 1),
    3: ((0, 1), 2),
    4: ((0, 1), (2, 3)),
    5: (((0, 1), (2, 3)), 4),
    6: (((0, 1), (2, 3)), (4, 5)),
    7: (((0, 1), (2, 3)), ((4, 5), 6)),
    8: (((0, 1), (2, 3)), ((4, 5), (6, 7))),
}
HALVING = {
    1: 0,
    2: (0, 1),
    4: ((0, 2), (1, 3)),
    8: (((0, 4), (2, 6)), ((1, 5), (3, 7))),
}


def spread(n, m, seed):
    """float32 values with exponents over [-20, 20] and random signs: sums
    bracketed differently round differently."""
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, size=(n, m))
    exp = rng.integers(-20, 21, size=(n, m)).astype(np.float64)
    sign = rng.choice([-1.0, 1.0], size=(n, m))
    return [(sign[r] * mant[r] * np.exp2(exp[r])).astype(np.float32) for r in range(n)]


def schedule(order, xs, op="sum", dtype="f32"):
    out, _ = order_allreduce(order, xs, op, dtype)
    return out


@pytest.mark.parametrize("order,n", [("tree", 3), ("tree", 4), ("tree", 5), ("recursive_doubling", 4),
                                     ("halving_doubling", 4)])
def test_brute_force_identifies_the_bracketing(order, n):
    xs = spread(n, 256, seed=10 + n)
    got = schedule(order, xs)[0]
    matches = [t for t in bracketings(range(n)) if same_bits(evaluate(t, xs), got, "f32")]
    assert len(matches) == 1
    want = HALVING[n] if order == "halving_doubling" else TREE[n]
    assert canonical(matches[0]) == canonical(want)


@pytest.mark.parametrize("n", [6, 7, 8])
def test_tree_matches_hand_typed_bracketing(n):
    xs = spread(n, 512, seed=n)
    got = schedule("tree", xs)
    for r in range(n):
        assert same_bits(got[r], evaluate(TREE[n], xs), "f32")
    # and not the ring's: chunk 0 of the ring is the plain left fold
    assert not same_bits(got[0], evaluate(ring_tree(0, n), xs), "f32")


def test_halving_matches_hand_typed_bracketing_8():
    xs = spread(8, 512, seed=8)
    got = schedule("halving_doubling", xs)
    for r in range(8):
        assert same_bits(got[r], evaluate(HALVING[8], xs), "f32")
    assert not same_bits(got[0], evaluate(TREE[8], xs), "f32")


@pytest.mark.parametrize("n", sorted(TREE))
def test_definitions_are_the_hand_typed_trees(n):
    assert binomial_tree(n) == TREE[n]
    if n in HALVING:
        assert halving_tree(n) == HALVING[n]


def test_recursive_doubling_and_tree_agree_on_powers_of_two():
    """Two different schedules, one bracketing."""
    for n in (2, 4, 8, 16):
        xs = spread(n, 300, seed=100 + n)
        assert same_bits(schedule("tree", xs)[0], schedule("recursive_doubling", xs)[0], "f32")


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "prod"), ("f32", "max"), ("bf16", "sum"),
                                      ("f16", "avg"), ("i32", "sum"), ("bf16acc32", "sum"),
                                      ("bf16acc32", "avg"), ("i32", "avg"), ("f32", "min")])
def test_schedule_equals_definition(order, dtype, op):
    """Each schedule, run step by step, equals its bracketing evaluated directly."""
    ns = (1, 2, 4, 8) if order != "tree" else (1, 2, 3, 5, 6, 7, 8, 11)
    for n in ns:
        for length in (0, 1, 3, 17, 64):
            rng = np.random.default_rng([n, length])
            if dtype == "i32":
                xs = [rng.integers(-2**31, 2**31, size=length, dtype=np.int64).astype(np.int32) for _ in range(n)]
            elif dtype in ("bf16", "bf16acc32"):
                xs = [f32_to_bf16_bits(rng.standard_normal(length).astype(np.float32)) for _ in range(n)]
            elif dtype == "f16":
                xs = [rng.standard_normal(length).astype(np.float16).view(np.uint16) for _ in range(n)]
            else:
                xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
            got = schedule(order, xs, op, dtype)
            want = tree_order_fold(xs, order_bracketing(order, n), op, dtype)
            for r in range(n):
                assert same_bits(got[r], want, dtype), (order, n, length, r)


@pytest.mark.parametrize("order", ORDERS)
def test_exact_integer_closed_forms(order):
    ns = (2, 4, 8, 16) if order != "tree" else (2, 3, 5, 8, 13)
    for n in ns:
        rng = np.random.default_rng(n)
        length = 45
        ints = [rng.integers(-8, 9, size=length) for _ in range(n)]
        # f32 sums of small integers are exact in any order
        out = schedule(order, [x.astype(np.float32) for x in ints])
        assert np.array_equal(out[0], np.sum(ints, axis=0).astype(np.float32))
        # int32 wraps modulo 2^32
        full = [rng.integers(-2**31, 2**31, size=length, dtype=np.int64) for _ in range(n)]
        out = schedule(order, [x.astype(np.int32) for x in full], "sum", "i32")
        want = ((np.sum(full, axis=0) + 2**31) % 2**32 - 2**31).astype(np.int32)
        assert np.array_equal(out[0], want)
        out = schedule(order, [x.astype(np.int32) for x in full], "min", "i32")
        assert np.array_equal(out[0], np.min(full, axis=0).astype(np.int32))
        out = schedule(order, [x.astype(np.int32) for x in full], "max", "i32")
        assert np.array_equal(out[0], np.max(full, axis=0).astype(np.int32))
        small = [rng.integers(-3, 4, size=length) for _ in range(n)]
        out = schedule(order, [x.astype(np.int32) for x in small], "prod", "i32")
        want = np.prod(np.array(small, dtype=object), axis=0)
        want = np.array([(int(v) + 2**31) % 2**32 - 2**31 for v in want], dtype=np.int32)
        assert np.array_equal(out[0], want)
        # avg of int32 truncates toward zero
        out = schedule(order, [x.astype(np.int32) for x in ints], "avg", "i32")
        s = np.sum(ints, axis=0)
        assert np.array_equal(out[0], (np.sign(s) * (np.abs(s) // n)).astype(np.int32))


@pytest.mark.parametrize("order", ORDERS)
def test_bf16_with_float32_partials_rounds_once(order):
    n = 8
    rng = np.random.default_rng(5)
    vals = [rng.integers(-300, 301, size=64).astype(np.float32) for _ in range(n)]
    xs = [f32_to_bf16_bits(v) for v in vals]
    exact = np.sum([bf16_bits_to_f32(x).astype(np.float64) for x in xs], axis=0)
    out = schedule(order, xs, "sum", "bf16acc32")
    assert np.array_equal(out[0], f32_to_bf16_bits(exact.astype(np.float32)))


@pytest.mark.parametrize("order", ORDERS)
def test_float32_error_within_the_tree_bound(order):
    """|result - exact| <= gamma_h * sum|x|, h the tree's height (pairwise summation)."""
    for n in (4, 8, 16):
        xs = [np.random.default_rng([7, n, r]).standard_normal(500).astype(np.float32) for r in range(n)]
        out = schedule(order, xs)[0]
        h = math.ceil(math.log2(n))
        u = 2.0 ** -24
        gamma = h * u / (1 - h * u)
        for i in range(500):
            col = [float(x[i]) for x in xs]
            exact = Fraction(math.fsum(col))
            err = abs(Fraction(float(out[i])) - exact)
            assert err <= Fraction(gamma) * Fraction(sum(abs(v) for v in col))


def test_stage_counts_and_bytes_follow_the_cost_models():
    for n in (2, 4, 8, 16, 32):
        length = 64 * n
        S = length * 4
        xs = [np.ones(length, np.float32) for _ in range(n)]
        log2n = n.bit_length() - 1
        _, st = recursive_doubling_allreduce(xs)
        assert st.stages == log2n and st.sent == [log2n * S] * n and st.received == st.sent
        _, st = halving_doubling_allreduce(xs)
        assert st.stages == 2 * log2n
        assert st.sent == [2 * (n - 1) * S // n] * n and st.received == st.sent
    for n in range(1, 20):
        length = 7 * n + 3
        S = length * 4
        xs = [np.ones(length, np.float32) for _ in range(n)]
        _, st = tree_allreduce(xs)
        assert st.stages == 2 * math.ceil(math.log2(n)) if n > 1 else st.stages == 0
        assert sum(st.sent) == 2 * (n - 1) * S and sum(st.received) == sum(st.sent)


def test_halving_total_bytes_with_uneven_chunks():
    """Uneven and empty chunks: all ranks together still send 2(N-1) * S."""
    for n in (4, 8, 16):
        for length in (1, 3, n - 1, 5 * n + 3, 1000):
            xs = [np.full(length, r, np.float32) for r in range(n)]
            out, st = halving_doubling_allreduce(xs)
            assert sum(st.sent) == 2 * (n - 1) * length * 4
            assert np.array_equal(out[0], np.full(length, n * (n - 1) / 2, np.float32))


def test_power_of_two_required():
    xs = [np.ones(4, np.float32) for _ in range(6)]
    with pytest.raises(ValueError):
        recursive_doubling_allreduce(xs)
    with pytest.raises(ValueError):
        halving_doubling_allreduce(xs)
    with pytest.raises(ValueError):
        order_bracketing("halving_doubling", 6)


def test_columns_form_matches_whole_buffers():
    xs = spread(8, 100, seed=3)
    cols = np.stack(xs)
    for order in ORDERS:
        t = order_bracketing(order, 8)
        assert same_bits(tree_order_fold_columns(cols[:, ::7], t), tree_order_fold(xs, t)[::7], "f32")


def test_orders_differ_from_the_ring():
    """On spread inputs the tree orders and the ring disagree somewhere (so parity can tell them apart)."""
    xs = spread(8, 4096, seed=11)
    ring = ring_order_fold(xs)
    for order in ORDERS:
        assert not same_bits(schedule(order, xs)[0], ring, "f32")
