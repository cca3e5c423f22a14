"""Pins for the double binary tree of the oracle (oracle/dbt.py).

What fixes it, without any implementation to compare against:

* the two trees, typed out by hand from the construction's statement (in-order
  positions, the node of height h at p with children p - 2^(h-1) and the
  largest p + 2^j that exists; the second tree one rank on), for N = 1..8;
* structure for every N up to 128: each tree is a binary tree over all N
  positions with heights falling towards the leaves and the in-order
  property, its root at height floor(log2 N), and no rank inner in both trees
  (the two-tree property of Sanders, Speck and Träff);
* brute force: among all (2N-3)!! bracketings of an N-term sum, exactly one
  agrees with the executed schedule on each half (N <= 6), and it is the
  hand-typed tree;
* the cost statement on tirogla.com "Ring all-reduce" ("How it works": about
  2 log2 N latency terms and 2 S/B): 2 floor(log2 N) <= 2 ceil(log2 N) stages,
  every rank sends at most 2 S (plus the halves' one-element difference),
  2 (N-1) S in all; a single tree over the whole buffer would make its inner
  ranks send 3 S;
* exact closed forms (integer sums, int32 wrap, min/max, int avg, bf16 with
  float32 partials on integers), and the float32 error bound of any
  bracketing against exact sums.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import dbt
from oracle.explore import bracketings, canonical, evaluate, ring_tree
from oracle.ring import bf16_bits_to_f32, f32_to_bf16_bits, same_bits

# typed by hand from the construction (oracle/dbt.py's module docstring)
TREE0 = {
    1: 0,
    2: (0, 1),
    3: ((0, 1), 2),
    4: (((0, 1), 2), 3),
    5: ((((0, 1), 2), 3), 4),
    6: ((((0, 1), 2), 3), (4, 5)),
    7: ((((0, 1), 2), 3), ((4, 5), 6)),
    8: (((((0, 1), 2), 3), ((4, 5), 6)), 7),
}
TREE1 = {
    1: 0,
    2: (1, 0),
    3: ((1, 2), 0),
    4: (((1, 2), 3), 0),
    5: ((((1, 2), 3), 4), 0),
    6: ((((1, 2), 3), 4), (5, 0)),
    7: ((((1, 2), 3), 4), ((5, 6), 0)),
    8: (((((1, 2), 3), 4), ((5, 6), 7)), 0),
}


def spread(n, m, seed):
    """float32 values with exponents over [-20, 20] and random signs: sums
    bracketed differently round differently."""
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, size=(n, m))
    exp = rng.integers(-20, 21, size=(n, m)).astype(np.float64)
    sign = rng.choice([-1.0, 1.0], size=(n, m))
    return [(sign[r] * mant[r] * np.exp2(exp[r])).astype(np.float32) for r in range(n)]


@pytest.mark.parametrize("n", sorted(TREE0))
def test_trees_are_the_hand_typed_ones(n):
    assert dbt.bracketing(0, n) == TREE0[n]
    assert dbt.bracketing(1, n) == TREE1[n]
    assert dbt.double_binary_trees(n) == (TREE0[n], TREE1[n])


def _leaves(t):
    return _leaves(t[0]) + _leaves(t[1]) if isinstance(t, tuple) else [t]


@pytest.mark.parametrize("n", range(1, 129))
def test_tree_structure_and_the_two_tree_property(n):
    par = dbt.parents(n)
    top = dbt.root(n)
    assert sorted(par) == [p for p in range(1, n + 1) if p != top]          # one parent each, root excepted
    assert dbt.height(top) == int(math.floor(math.log2(n)))
    for c, p in par.items():
        assert dbt.height(c) < dbt.height(p)

    def subtree(p):
        left, right = dbt.children(p, n)
        out = [p]
        for ch in (left, right):
            if ch is not None:
                out += subtree(ch)
        return out

    assert sorted(subtree(top)) == list(range(1, n + 1))
    for p in range(1, n + 1):                                                # in-order
        left, right = dbt.children(p, n)
        if left is not None:
            assert max(subtree(left)) < p
        if right is not None:
            assert min(subtree(right)) > p
    for t in (0, 1):
        assert sorted(_leaves(dbt.bracketing(t, n))) == list(range(n))
    assert not dbt.inner_ranks(0, n) & dbt.inner_ranks(1, n)                 # no rank inner in both


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6])
def test_brute_force_identifies_each_half(n):
    m = 256
    xs = spread(n, 2 * m, seed=40 + n)
    got, _ = dbt.double_binary_tree_allreduce(xs)
    for t, want in ((0, TREE0[n]), (1, TREE1[n])):
        part = [x[t * m:(t + 1) * m] for x in xs]
        matches = [b for b in bracketings(range(n)) if same_bits(evaluate(b, part), got[0][t * m:(t + 1) * m], "f32")]
        assert len(matches) == 1, (t, len(matches))
        assert canonical(matches[0]) == canonical(want)


def test_not_the_ring_nor_one_tree():
    """At 6 ranks and more the first half is not the ring's left fold, and the halves differ."""
    xs = spread(8, 512, seed=8)
    got, _ = dbt.double_binary_tree_allreduce(xs)
    assert not same_bits(got[0][:256], evaluate(ring_tree(0, 8), [x[:256] for x in xs]), "f32")
    assert not same_bits(got[0][256:], evaluate(TREE0[8], [x[256:] for x in xs]), "f32")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13, 16, 64, 100, 128])
def test_stage_count(n):
    _, st = dbt.double_binary_tree_allreduce([np.ones(4, np.float32)] * n)
    assert st.stages == 2 * int(math.floor(math.log2(n)))
    assert st.stages <= 2 * math.ceil(math.log2(n)) if n > 1 else st.stages == 0


@pytest.mark.parametrize("n,length", [(2, 10), (3, 7), (5, 1003), (8, 4096), (13, 999), (64, 64 * 3 + 5)])
def test_bytes_per_rank_against_the_cost_model(n, length):
    xs = [np.zeros(length, np.float32) for _ in range(n)]
    _, st = dbt.double_binary_tree_allreduce(xs)
    S = 4 * length
    half = [4 * (e - b) for b, e in dbt.halves(length)]
    assert sum(st.sent) == sum(st.received) == 2 * (n - 1) * S
    # per rank: one message up unless root, one down per child, in each tree
    par = dbt.parents(n)
    for r in range(n):
        want = 0
        for t in (0, 1):
            p = (r - t) % n + 1
            kids = sum(c is not None for c in dbt.children(p, n))
            want += half[t] * ((p in par) + kids)
        assert st.sent[r] == want
        assert st.sent[r] <= 2 * S + 8
    # one binary tree carrying the whole buffer: an inner rank below the root would send 3 S
    if n >= 4:
        assert max(S * ((p in par) + sum(c is not None for c in dbt.children(p, n))) for p in range(1, n + 1)) \
            == 3 * S


@pytest.mark.parametrize("n", [1, 2, 3, 6, 8, 17])
def test_closed_forms(n):
    rng = np.random.default_rng(n)
    length = 301
    ints = [rng.integers(-8, 9, size=length).astype(np.float32) for _ in range(n)]
    got, _ = dbt.double_binary_tree_allreduce(ints)
    exact = np.sum(np.stack(ints).astype(np.int64), axis=0)
    for o in got:
        assert np.array_equal(o.astype(np.int64), exact)
    i32 = [rng.integers(-2**31, 2**31, size=length, dtype=np.int64).astype(np.int32) for _ in range(n)]
    wrap = (np.sum(np.stack(i32).astype(np.int64), axis=0) % 2**32).astype(np.uint32).view(np.int32)
    assert np.array_equal(dbt.double_binary_tree_allreduce(i32, "sum", "i32")[0][0], wrap)
    assert np.array_equal(dbt.double_binary_tree_allreduce(i32, "min", "i32")[0][0], np.min(np.stack(i32), axis=0))
    assert np.array_equal(dbt.double_binary_tree_allreduce(i32, "max", "i32")[0][0], np.max(np.stack(i32), axis=0))
    w = wrap.astype(np.int64)
    trunc = np.where(w >= 0, w // n, -((-w) // n)).astype(np.int32)
    assert np.array_equal(dbt.double_binary_tree_allreduce(i32, "avg", "i32")[0][0], trunc)
    # bf16 buffers with float32 partials on small integers: the exact sum rounded once to bf16
    b = [f32_to_bf16_bits(x * np.float32(3.0)) for x in ints]
    exact3 = (exact * 3).astype(np.float32)
    assert np.array_equal(dbt.double_binary_tree_allreduce(b, "sum", "bf16acc32")[0][0], f32_to_bf16_bits(exact3))


def test_float32_error_bound():
    n = 24
    xs = spread(n, 400, seed=3)
    got = dbt.double_binary_tree_allreduce(xs)[0][0]
    u = 2.0 ** -24
    for i in range(400):
        exact = sum(Fraction(float(x[i])) for x in xs)
        mag = sum(abs(Fraction(float(x[i]))) for x in xs)
        assert abs(Fraction(float(got[i])) - exact) <= (n - 1) * u * mag


@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "prod"), ("f32", "max"), ("f32", "min"),
                                      ("bf16", "sum"), ("f16", "avg"), ("i32", "sum"), ("i32", "avg"),
                                      ("bf16acc32", "sum"), ("bf16acc32", "avg")])
def test_schedule_equals_definition(dtype, op):
    """The stage-by-stage schedule equals each half's bracketing evaluated directly."""
    for n in (1, 2, 3, 4, 5, 7, 8, 11, 16):
        for length in (0, 1, 2, 3, 17, 64):
            rng = np.random.default_rng([n, length, 7])
            if dtype == "i32":
                xs = [rng.integers(-2**31, 2**31, size=length, dtype=np.int64).astype(np.int32) for _ in range(n)]
            elif dtype in ("bf16", "bf16acc32"):
                xs = [f32_to_bf16_bits(rng.standard_normal(length).astype(np.float32)) for _ in range(n)]
            elif dtype == "f16":
                xs = [rng.standard_normal(length).astype(np.float16).view(np.uint16) for _ in range(n)]
            else:
                xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
            got, _ = dbt.double_binary_tree_allreduce(xs, op, dtype)
            want = dbt.double_binary_tree_fold(xs, op, dtype)
            for r in range(n):
                assert same_bits(got[r], want, dtype), (n, length, r)


def test_bf16_float32_partials_round_once():
    """bf16acc32: the partials stay float32 and only the root's value is rounded.

    Ranks hold 1, 2^-8, 2^-8, 2^-8, 0, 0.  The exact sum 1 + 3 * 2^-8 lies
    halfway between bf16 neighbours and rounds to even, 1 + 2^-6.  Rounded
    after every step instead, tree 0 adds each 2^-8 to 1 and loses it (a tie
    rounded to even), while tree 1 sums the three small terms first (3 * 2^-8
    is exact in bf16) and then meets 1: the same tie, 1 + 2^-6.
    """
    n = 6
    xs = [f32_to_bf16_bits(np.full(8, v, np.float32)) for v in (1.0, 2.0 ** -8, 2.0 ** -8, 2.0 ** -8, 0.0, 0.0)]
    once = bf16_bits_to_f32(dbt.double_binary_tree_allreduce(xs, "sum", "bf16acc32")[0][0])
    assert np.all(once == np.float32(1.0 + 2.0 ** -6))
    step = bf16_bits_to_f32(dbt.double_binary_tree_allreduce(xs, "sum", "bf16")[0][0])
    assert np.all(step[:4] == np.float32(1.0)) and np.all(step[4:] == np.float32(1.0 + 2.0 ** -6))
