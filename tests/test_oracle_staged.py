"""Pins of the reduce-then-broadcast oracle (oracle/staged.py) against the pages
and the mathematics, on the CPU.

* the Reduce example printed in "2.1 Collective communication primitives in
  detail", section 3.3 (tests/golden/p4_worked_examples.json): GPU0 ends
  with the sum, the other GPUs keep their vectors;
* the page's AllReduce example (section 3.4) through reduce then broadcast;
* the reading that the root folds each chunk in the ring's order: bit for
  bit the ring AllReduce's result over every dtype and operator and ragged
  shapes, and on inputs where bracketings give different float32 sums, the
  ring's bracketing and not the plain fold over ranks 0, 1, 2, ...;
* the traffic bitfern.com "AllReduce Explained" warns of: the root
  receives and sends N-1 whole buffers, every other rank one each way.
"""

import json
import os
import zlib

import numpy as np
import pytest

import oracle
from oracle.ring import f32_to_bf16_bits, f32_to_f16_bits, same_bits
from oracle.staged import reduce_then_broadcast, reduce_to_root

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "p4_worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_reduce_example_of_the_page():
    ex = _golden()["reduce_sum_3_4_onto_gpu0"]
    xs = [np.array(v, np.float32) for v in ex["inputs"]]
    out, _ = reduce_to_root(xs, root=ex["root"])
    for r, want in enumerate(ex["expected"]):
        assert np.array_equal(out[r], np.array(want, np.float32)), r
    # the inputs themselves are left alone
    assert np.array_equal(xs[0], np.array(ex["inputs"][0], np.float32))


def test_allreduce_example_through_reduce_then_broadcast():
    ex = _golden()["allreduce_sum_3_4"]
    xs = [np.array(v, np.float32) for v in ex["inputs"]]
    for root in range(4):
        out, _ = reduce_then_broadcast(xs, root=root)
        for r in range(4):
            assert np.array_equal(out[r], np.array(ex["expected"], np.float32)), (root, r)


def _draw(dtype, n, length, rng):
    if dtype == "i32":
        return [rng.integers(-(2**31), 2**31, size=length, dtype=np.int32) for _ in range(n)]
    xs = [(rng.standard_normal(length) * 2.0 ** rng.integers(-20, 20, size=length)).astype(np.float32)
          for _ in range(n)]
    if dtype == "f16":
        return [f32_to_f16_bits(x) for x in xs]
    if dtype in ("bf16", "bf16acc32"):
        return [f32_to_bf16_bits(x) for x in xs]
    return xs


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "i32", "bf16acc32"])
@pytest.mark.parametrize("op", ["sum", "prod", "min", "max", "avg"])
def test_same_bits_as_the_ring(dtype, op):
    rng = np.random.default_rng(zlib.crc32(f"{dtype}-{op}".encode()))
    for n, length in ((1, 5), (2, 3), (3, 100), (4, 1003), (5, 4), (7, 50), (9, 200)):
        xs = _draw(dtype, n, length, rng)
        ring, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
        for root in (0, n - 1):
            got, _ = reduce_then_broadcast(xs, op=op, dtype=dtype, root=root)
            for r in range(n):
                assert same_bits(got[r], ring[r], dtype), (n, length, root, r)


def test_root_folds_in_the_ring_order():
    # 4 ranks, 4 elements: element i belongs to chunk i.  Rotations of
    # (1e8, 1, -1e8, 1): float32 sums depend on the bracketing.
    base = np.array([1e8, 1.0, -1e8, 1.0], np.float32)
    xs = [np.roll(base, -r) for r in range(4)]
    out, _ = reduce_then_broadcast(xs)
    ring = oracle.ring_order_fold(xs)
    plain = np.empty(4, np.float32)
    for i in range(4):
        acc = xs[0][i]
        for r in range(1, 4):
            acc = np.float32(acc + xs[r][i])
        plain[i] = acc
    assert np.array_equal(out[0], ring)
    assert not np.array_equal(ring, plain)          # the inputs do tell the two orders apart
    # chunk 0 starts at rank 0, so there the two orders agree
    assert out[0][0] == plain[0]


@pytest.mark.parametrize("n,length", [(2, 8), (4, 1003), (8, 64)])
def test_bytes_moved(n, length):
    xs = [np.ones(length, np.float32) for _ in range(n)]
    s = 4 * length
    for root in (0, n - 1):
        _, st = reduce_to_root(xs, root=root)
        assert st.received[root] == (n - 1) * s and st.sent[root] == 0
        assert all(st.sent[r] == s and st.received[r] == 0 for r in range(n) if r != root)
        _, st = reduce_then_broadcast(xs, root=root)
        assert st.received[root] == (n - 1) * s and st.sent[root] == (n - 1) * s
        assert all(st.sent[r] == s and st.received[r] == s for r in range(n) if r != root)
        assert sum(st.sent) == sum(st.received) == 2 * (n - 1) * s


def test_rejects_a_root_outside_the_ranks():
    with pytest.raises(ValueError):
        reduce_to_root([np.ones(3, np.float32)] * 2, root=2)
