"""Brute-force checks of the oracle on tiny rings, the threaded ring, and
planted mistakes that the pins must catch."""

import numpy as np
import pytest

import oracle
from oracle import explore as E
from oracle import ring as R
from oracle.threaded import RingTimeout, ring_allreduce_threaded


def _disc_values(n, length, seed):
    """float32 values with widely spread magnitudes, so the order of additions shows."""
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(length) * 2.0 ** rng.integers(-12, 24, size=length)).astype(np.float32)
            for _ in range(n)]


@pytest.mark.parametrize("n,length", [(2, 2), (2, 3), (3, 3), (3, 4), (4, 4), (4, 5)])
def test_every_interleaving_ends_with_the_same_result(n, length):
    xs = _disc_values(n, length, seed=n * 10 + length)
    res = E.explore_interleavings(xs)
    assert res["deadlocks"] == []
    assert not res["nondeterministic"]
    want, _ = oracle.ring_allreduce(xs)
    for got, w in zip(res["final"], want):
        assert np.array_equal(got.view(np.uint32), w.view(np.uint32))
    # reachable program-counter vectors: at most (4(N-1)+1)^N
    assert res["states"] <= (4 * (n - 1) + 1) ** n


@pytest.mark.parametrize("n", [2, 3, 4])
def test_single_slot_channels_do_not_deadlock(n):
    xs = _disc_values(n, n, seed=n)
    res = E.explore_interleavings(xs, capacity=1)
    assert res["deadlocks"] == [] and not res["nondeterministic"]
    want, _ = oracle.ring_allreduce(xs)
    assert all(np.array_equal(a, b) for a, b in zip(res["final"], want))


@pytest.mark.parametrize("n", [2, 3, 4])
def test_rendezvous_channels_deadlock_at_the_first_send(n):
    xs = _disc_values(n, n, seed=n)
    res = E.explore_interleavings(xs, capacity=0)
    assert res["deadlocks"] == [tuple([0] * n)]
    assert res["final"] is None


@pytest.mark.parametrize("n,count", [(1, 1), (2, 1), (3, 3), (4, 15), (5, 105), (6, 945)])
def test_number_of_bracketings(n, count):
    trees = E.bracketings(range(n))
    assert len(trees) == count
    assert len({repr(E.canonical(t)) for t in trees}) == count


@pytest.mark.parametrize("n", [3, 4, 5])
def test_the_oracle_follows_exactly_one_bracketing_per_chunk(n):
    trees = E.bracketings(range(n))
    consistent = {c: set(range(len(trees))) for c in range(n)}
    for trial in range(40):
        xs = _disc_values(n, n, seed=1000 + trial)       # one element per chunk
        out, _ = oracle.ring_allreduce(xs)
        for c in range(n):
            vals = [x[c] for x in xs]
            for t in list(consistent[c]):
                if E.evaluate(trees[t], vals).view(np.uint32) != out[0][c].view(np.uint32):
                    consistent[c].discard(t)
    for c in range(n):
        assert [repr(E.canonical(trees[t])) for t in consistent[c]] == [repr(E.canonical(E.ring_tree(c, n)))]


def test_cancelling_rotations_single_out_the_ring_order():
    # {1e8, 1, -1e8, 1} rotated over 4 ranks: the chunk's result depends on where the fold starts
    n = 4
    base = np.array([1e8, 1.0, -1e8, 1.0], np.float32)
    for c in range(n):
        xs = [np.zeros(n, np.float32) for _ in range(n)]
        for r in range(n):
            xs[r][c] = base[(r - c) % n]
        out, _ = oracle.ring_allreduce(xs)
        # the fold starts at rank c: ((1e8 + 1) - 1e8) + 1 = 1 in float32
        assert out[0][c] == np.float32(1.0)


@pytest.mark.parametrize("n,length", [(1, 7), (2, 5), (3, 1), (6, 1001), (8, 8 * 64 + 3)])
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "sum"), ("i32", "max")])
def test_threaded_ring_equals_lockstep(dtype, op, n, length):
    rng = np.random.default_rng(4)
    if dtype == "f32":
        xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
    elif dtype == "bf16":
        xs = [R.f32_to_bf16_bits(rng.standard_normal(length).astype(np.float32)) for _ in range(n)]
    else:
        xs = [rng.integers(-(2**31), 2**31, size=length, dtype=np.int32) for _ in range(n)]
    want, st = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    got, sent = ring_allreduce_threaded(xs, op=op, dtype=dtype)
    for g, w in zip(got, want):
        assert R.same_bits(g, w, dtype)
    assert sent == st.sent


def test_a_rank_that_skips_a_send_times_out_instead_of_hanging():
    xs = _disc_values(4, 8, seed=1)
    with pytest.raises(RingTimeout):
        ring_allreduce_threaded(xs, timeout=0.5, skip=(2, ("rs", 1)))


# --------------------------------------------------------------------------
# planted mistakes: a wrong oracle must fail its pins
# --------------------------------------------------------------------------

def test_planted_wrong_receive_index_is_caught(monkeypatch):
    orig = R._reduce_scatter_phase

    def wrong(buf, mailbox, stats, op, dtype, on_step):
        n = len(buf)
        length = len(buf[0])
        for s in range(n - 1):
            for r in range(n):
                c = (r - s) % n
                a, b = R.chunk(c, n, length)
                mailbox[(r + 1) % n].append((c, buf[r][a:b].copy()))
            for r in range(n):
                c, msg = mailbox[r].popleft()
                a, b = R.chunk((r - s) % n, n, length)    # planted: adds into its own chunk
                if b - a == len(msg):
                    buf[r][a:b] = R.reduce_op(op, dtype, buf[r][a:b], msg)
    monkeypatch.setattr(R, "_reduce_scatter_phase", wrong)
    xs = [np.full(8, r + 1, np.float32) for r in range(4)]
    with pytest.raises(AssertionError):
        oracle.ring_allreduce(xs)
    monkeypatch.setattr(R, "_reduce_scatter_phase", orig)


def test_planted_wrong_fold_start_is_caught(monkeypatch):
    def shifted(xs, op="sum", dtype="f32"):
        n, length = len(xs), len(xs[0])
        out = np.empty(length, np.float32)
        for c in range(n):
            a, b = R.chunk(c, n, length)
            acc = xs[(c + 1) % n][a:b].copy()               # planted: starts one rank late
            for k in range(2, n + 1):
                acc = R.reduce_op(op, dtype, acc, xs[(c + k) % n][a:b])
            out[a:b] = acc
        return out
    xs = _disc_values(4, 4, seed=77)
    want, _ = oracle.ring_allreduce(xs, check=False)
    got = shifted(xs)
    assert not np.array_equal(got, want[0])


def test_planted_ceil_chunks_fail_the_chunk_pin():
    def ceil_chunk(c, n, length):
        return -(-c * length // n), -(-(c + 1) * length // n)
    assert [ceil_chunk(c, 5, 1003) for c in range(5)] != [R.chunk(c, 5, 1003) for c in range(5)]
