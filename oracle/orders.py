"""AllReduce in tree-shaped orders, executed literally on N host arrays — TEST INFRASTRUCTURE ONLY.

Sources (the pages on AllReduce algorithms):

* bitfern.com "AllReduce Explained: Algorithms, Performance, and Distributed
  Training", section "Common AllReduce Algorithms":
  - "Tree AllReduce": workers form a tree; partial results climb to the root,
    then the result travels back down, in a number of stages logarithmic in
    the worker count;
  - "Recursive Doubling": in each round a process swaps data with a partner
    and combines what it receives with its own; the partner distance grows
    from round to round until every process has everyone's data.
* tirogla.com "Ring all-reduce", section "How it works", cost model:
  Rabenseifner's AllReduce is a recursive-halving reduce-scatter followed by
  a recursive-doubling all-gather, for a power-of-two number of ranks, with
  2 log2 N latency terms and the ring's 2(N-1)/N * S bandwidth term.

Readings where the pages leave a step open:

* the tree is the binomial tree rooted at rank 0: in reduction stage k
  (k = 0, 1, ...) rank r with r mod 2^(k+1) = 0 receives the partial of rank
  r + 2^k, when that rank exists, and combines it into its own; the
  distribution retraces the stages in reverse order, each parent sending the
  finished result to the child it received from;
* recursive doubling pairs rank r with r XOR 2^k in round k (distance 1, 2,
  4, ...); it needs a power-of-two N;
* recursive halving pairs rank r with r XOR N/2^(k+1) in stage k; of the
  pair's common range of chunks (the floor chunk plan of the ring), the rank
  whose bit N/2^(k+1) is clear keeps the lower half and the other the upper
  half, so rank r finishes chunk r; the all-gather then doubles the distance
  (1, 2, ..., N/2) and each rank sends everything it holds;
* every combination is "own (op) received", rounded to the working type; the
  finishing step (avg's one division by N, bf16acc32's rounding to bf16)
  happens where a value is complete: at the root (tree), on every rank
  (recursive doubling), on a chunk's last keeper (recursive halving).

Because the operators are commutative, each schedule computes one fixed
bracketing of the N-term reduction for every element, whatever rank holds
it.  :func:`binomial_tree` and :func:`halving_tree` write those bracketings
down from their definitions, and :func:`tree_order_fold` evaluates one
directly: the second implementation the schedules are checked against.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

from .ring import _ITEMSIZE, _STORAGE, _WORK, _check_inputs, _same_bits, chunk, finish, reduce_op, to_work

ORDERS = ("tree", "recursive_doubling", "halving_doubling")


@dataclass
class OrderStats:
    """What a schedule did: per-rank bytes sent and received, and its stage count."""

    sent: list = field(default_factory=list)
    received: list = field(default_factory=list)
    stages: int = 0


def _power_of_two(n: int) -> bool:
    return n >= 1 and (n & (n - 1)) == 0


def _deliver(mailbox, stats, esz, src, dst, payload):
    mailbox[dst].append((src, payload))
    stats.sent[src] += payload[-1].size * esz


def _take(mailbox, stats, esz, dst, want_src):
    src, payload = mailbox[dst].popleft()
    if src != want_src:
        raise AssertionError(f"rank {dst} expected a message from {want_src}, got one from {src}")
    stats.received[dst] += payload[-1].size * esz
    return payload


def _check_equal(out, dtype):
    for r in range(1, len(out)):
        if not _same_bits(out[r], out[0], dtype):
            raise AssertionError("ranks disagree at the end of the schedule")


# --------------------------------------------------------------------------
# binomial tree: reduce to rank 0, then distribute
# --------------------------------------------------------------------------

def tree_allreduce(xs, op: str = "sum", dtype: str = "f32", check: bool = True):
    """Reduce up a binomial tree to rank 0, then send the result back down.

    Returns (outputs, stats).  Stage k of the reduction (distance d = 2^k):
    every rank r with r mod 2d = d sends its partial to r - d, which combines
    it into its own.  After ceil(log2 N) stages rank 0 holds the complete
    value, finishes it, and the distribution runs the stages backwards
    (d = ..., 2, 1): each rank r with r mod 2d = 0 sends the result to r + d.
    """
    n, length = _check_inputs(xs, dtype)
    wd = _WORK[dtype]
    stats = OrderStats(sent=[0] * n, received=[0] * n)
    buf = [to_work(x, dtype) for x in xs]
    mailbox = [deque() for _ in range(n)]
    d = 1
    while d < n:
        for r in range(n):
            if r % (2 * d) == d:
                _deliver(mailbox, stats, _ITEMSIZE[wd], r, r - d, (buf[r].copy(),))
        for r in range(n):
            if r % (2 * d) == 0 and r + d < n:
                (msg,) = _take(mailbox, stats, _ITEMSIZE[wd], r, r + d)
                buf[r] = reduce_op(op, wd, buf[r], msg)
        stats.stages += 1
        d *= 2
    out = [None] * n
    out[0] = finish(op, dtype, buf[0], n)
    d //= 2
    while d >= 1:
        for r in range(n):
            if r % (2 * d) == 0 and r + d < n:
                _deliver(mailbox, stats, _ITEMSIZE[dtype], r, r + d, (out[r].copy(),))
        for r in range(n):
            if r % (2 * d) == d:
                (msg,) = _take(mailbox, stats, _ITEMSIZE[dtype], r, r - d)
                out[r] = msg
        stats.stages += 1
        d //= 2
    if any(mailbox):
        raise AssertionError("messages left undelivered")
    if check:
        _check_equal(out, dtype)
    return out, stats


# --------------------------------------------------------------------------
# recursive doubling: every rank exchanges whole buffers with r XOR 2^k
# --------------------------------------------------------------------------

def recursive_doubling_allreduce(xs, op: str = "sum", dtype: str = "f32", check: bool = True):
    """log2 N rounds; in round k rank r swaps its whole partial with r XOR 2^k.

    Returns (outputs, stats).  Each rank combines "own (op) received"; after
    the last round every rank holds the complete value and finishes it.
    """
    n, length = _check_inputs(xs, dtype)
    if not _power_of_two(n):
        raise ValueError("recursive doubling needs a power-of-two number of ranks")
    wd = _WORK[dtype]
    stats = OrderStats(sent=[0] * n, received=[0] * n)
    buf = [to_work(x, dtype) for x in xs]
    mailbox = [deque() for _ in range(n)]
    d = 1
    while d < n:
        for r in range(n):
            _deliver(mailbox, stats, _ITEMSIZE[wd], r, r ^ d, (buf[r].copy(),))
        for r in range(n):
            (msg,) = _take(mailbox, stats, _ITEMSIZE[wd], r, r ^ d)
            buf[r] = reduce_op(op, wd, buf[r], msg)
        stats.stages += 1
        d *= 2
    out = [finish(op, dtype, b, n) for b in buf]
    if check:
        _check_equal(out, dtype)
    return out, stats


# --------------------------------------------------------------------------
# Rabenseifner: recursive-halving reduce-scatter + recursive-doubling all-gather
# --------------------------------------------------------------------------

def _chunk_span(lo: int, hi: int, n: int, length: int) -> tuple:
    """Element bounds of the chunks [lo, hi) of the floor chunk plan."""
    return chunk(lo, n, length)[0], chunk(hi - 1, n, length)[1]


def halving_doubling_allreduce(xs, op: str = "sum", dtype: str = "f32", check: bool = True):
    """Recursive-halving reduce-scatter, then recursive-doubling all-gather.

    Returns (outputs, stats).  Every rank starts with the chunk range [0, N).
    Reduce-scatter stage k (d = N/2^(k+1)): rank r and r XOR d share a range;
    the one with bit d clear keeps its lower half and the other its upper
    half; each sends the half it gives up and combines the half it receives
    into its own.  After log2 N stages rank r holds chunk r complete and
    finishes it.  All-gather stage k (d = 2^k): rank r sends all the chunks
    it holds to r XOR d and stores what it receives.
    """
    n, length = _check_inputs(xs, dtype)
    if not _power_of_two(n):
        raise ValueError("recursive halving needs a power-of-two number of ranks")
    wd = _WORK[dtype]
    stats = OrderStats(sent=[0] * n, received=[0] * n)
    buf = [to_work(x, dtype) for x in xs]
    mailbox = [deque() for _ in range(n)]
    lo, hi = [0] * n, [n] * n

    def halves(r, d):
        mid = (lo[r] + hi[r]) // 2
        low, high = (lo[r], mid), (mid, hi[r])
        return (low, high) if r & d == 0 else (high, low)     # (kept, given up)

    d = n // 2
    while d >= 1:
        for r in range(n):
            (_, (g0, g1)) = halves(r, d)
            a, b = _chunk_span(g0, g1, n, length)
            _deliver(mailbox, stats, _ITEMSIZE[wd], r, r ^ d, ((g0, g1), buf[r][a:b].copy()))
        for r in range(n):
            (k0, k1), _ = halves(r, d)
            rng, msg = _take(mailbox, stats, _ITEMSIZE[wd], r, r ^ d)
            if rng != (k0, k1):
                raise AssertionError("recursive halving received the wrong chunk range")
            a, b = _chunk_span(k0, k1, n, length)
            buf[r][a:b] = reduce_op(op, wd, buf[r][a:b], msg)
        for r in range(n):
            lo[r], hi[r] = halves(r, d)[0]
        stats.stages += 1
        d //= 2
    out = []
    for r in range(n):
        if (lo[r], hi[r]) != (r, r + 1):
            raise AssertionError(f"rank {r} finished chunks [{lo[r]}, {hi[r]}) instead of chunk {r}")
        a, b = chunk(r, n, length)
        o = np.zeros(length, dtype=_STORAGE[dtype])
        o[a:b] = finish(op, dtype, buf[r][a:b], n)
        out.append(o)
    d = 1
    while d < n:
        for r in range(n):
            a, b = _chunk_span(lo[r], hi[r], n, length)
            _deliver(mailbox, stats, _ITEMSIZE[dtype], r, r ^ d, ((lo[r], hi[r]), out[r][a:b].copy()))
        new = []
        for r in range(n):
            (g0, g1), msg = _take(mailbox, stats, _ITEMSIZE[dtype], r, r ^ d)
            if g0 != hi[r] and g1 != lo[r]:
                raise AssertionError("recursive doubling received a range that does not adjoin its own")
            a, b = _chunk_span(g0, g1, n, length)
            out[r][a:b] = msg
            new.append((min(lo[r], g0), max(hi[r], g1)))
        for r in range(n):
            lo[r], hi[r] = new[r]
        stats.stages += 1
        d *= 2
    if any(mailbox):
        raise AssertionError("messages left undelivered")
    if check:
        for r in range(n):
            if (lo[r], hi[r]) != (0, n):
                raise AssertionError(f"rank {r} ends the all-gather without every chunk")
        _check_equal(out, dtype)
    return out, stats


def order_allreduce(order: str, xs, op: str = "sum", dtype: str = "f32", check: bool = True):
    """Run the schedule named ``order`` (one of :data:`ORDERS`)."""
    if order == "tree":
        return tree_allreduce(xs, op, dtype, check)
    if order == "recursive_doubling":
        return recursive_doubling_allreduce(xs, op, dtype, check)
    if order == "halving_doubling":
        return halving_doubling_allreduce(xs, op, dtype, check)
    raise ValueError(f"unknown order {order!r}")


# --------------------------------------------------------------------------
# the bracketings these schedules compute, written from their definitions
# --------------------------------------------------------------------------

def binomial_tree(n: int):
    """The bracketing of the binomial tree over ranks 0..n-1 (nested 2-tuples).

    The subtree of rank r at level m (a power of two) covers ranks
    [r, r + m) that exist; it joins the subtrees of r and r + m/2 at level
    m/2, or is just r's subtree when r + m/2 does not exist.
    """
    if n < 1:
        raise ValueError("need at least one rank")

    def t(r, m):
        if m == 1:
            return r
        h = m // 2
        if r + h >= n:
            return t(r, h)
        return (t(r, h), t(r + h, h))

    m = 1
    while m < n:
        m *= 2
    return t(0, m)


def halving_tree(n: int):
    """The bracketing of recursive halving over ranks 0..n-1, n a power of two.

    Its last stage joins the ranks of even and odd index (partners at
    distance 1), each of which was joined at distance 2 the stage before, and
    so on: a set of ranks that agree on their low bits splits on the lowest
    bit that still varies, the half with that bit clear on the left.
    """
    if not _power_of_two(n):
        raise ValueError("recursive halving needs a power-of-two number of ranks")

    def t(ranks, bit):
        if len(ranks) == 1:
            return ranks[0]
        return (t([r for r in ranks if not r & bit], bit * 2), t([r for r in ranks if r & bit], bit * 2))

    return t(list(range(n)), 1)


def order_bracketing(order: str, n: int):
    """The bracketing the schedule ``order`` computes for every element."""
    if order in ("tree", "recursive_doubling"):
        if order == "recursive_doubling" and not _power_of_two(n):
            raise ValueError("recursive doubling needs a power-of-two number of ranks")
        return binomial_tree(n)
    if order == "halving_doubling":
        return halving_tree(n)
    raise ValueError(f"unknown order {order!r}")


def tree_order_fold(xs, tree, op: str = "sum", dtype: str = "f32") -> np.ndarray:
    """Evaluate a bracketing on whole buffers: the AllReduce result as a definition.

    Leaves are the ranks' buffers in working precision; each inner node is one
    operation rounded to the working type; the root is finished once (avg's
    division by N, bf16acc32's rounding to bf16).
    """
    n, _ = _check_inputs(xs, dtype)
    wd = _WORK[dtype]

    def ev(t):
        if isinstance(t, tuple):
            return reduce_op(op, wd, ev(t[0]), ev(t[1]))
        return to_work(xs[t], dtype)

    return finish(op, dtype, ev(tree), n)


def tree_order_fold_columns(cols: np.ndarray, tree, op: str = "sum", dtype: str = "f32") -> np.ndarray:
    """:func:`tree_order_fold` on chosen positions: ``cols[r, j]`` is rank r's value at position j."""
    cols = np.asarray(cols)
    return tree_order_fold([cols[r] for r in range(cols.shape[0])], tree, op, dtype)
