"""Reduce followed by broadcast, executed on N host arrays — TEST INFRASTRUCTURE ONLY.

Sources:

* bitfern.com "AllReduce Explained", section "Reduce Followed by Broadcast":
  the plainest way to an AllReduce.  Each process's values go to one chosen
  process, which adds them up and then sends the finished sum out to all the
  others.  The page notes the load this puts on that one process.
* "2.1 Collective communication primitives in detail", section 3.3
  (Reduce): the reduced result lands on the root only and the other ranks'
  buffers stay as they were; the section's note states that AllReduce is a
  Reduce followed by a Broadcast.

Reading where the pages leave a step open: they fix no order in which the
root combines what it receives.  Here the root folds chunk c (the ring's
floor chunks) starting from rank c's values, then rank c+1's, and so on,
ranks mod N: the ring's association order.  So this schedule reaches the
ring AllReduce's bits, and only the movement of the data differs.  The
messages are counted like the ring's: the root receives N-1 whole buffers
and sends N-1 whole buffers, every other rank sends and receives one.
"""

from __future__ import annotations

from collections import deque

import numpy as np

from .ring import _ITEMSIZE, _STORAGE, _WORK, RingStats, _check_inputs, chunk, finish, reduce_op, to_work


def reduce_to_root(xs, op: str = "sum", dtype: str = "f32", root: int = 0):
    """Reduce onto ``root``; return (buffers, stats).

    Every rank other than the root sends its whole buffer to the root's
    mailbox; the root combines them chunk by chunk in the ring's association
    order and keeps the result.  The other ranks' buffers come back
    unchanged (copies of ``xs``).
    """
    n, length = _check_inputs(xs, dtype)
    if not 0 <= root < n:
        raise ValueError(f"root {root} is not a rank of {n}")
    esz = _ITEMSIZE[dtype]
    stats = RingStats(sent=[0] * n, received=[0] * n)
    mailbox = deque()
    for r in range(n):
        if r != root:
            mailbox.append((r, np.array(xs[r], dtype=_STORAGE[dtype], copy=True)))
            stats.sent[r] += length * esz
    have = {root: np.array(xs[root], dtype=_STORAGE[dtype], copy=True)}
    while mailbox:
        r, msg = mailbox.popleft()
        stats.received[root] += msg.size * esz
        have[r] = msg
    if len(have) != n:
        raise AssertionError("the root is missing a rank's buffer")
    wd = _WORK[dtype]
    out = np.empty(length, dtype=_STORAGE[dtype])
    for c in range(n):
        a, b = chunk(c, n, length)
        acc = to_work(have[c][a:b], dtype)
        for k in range(1, n):
            acc = reduce_op(op, wd, acc, to_work(have[(c + k) % n][a:b], dtype))
        out[a:b] = finish(op, dtype, acc, n)
    bufs = [np.array(x, dtype=_STORAGE[dtype], copy=True) for x in xs]
    bufs[root] = out
    stats.rs_steps = 1
    return bufs, stats


def reduce_then_broadcast(xs, op: str = "sum", dtype: str = "f32", root: int = 0):
    """AllReduce as :func:`reduce_to_root` followed by a broadcast from the
    root; return (buffers, stats).  Every rank ends with the root's result."""
    n, length = _check_inputs(xs, dtype)
    bufs, stats = reduce_to_root(xs, op, dtype, root)
    esz = _ITEMSIZE[dtype]
    mailbox = [deque() for _ in range(n)]
    for r in range(n):
        if r != root:
            mailbox[r].append(bufs[root].copy())
            stats.sent[root] += length * esz
    for r in range(n):
        if r != root:
            msg = mailbox[r].popleft()
            stats.received[r] += msg.size * esz
            bufs[r] = msg
    stats.ag_steps = 1
    return bufs, stats
