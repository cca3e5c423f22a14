"""Brute force over tiny rings — TEST INFRASTRUCTURE ONLY.

Two searches that check the lockstep oracle (:mod:`oracle.ring`) from the
outside, on buffers small enough to enumerate:

1. :func:`explore_interleavings` runs every rank's program of the ring
   (tirogla.com "Ring all-reduce", section "How it works": per step, send one
   chunk to rank+1, then receive one from rank-1 and add or overwrite) under
   every possible interleaving of the ranks' events.  With buffered channels
   every interleaving must end, and every path to the same program-counter
   vector must leave the same buffer contents (the result does not depend on
   timing).  With rendezvous channels (a send waits for the matching
   receive) every rank blocks in its first send: the deadlock that
   "2.1 Collective communication primitives in detail", section 1 (point to
   point), warns of for blocking send-then-receive.

2. :func:`bracketings` lists every way to bracket an N-term reduction with a
   commutative operator ((2N-3)!! trees), so a test can show which single
   bracketing the oracle's results agree with.
"""

from __future__ import annotations

from collections import deque

import numpy as np

from .ring import _STORAGE, chunk, reduce_op


def _programs(n: int):
    """Per-rank event lists: ('send', chunk) / ('recv', chunk, 'add'|'copy')."""
    progs = []
    for r in range(n):
        ev = []
        for s in range(n - 1):
            ev.append(("send", (r - s) % n))
            ev.append(("recv", (r - s - 1) % n, "add"))
        for s in range(n - 1):
            ev.append(("send", (r + 1 - s) % n))
            ev.append(("recv", (r - s) % n, "copy"))
        progs.append(ev)
    return progs


def explore_interleavings(xs, op="sum", dtype="f32", capacity=None, max_states=2_000_000):
    """Depth-first search over all interleavings of the ring's events.

    ``capacity``: None for unbounded FIFO channels, k >= 1 for channels that
    hold at most k messages (a send blocks while full), 0 for rendezvous (a
    send completes only together with the matching receive).

    Returns a dict with the number of distinct states, the deadlocked
    program-counter vectors, whether any state was reached with two
    different contents, and the final buffers (None if no path finished).
    """
    n = len(xs)
    length = len(xs[0])
    progs = _programs(n)
    end = tuple(len(p) for p in progs)

    def fingerprint(bufs, chans):
        return (tuple(b.tobytes() for b in bufs),
                tuple(tuple((c, m.tobytes()) for c, m in ch) for ch in chans))

    def apply_recv(bufs, r, ev, msg_c, msg):
        if msg_c != ev[1]:
            raise AssertionError("a rank received a chunk it did not expect")
        a, b = chunk(ev[1], n, length)
        if ev[2] == "add":
            bufs[r][a:b] = reduce_op(op, dtype, bufs[r][a:b], msg)
        else:
            bufs[r][a:b] = msg

    start_bufs = [np.array(x, dtype=_STORAGE[dtype], copy=True) for x in xs]
    start = (tuple([0] * n), start_bufs, [deque() for _ in range(n)])
    seen = {}
    deadlocks = []
    nondeterministic = False
    final = None
    stack = [start]
    while stack:
        pcs, bufs, chans = stack.pop()
        fp = fingerprint(bufs, chans)
        if pcs in seen:
            if seen[pcs] != fp:
                nondeterministic = True
            continue
        seen[pcs] = fp
        if len(seen) > max_states:
            raise RuntimeError("state space larger than max_states")
        if pcs == end:
            final = [b.copy() for b in bufs]
            continue
        moves = []
        for r in range(n):
            if pcs[r] == end[r]:
                continue
            ev = progs[r][pcs[r]]
            dst = (r + 1) % n
            if ev[0] == "send":
                a, b = chunk(ev[1], n, length)
                if capacity == 0:
                    # rendezvous: only together with the receiver's matching receive
                    if pcs[dst] < end[dst] and progs[dst][pcs[dst]][0] == "recv":
                        nb = [x.copy() for x in bufs]
                        apply_recv(nb, dst, progs[dst][pcs[dst]], ev[1], bufs[r][a:b].copy())
                        npc = list(pcs)
                        npc[r] += 1
                        npc[dst] += 1
                        moves.append((tuple(npc), nb, [deque(c) for c in chans]))
                elif capacity is None or len(chans[dst]) < capacity:
                    nch = [deque(c) for c in chans]
                    nch[dst].append((ev[1], bufs[r][a:b].copy()))
                    npc = list(pcs)
                    npc[r] += 1
                    moves.append((tuple(npc), [x.copy() for x in bufs], nch))
            else:
                if capacity != 0 and chans[r]:
                    nch = [deque(c) for c in chans]
                    msg_c, msg = nch[r].popleft()
                    nb = [x.copy() for x in bufs]
                    apply_recv(nb, r, ev, msg_c, msg)
                    npc = list(pcs)
                    npc[r] += 1
                    moves.append((tuple(npc), nb, nch))
        if not moves:
            deadlocks.append(pcs)
        stack.extend(moves)
    return {"states": len(seen), "deadlocks": deadlocks,
            "nondeterministic": nondeterministic, "final": final}


# --------------------------------------------------------------------------
# bracketings of an N-term reduction
# --------------------------------------------------------------------------

def bracketings(leaves):
    """Every full binary tree over ``leaves`` with unordered children.

    A tree is a leaf (an int) or a 2-tuple of trees.  The smallest leaf is
    kept in the first subtree of every split, so each unordered tree appears
    once: 1, 1, 3, 15, 105 trees for 1..5 leaves, that is (2N-3)!!.
    """
    leaves = tuple(sorted(leaves))
    if len(leaves) == 1:
        return [leaves[0]]
    first, rest = leaves[0], leaves[1:]
    out = []
    m = len(rest)
    for mask in range(0, 1 << m):
        left = (first,) + tuple(rest[i] for i in range(m) if mask >> i & 1)
        right = tuple(rest[i] for i in range(m) if not mask >> i & 1)
        if not right:
            continue
        for lt in bracketings(left):
            for rt in bracketings(right):
                out.append((lt, rt))
    return out


def canonical(tree):
    """A form of ``tree`` that is the same for trees equal up to swapping children."""
    if isinstance(tree, tuple):
        a, b = canonical(tree[0]), canonical(tree[1])
        return (a, b) if repr(a) <= repr(b) else (b, a)
    return tree


def ring_tree(c: int, n: int):
    """The ring's bracketing of chunk c: (((x_c, x_c+1), x_c+2), ...), ranks mod n."""
    t = c % n
    for k in range(1, n):
        t = (t, (c + k) % n)
    return t


def evaluate(tree, values, op="sum", dtype="f32"):
    """Value of a bracketing, rounding to the dtype after every operation."""
    if isinstance(tree, tuple):
        return reduce_op(op, dtype, evaluate(tree[0], values, op, dtype),
                         evaluate(tree[1], values, op, dtype))
    return np.asarray(values[tree])
