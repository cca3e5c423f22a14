"""The ring with one thread per rank, driven by message arrival — TEST INFRASTRUCTURE ONLY.

tirogla.com "Ring all-reduce", section "How it works", states the ring as a
rule per rank and step: in reduce-scatter step s rank r passes chunk
(r-s) mod N to rank r+1 and combines the chunk (r-s-1) mod N arriving from
rank r-1 into its own; in all-gather step s it passes chunk (r+1-s) mod N and
overwrites its chunk (r-s) mod N with the arriving one.  The same page runs
the ring as concurrent workers connected by channels.

Here each rank is a small state machine in its own thread.  Its steps are a
table built from the rule above.  It starts by sending its first chunk; from
then on it only reacts to arrivals: each message is checked against the step
it should answer, combined or copied, and the chunk that this just completed
(the next step's outgoing chunk, by the rule) is sent on at once.  No rank
waits for a global step boundary, so the ring runs as a pipeline, and
whatever the interleaving the result must equal the lockstep run in
:mod:`oracle.ring` bit for bit.  A rank that never sends leaves its
neighbour waiting; the wait is bounded and ends in :class:`RingTimeout`
instead of a hang (the pages warn that ranks that disagree on the collective
hang with no error).
"""

from __future__ import annotations

import queue
import threading

import numpy as np

from .ring import _ITEMSIZE, _STORAGE, chunk, reduce_op


class RingTimeout(RuntimeError):
    """A rank waited longer than the time-out for its left neighbour's message."""


def step_table(rank: int, n: int) -> list:
    """Rank ``rank``'s steps in order: (phase, step, chunk sent, chunk received)."""
    table = [("rs", s, (rank - s) % n, (rank - s - 1) % n) for s in range(n - 1)]
    table += [("ag", s, (rank + 1 - s) % n, (rank - s) % n) for s in range(n - 1)]
    return table


class _RankMachine:
    """One rank: its buffer, its step table, and where it stands in it."""

    def __init__(self, rank, n, data, outbox, inbox, op, dtype, timeout, skip, sent):
        self.rank, self.n, self.data = rank, n, data
        self.outbox, self.inbox = outbox, inbox
        self.op, self.dtype, self.timeout = op, dtype, timeout
        self.skip, self.sent = skip, sent
        self.steps = step_table(rank, n)
        self.pos = 0                       # index of the step whose message is awaited

    def _span(self, c):
        return chunk(c, self.n, len(self.data))

    def _send(self, k):
        phase, s, c, _ = self.steps[k]
        if self.skip == (phase, s):
            return                         # a planted fault: this message is never sent
        a, b = self._span(c)
        self.outbox.put((k, c, self.data[a:b].copy()))
        self.sent[self.rank] += (b - a) * _ITEMSIZE[self.dtype]

    def _on_message(self, k, c, payload):
        phase, s, _, want = self.steps[self.pos]
        if k != self.pos or c != want:
            raise AssertionError(f"rank {self.rank} at {phase} step {s} expected chunk {want}, got {c}")
        a, b = self._span(c)
        if phase == "rs":
            self.data[a:b] = reduce_op(self.op, self.dtype, self.data[a:b], payload)
        else:
            self.data[a:b] = payload
        self.pos += 1
        if self.pos < len(self.steps):
            self._send(self.pos)           # forward the chunk just completed

    def run(self):
        if not self.steps:
            return
        self._send(0)
        while self.pos < len(self.steps):
            try:
                k, c, payload = self.inbox.get(timeout=self.timeout)
            except queue.Empty:
                phase, s, _, _ = self.steps[self.pos]
                raise RingTimeout(f"rank {self.rank} got nothing from rank {(self.rank - 1) % self.n} "
                                  f"at {phase} step {s}") from None
            self._on_message(k, c, payload)


def ring_allreduce_threaded(xs, op="sum", dtype="f32", timeout=30.0, skip=None):
    """Run every rank's state machine in its own thread; return (buffers, bytes sent per rank).

    ``skip=(rank, (phase, step))`` makes that rank skip one send ("rs" or "ag",
    step s), which must end in :class:`RingTimeout` rather than a hang.
    """
    n = len(xs)
    bufs = [np.array(x, dtype=_STORAGE[dtype], copy=True) for x in xs]
    inbox = [queue.Queue() for _ in range(n)]               # inbox[r] holds what rank r-1 sent
    sent = [0] * n
    errors = []
    machines = [_RankMachine(r, n, bufs[r], inbox[(r + 1) % n], inbox[r], op, dtype, timeout,
                             skip[1] if (skip is not None and skip[0] == r) else None, sent)
                for r in range(n)]

    def run(m):
        try:
            m.run()
        except BaseException as e:  # noqa: BLE001 - reported to the caller below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(m,), daemon=True) for m in machines]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errors:
        timeouts = [e for e in errors if isinstance(e, RingTimeout)]
        raise timeouts[0] if timeouts else errors[0]
    return bufs, sent
