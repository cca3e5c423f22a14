"""The ring with one thread per rank and queue channels — TEST INFRASTRUCTURE ONLY.

tirogla.com "Ring all-reduce", section "Code", runs the ring as one thread
per rank connected by channels: each rank sends to rank+1 and receives from
rank-1, reduce-scatter first and all-gather second, with the same chunk
indices as the lockstep schedule in :mod:`oracle.ring`.  This module runs
that program with Python threads and ``queue.Queue`` channels.  It must give
the same bits as the lockstep run (the ranks' programs are deterministic
whatever the interleaving), and a rank that never sends makes its neighbour's
receive time out, which is reported as :class:`RingTimeout` instead of a hang
(the pages' pitfall: ranks that disagree on the collective order hang with no
error).
"""

from __future__ import annotations

import queue
import threading

import numpy as np

from .ring import _ITEMSIZE, _STORAGE, chunk, reduce_op


class RingTimeout(RuntimeError):
    """A rank waited longer than the time-out for its left neighbour's message."""


def _rank_program(rank, n, data, tx, rx, op, dtype, timeout, skip, sent):
    length = len(data)
    esz = _ITEMSIZE[dtype]

    def exchange(send_c, recv_c, step_id):
        a, b = chunk(send_c, n, length)
        if skip != step_id:
            tx.put((send_c, data[a:b].copy()))
            sent[rank] += (b - a) * esz
        try:
            c, msg = rx.get(timeout=timeout)
        except queue.Empty:
            raise RingTimeout(f"rank {rank} got nothing from rank {(rank - 1) % n} at {step_id}") from None
        if c != recv_c:
            raise AssertionError(f"rank {rank} expected chunk {recv_c}, got {c}")
        return chunk(c, n, length), msg

    for s in range(n - 1):                                   # reduce-scatter
        (a, b), msg = exchange((rank - s) % n, (rank - s - 1) % n, ("rs", s))
        data[a:b] = reduce_op(op, dtype, data[a:b], msg)
    for s in range(n - 1):                                   # all-gather
        (a, b), msg = exchange((rank + 1 - s) % n, (rank - s) % n, ("ag", s))
        data[a:b] = msg


def ring_allreduce_threaded(xs, op="sum", dtype="f32", timeout=30.0, skip=None):
    """Run every rank's program in its own thread; return (buffers, bytes sent per rank).

    ``skip=(rank, (phase, step))`` makes that rank skip one send, which must
    end in :class:`RingTimeout` rather than a hang.
    """
    n = len(xs)
    bufs = [np.array(x, dtype=_STORAGE[dtype], copy=True) for x in xs]
    chans = [queue.Queue() for _ in range(n)]               # chans[r] delivers to rank r
    sent = [0] * n
    errors = []

    def run(r):
        try:
            my_skip = skip[1] if (skip is not None and skip[0] == r) else None
            _rank_program(r, n, bufs[r], chans[(r + 1) % n], chans[r], op, dtype,
                          timeout, my_skip, sent)
        except BaseException as e:  # noqa: BLE001 - reported to the caller below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(r,), daemon=True) for r in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errors:
        timeouts = [e for e in errors if isinstance(e, RingTimeout)]
        raise timeouts[0] if timeouts else errors[0]
    return bufs, sent
