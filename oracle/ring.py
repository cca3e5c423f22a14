"""Ring AllReduce executed literally on N host arrays — TEST INFRASTRUCTURE ONLY.

Sources (the pages on ring AllReduce):

* tirogla.com "Ring all-reduce", section "How it works": ranks 0..N-1 form a
  ring and the buffer is cut into N chunks.  Reduce-scatter step s
  (s = 0..N-2): rank r sends chunk (r-s) mod N to rank r+1, receives chunk
  (r-s-1) mod N from rank r-1 and adds it to its own copy; afterwards rank r
  holds the complete sum of chunk (r+1) mod N.  All-gather step s: rank r
  sends chunk (r+1-s) mod N, receives chunk (r-s) mod N and overwrites.  The
  same page's "Code" section fixes the chunk bounds as
  [c*len/N, (c+1)*len/N) with integer (floor) division, uneven on purpose,
  and the receiving rank adds the incoming values into its own buffer.
* ramchalamkr.github.io "NCCL Primitives Deep Dive", section "Ring
  All-Gather": the standalone all-gather in which rank r starts with shard r
  in slot r and at step s sends slot (r-s) mod N and receives slot
  (r-s-1) mod N.
* "2.1 Collective communication primitives in detail", section 3.5
  (ReduceScatter): rank i keeps the reduced shard i.

Readings where the pages leave a step open:

* standalone reduce-scatter returns shard c to rank c.  The ring finishes
  chunk c on rank c-1; the oracle takes the finished chunk from there, so
  reduce-scatter followed by all-gather reproduces AllReduce bit for bit;
* bf16 buffers are rounded to bf16 after every ring step (the sum of two
  bf16 values is formed in float32 and rounded to nearest-even once);
* int32 sum and product wrap modulo 2^32;
* float min/max follow IEEE 754-2019 minimum/maximum: a NaN operand gives
  NaN, and -0 is below +0;
* ``avg`` is the ring's sum followed by one division by N, done by the rank
  that finishes the chunk ("2.1 Collective communication primitives in
  detail", section 3.4, and bitfern.com "AllReduce Explained": sum, then
  divide by the number of workers): float division rounded once to the
  buffer type, integer division truncating toward zero;
* ``bf16acc32`` keeps bf16 buffers but lets the partial sums travel in
  float32, rounding to bf16 once when a chunk is finished (tirogla.com "Ring
  all-reduce", implementation notes: reduce in fp32, or bf16 with fp32
  accumulation).

Buffers: ``f32`` -> numpy float32, ``i32`` -> numpy int32, ``bf16``,
``bf16acc32`` and ``f16`` -> numpy uint16 holding the raw bit patterns.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "bf16", "i32", "f16", "bf16acc32")
OPS = ("sum", "prod", "min", "max", "avg")

_STORAGE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "f16": np.uint16, "bf16acc32": np.uint16}
_ITEMSIZE = {"f32": 4, "bf16": 2, "i32": 4, "f16": 2, "bf16acc32": 2}
# precision the partial sums travel in: the buffer's own, except float32 partials for bf16acc32
_WORK = {"f32": "f32", "bf16": "bf16", "i32": "i32", "f16": "f16", "bf16acc32": "f32"}


# --------------------------------------------------------------------------
# chunk plan (tirogla.com "Ring all-reduce", section "Code": chunk(c, n, len))
# --------------------------------------------------------------------------

def chunk(c: int, n: int, length: int) -> tuple:
    """Bounds [start, end) of chunk ``c`` of a ``length``-element buffer cut in ``n``.

    Floor division as on the page: chunks differ in length by at most one
    element and may be empty when ``length < n``.
    """
    return (c * length) // n, ((c + 1) * length) // n


def chunk_owner(positions, n: int, length: int) -> np.ndarray:
    """Index of the chunk that holds each element position.

    Found by searching the chunk ends produced by :func:`chunk` (the first
    chunk whose end lies beyond the position), so empty chunks are skipped.
    """
    ends = np.array([chunk(c, n, length)[1] for c in range(n)], dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    if pos.size and (pos.min() < 0 or pos.max() >= length):
        raise IndexError("position outside the buffer")
    return np.searchsorted(ends, pos, side="right").astype(np.int64)


# --------------------------------------------------------------------------
# bfloat16 (bit patterns in uint16)
# --------------------------------------------------------------------------

def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32: the bf16 bits are the top half."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, to nearest with ties to even.

    The 16 discarded bits are compared with one half of the last kept bit:
    adding 0x7FFF plus the last kept bit carries into the kept half exactly
    when the discarded part is above one half, or equal to one half with an
    odd last kept bit.  A carry out of the mantissa raises the exponent, and
    past the largest finite value gives infinity, as IEEE rounding does.
    NaN inputs give a quiet NaN with the input's sign.
    """
    f = np.ascontiguousarray(f, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    quiet_nan = ((bits >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return np.where(np.isnan(f), quiet_nan, rounded)


def f16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen IEEE binary16 bit patterns to float32 (exact)."""
    return np.asarray(u, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16, to nearest with ties to even (numpy's conversion).

    Overflow gives infinity, results below the normal range keep binary16's
    subnormal spacing of 2^-24, and NaN stays NaN.
    """
    with np.errstate(over="ignore", invalid="ignore"):
        return np.ascontiguousarray(f, dtype=np.float32).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# element operators
# --------------------------------------------------------------------------

def _ieee_minimum(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    out = np.where(a < b, a, b)
    tie = a == b                      # equal values, including +0 against -0
    out = np.where(tie, np.where(np.signbit(a), a, b), out)
    return np.where(np.isnan(a) | np.isnan(b), np.float32(np.nan), out).astype(np.float32)


def _ieee_maximum(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    out = np.where(a > b, a, b)
    tie = a == b
    out = np.where(tie, np.where(np.signbit(a), b, a), out)
    return np.where(np.isnan(a) | np.isnan(b), np.float32(np.nan), out).astype(np.float32)


def _f32_op(op: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    if op == "sum":
        with np.errstate(over="ignore", invalid="ignore"):
            return np.add(a, b, dtype=np.float32)
    if op == "prod":
        with np.errstate(over="ignore", under="ignore", invalid="ignore"):
            return np.multiply(a, b, dtype=np.float32)
    if op == "min":
        return _ieee_minimum(a, b)
    if op == "max":
        return _ieee_maximum(a, b)
    raise ValueError(f"unknown op {op!r}")


def reduce_op(op: str, dtype: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """``a (op) b`` elementwise, rounded to the buffer dtype.

    f32: one IEEE binary32 operation, round to nearest even.
    bf16 / f16: the operation in float32 on the widened values, then one
    rounding to the 16-bit type (the per-step rounding such a ring performs).
    i32: sum and product wrap modulo 2^32; min and max are exact.
    ``avg`` combines like ``sum``; its division happens once, in :func:`finish`.
    """
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}")
    if op == "avg":
        op = "sum"
    if dtype == "f32":
        return _f32_op(op, np.asarray(a, np.float32), np.asarray(b, np.float32))
    if dtype == "bf16":
        return f32_to_bf16_bits(_f32_op(op, bf16_bits_to_f32(a), bf16_bits_to_f32(b)))
    if dtype == "f16":
        return f32_to_f16_bits(_f32_op(op, f16_bits_to_f32(a), f16_bits_to_f32(b)))
    if dtype == "i32":
        a = np.asarray(a, np.int32)
        b = np.asarray(b, np.int32)
        if op == "sum":
            return np.add(a.view(np.uint32), b.view(np.uint32), dtype=np.uint32).view(np.int32)
        if op == "prod":
            return np.multiply(a.view(np.uint32), b.view(np.uint32), dtype=np.uint32).view(np.int32)
        if op == "min":
            return np.minimum(a, b)
        return np.maximum(a, b)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_work(x: np.ndarray, dtype: str) -> np.ndarray:
    """A rank's buffer in the precision its partial sums travel in (a copy)."""
    if dtype == "bf16acc32":
        return bf16_bits_to_f32(x)
    return np.array(x, dtype=_STORAGE[dtype], copy=True)


def finish(op: str, dtype: str, v: np.ndarray, n: int) -> np.ndarray:
    """Complete a finished chunk (in working precision) and return it in the buffer type.

    ``avg`` divides the sum by N once: float division rounded to the buffer
    type (16-bit types: the float32 quotient rounded once more, which is the
    correctly rounded quotient since 24 >= 2*11+2), int32 division truncating
    toward zero.  bf16acc32 rounds its float32 partial to bf16 here.
    """
    wd = _WORK[dtype]
    if op == "avg":
        if wd == "f32":
            with np.errstate(over="ignore", invalid="ignore"):
                v = np.divide(np.asarray(v, np.float32), np.float32(n), dtype=np.float32)
        elif wd == "bf16":
            v = f32_to_bf16_bits(np.divide(bf16_bits_to_f32(v), np.float32(n), dtype=np.float32))
        elif wd == "f16":
            v = f32_to_f16_bits(np.divide(f16_bits_to_f32(v), np.float32(n), dtype=np.float32))
        else:
            w = np.asarray(v, np.int32).astype(np.int64)
            q = np.where(w >= 0, w // n, -((-w) // n))
            v = q.astype(np.int32)
    if dtype == "bf16acc32":
        return f32_to_bf16_bits(np.asarray(v, np.float32))
    return np.asarray(v, dtype=_STORAGE[dtype])


# --------------------------------------------------------------------------
# the ring schedule, executed
# --------------------------------------------------------------------------

@dataclass
class RingStats:
    """What the schedule did: per-rank bytes sent and received, and step counts."""

    sent: list = field(default_factory=list)
    received: list = field(default_factory=list)
    rs_steps: int = 0
    ag_steps: int = 0


def _check_inputs(xs, dtype: str):
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    n = len(xs)
    if n < 1:
        raise ValueError("need at least one rank")
    length = len(xs[0])
    for x in xs:
        if len(x) != length:
            raise ValueError("every rank must hold the same number of elements")
    return n, length


def _reduce_scatter_phase(buf, mailbox, stats, op, dtype, on_step):
    """Reduce-scatter: N-1 steps; each rank sends one chunk right and adds the one from the left.

    ``buf`` holds the ranks' working copies and ``dtype`` is the working
    precision (messages are counted at its element size).
    """
    n = len(buf)
    length = len(buf[0])
    esz = _ITEMSIZE[dtype]
    for s in range(n - 1):
        for r in range(n):                                  # every rank sends ...
            c = (r - s) % n
            a, b = chunk(c, n, length)
            msg = buf[r][a:b].copy()
            mailbox[(r + 1) % n].append((c, msg))
            stats.sent[r] += msg.size * esz
        for r in range(n):                                  # ... then every rank receives and adds
            c, msg = mailbox[r].popleft()
            if c != (r - s - 1) % n:
                raise AssertionError("reduce-scatter received the wrong chunk")
            stats.received[r] += msg.size * esz
            a, b = chunk(c, n, length)
            buf[r][a:b] = reduce_op(op, dtype, buf[r][a:b], msg)
        stats.rs_steps += 1
        if on_step is not None:
            on_step("reduce_scatter", s, buf)


def _all_gather_phase(buf, mailbox, stats, dtype, on_step, send_of, recv_of, phase):
    n = len(buf)
    length = len(buf[0])
    esz = _ITEMSIZE[dtype]
    for s in range(n - 1):
        for r in range(n):
            c = send_of(r, s) % n
            a, b = chunk(c, n, length)
            msg = buf[r][a:b].copy()
            mailbox[(r + 1) % n].append((c, msg))
            stats.sent[r] += msg.size * esz
        for r in range(n):
            c, msg = mailbox[r].popleft()
            if c != recv_of(r, s) % n:
                raise AssertionError("all-gather received the wrong chunk")
            stats.received[r] += msg.size * esz
            a, b = chunk(c, n, length)
            buf[r][a:b] = msg                               # overwrite, no arithmetic
        stats.ag_steps += 1
        if on_step is not None:
            on_step(phase, s, buf)


def ring_allreduce(xs, op: str = "sum", dtype: str = "f32", on_step=None, check=True):
    """Run the ring AllReduce schedule on N host arrays; return (outputs, stats).

    ``xs[r]`` is rank r's buffer (left untouched).  The schedule is the one
    stated on tirogla.com "Ring all-reduce" ("How it works"): N-1
    reduce-scatter steps, then N-1 all-gather steps, with each message placed
    in the receiver's FIFO mailbox and counted in bytes.  ``on_step(phase, s,
    bufs)`` is called after every step with the ranks' current buffers.

    With ``check`` the run also asserts what the page states about it: after
    reduce-scatter rank r's chunk (r+1) mod N is complete (compared with the
    closed definition, :func:`ring_order_fold`), and afterwards every rank
    holds the same bits.
    """
    n, length = _check_inputs(xs, dtype)
    stats = RingStats(sent=[0] * n, received=[0] * n)
    buf = _reduce_scatter_and_finish(xs, op, dtype, on_step, stats)
    mailbox = [deque() for _ in range(n)]
    if check and n > 1:
        want = ring_order_fold(xs, op, dtype)
        for r in range(n):
            a, b = chunk((r + 1) % n, n, length)
            if not _same_bits(buf[r][a:b], want[a:b], dtype):
                raise AssertionError(f"rank {r} does not hold the finished chunk {(r + 1) % n}")

    _all_gather_phase(buf, mailbox, stats, dtype, on_step,
                      send_of=lambda r, s: r + 1 - s, recv_of=lambda r, s: r - s,
                      phase="all_gather")
    if any(mailbox):
        raise AssertionError("messages left undelivered")
    if check:
        for r in range(1, n):
            if not _same_bits(buf[r], buf[0], dtype):
                raise AssertionError("ranks disagree after the all-gather")
    return buf, stats


def _reduce_scatter_and_finish(xs, op, dtype, on_step, stats):
    """The reduce-scatter steps in working precision; then rank r completes the
    chunk it finished, chunk (r+1) mod N, and every buffer returns to the
    buffer type (its unfinished chunks are overwritten by the all-gather)."""
    n, length = len(xs), len(xs[0])
    buf = [to_work(x, dtype) for x in xs]
    mailbox = [deque() for _ in range(n)]
    _reduce_scatter_phase(buf, mailbox, stats, op, _WORK[dtype], on_step)
    if any(mailbox):
        raise AssertionError("messages left undelivered")
    out = []
    for r in range(n):
        a, b = chunk((r + 1) % n, n, length)
        o = f32_to_bf16_bits(buf[r]) if dtype == "bf16acc32" else buf[r]
        o[a:b] = finish(op, dtype, buf[r][a:b], n)
        out.append(o)
    return out


def reduce_scatter(xs, op: str = "sum", dtype: str = "f32", on_step=None):
    """Standalone reduce-scatter: returns (shards, stats) with shard c on rank c.

    Runs the ring's N-1 reduce-scatter steps; rank c-1 then holds the finished
    chunk c, which is handed to rank c (the reduced shard i belongs to rank i,
    "2.1 Collective communication primitives in detail", section 3.5).
    """
    n, length = _check_inputs(xs, dtype)
    stats = RingStats(sent=[0] * n, received=[0] * n)
    buf = _reduce_scatter_and_finish(xs, op, dtype, on_step, stats)
    shards = []
    for c in range(n):
        a, b = chunk(c, n, length)
        shards.append(buf[(c - 1) % n][a:b].copy())
    return shards, stats


def all_gather(shards, length: int, dtype: str = "f32", on_step=None, poison=None):
    """Standalone ring all-gather: rank r starts with shard r; returns (buffers, stats).

    Follows ramchalamkr.github.io "NCCL Primitives Deep Dive", section "Ring
    All-Gather": the shard sits in slot r, and at step s rank r sends slot
    (r-s) mod N and receives slot (r-s-1) mod N.  Slots not yet received hold
    ``poison`` (NaN for float32, 0xDEADBEEF for int32, 0xDEAD for the 16-bit
    types) so a missed slot cannot pass unnoticed.  ``on_step`` also sees the
    starting state, as phase "start" with step -1.
    """
    n = len(shards)
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    if poison is None:
        poison = {"f32": np.float32(np.nan), "bf16": np.uint16(0xDEAD), "bf16acc32": np.uint16(0xDEAD),
                  "f16": np.uint16(0xDEAD), "i32": np.uint32(0xDEADBEEF).view(np.int32)}[dtype]
    buf = []
    for r in range(n):
        a, b = chunk(r, n, length)
        if len(shards[r]) != b - a:
            raise ValueError(f"shard {r} must hold {b - a} elements")
        x = np.full(length, poison, dtype=_STORAGE[dtype])
        x[a:b] = shards[r]
        buf.append(x)
    mailbox = [deque() for _ in range(n)]
    stats = RingStats(sent=[0] * n, received=[0] * n)
    if on_step is not None:
        on_step("start", -1, buf)
    _all_gather_phase(buf, mailbox, stats, dtype, on_step,
                      send_of=lambda r, s: r - s, recv_of=lambda r, s: r - s - 1,
                      phase="all_gather")
    return buf, stats


# --------------------------------------------------------------------------
# the closed definition of the result (the ring's association order)
# --------------------------------------------------------------------------

def ring_order_fold(xs, op: str = "sum", dtype: str = "f32") -> np.ndarray:
    """The AllReduce result written as a definition, without the schedule.

    Chunk c starts on rank c and picks up one rank's values per hop
    (arjunsriva.com "AllReduce, All the Way Down", figure "Ring AllReduce ·
    follow chunk 0": A0, then A0+B0, then +C0, then +D0; tirogla.com "Ring
    all-reduce": chunk c travels r = c, c+1, ... accumulating), so each
    element of chunk c is the left fold
    ((x_c (op) x_{c+1}) (op) x_{c+2}) ... (op) x_{c+N-1}, ranks mod N,
    rounded to the buffer dtype after every operation.
    """
    n, length = _check_inputs(xs, dtype)
    wd = _WORK[dtype]
    out = np.empty(length, dtype=_STORAGE[dtype])
    for c in range(n):
        a, b = chunk(c, n, length)
        acc = to_work(xs[c][a:b], dtype)
        for k in range(1, n):
            acc = reduce_op(op, wd, acc, to_work(xs[(c + k) % n][a:b], dtype))
        out[a:b] = finish(op, dtype, acc, n)
    return out


def ring_order_fold_columns(cols: np.ndarray, owners, op: str = "sum", dtype: str = "f32") -> np.ndarray:
    """:func:`ring_order_fold` at chosen positions only.

    ``cols[r, j]`` is rank r's value at the j-th chosen position and
    ``owners[j]`` the chunk that position belongs to; the fold starts at rank
    ``owners[j]`` and goes round the ring.  Used to check single elements of
    buffers too large to run the whole schedule on.
    """
    cols = np.asarray(cols)
    n, m = cols.shape
    wd = _WORK.get(dtype, dtype)
    owners = np.asarray(owners, dtype=np.int64)
    j = np.arange(m)
    acc = to_work(cols[owners % n, j], dtype)
    for k in range(1, n):
        acc = reduce_op(op, wd, acc, to_work(cols[(owners + k) % n, j], dtype))
    return finish(op, dtype, acc, n)


def _same_bits(a: np.ndarray, b: np.ndarray, dtype: str) -> bool:
    """Bitwise equality, except that any two NaNs of a float dtype are equal."""
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return False
    if dtype == "f32":
        nan_a, nan_b = np.isnan(a), np.isnan(b)
        return bool(np.array_equal(nan_a, nan_b)
                    and np.array_equal(a.view(np.uint32)[~nan_a], b.view(np.uint32)[~nan_b]))
    if dtype in ("bf16", "bf16acc32", "f16"):
        widen = f16_bits_to_f32 if dtype == "f16" else bf16_bits_to_f32
        fa, fb = widen(a), widen(b)
        nan_a, nan_b = np.isnan(fa), np.isnan(fb)
        return bool(np.array_equal(nan_a, nan_b) and np.array_equal(a[~nan_a], b[~nan_b]))
    return bool(np.array_equal(a, b))


def same_bits(a, b, dtype: str) -> bool:
    """Public form of the comparison the tests use (NaNs compared as a class)."""
    return _same_bits(a, b, dtype)
