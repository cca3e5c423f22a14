"""Mutation tests of the oracle: a plausible mistake anywhere in it must fail a pin.

Each case applies one textual change to the oracle's own source
(oracle/ring.py or oracle/orders.py), loads the result as a separate module,
and runs a battery of pins against it: values the pages print, closed forms,
hand-typed bracketings and invariants, none of them computed by the module
under test.  The unchanged source passes every pin; every mutant must fail at
least one.  A mutant may also fail by raising (its own consistency checks
firing is a pin doing its job).
"""

import json
import os
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


# a mutant that loops forever fails instead of hanging the suite
pytestmark = pytest.mark.timeout(60)


def _load(relpath, mutation=None, name="mutant"):
    """The module at relpath, with ``mutation`` (one (old, new) pair or a list of them) applied."""
    src = open(os.path.join(ROOT, relpath)).read()
    if mutation is not None:
        pairs = [mutation] if isinstance(mutation[0], str) else mutation
        for old, new in pairs:
            assert src.count(old) == 1, f"mutation target must occur once: {old!r}"
            src = src.replace(old, new)
    mod = types.ModuleType(f"oracle._{name}")
    mod.__package__ = "oracle"
    mod.__file__ = os.path.join(ROOT, relpath)
    sys.modules[mod.__name__] = mod
    try:
        exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
    return mod


# --------------------------------------------------------------------------
# pins against oracle/ring.py
# --------------------------------------------------------------------------

def _ring_pins(R):
    """(name, ok) for each pin; ok is False or an exception when the pin catches something."""
    out = []

    def pin(name, fn):
        try:
            out.append((name, bool(fn())))
        except Exception as e:  # noqa: BLE001 - a raising mutant is a caught mutant
            out.append((name, e))

    # chunk bounds of the 5 x 1003 example (tirogla.com "Ring all-reduce", section "Code"), worked by hand
    pin("chunks", lambda: [R.chunk(c, 5, 1003) for c in range(5)] ==
        [(0, 200), (200, 401), (401, 601), (601, 802), (802, 1003)])

    # every rank gets the plain sum of small integers (exact in any order)
    def exact_sum():
        rng = np.random.default_rng(1)
        for n in (2, 3, 4, 7):
            xs = [rng.integers(-8, 9, size=37).astype(np.float32) for _ in range(n)]
            out, st = R.ring_allreduce(xs)
            if not all(np.array_equal(o, np.sum(xs, axis=0).astype(np.float32)) for o in out):
                return False
        return True
    pin("exact sum", exact_sum)

    # bytes per rank: 2(N-1)/N * S when N divides len
    def bytes_sent():
        xs = [np.ones(40, np.float32) for _ in range(4)]
        _, st = R.ring_allreduce(xs)
        return st.sent == [2 * 3 * 40 * 4 // 4] * 4
    pin("bytes", bytes_sent)

    # the chunk-0 journey figure: chunk 0 is ((A0 + B0) + C0) + D0, so cancelling
    # values in that order give an exact 1 where other orders give 0
    def journey():
        # four ranks, one element per chunk; position 0 (chunk 0) holds A0..D0
        xs = [np.array([v, 0, 0, 0], np.float32) for v in (1e8, 1.0, -1e8, 1.0)]
        out, _ = R.ring_allreduce(xs)
        return all(float(o[0]) == 1.0 for o in out)
    pin("chunk-0 order", journey)

    # reduce-scatter gives shard c to rank c ("2.1 ...", section 3.5 example)
    def rs_example():
        ex = json.load(open(os.path.join(GOLDEN, "p4_worked_examples.json")))
        case = ex["reduce_scatter_sum_4x4"]
        shards, _ = R.reduce_scatter([np.array(v, np.float32) for v in case["inputs"]])
        return all(np.array_equal(s, np.array(w, np.float32).reshape(-1)) for s, w in zip(shards, case["expected_shards"]))
    pin("reduce-scatter example", rs_example)

    # bf16 rounding against torch's conversion on ties and random patterns
    def bf16():
        import torch
        rng = np.random.default_rng(3)
        bits = np.concatenate([rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32),
                               (np.arange(2**12, dtype=np.uint32) << 16) | 0x8000]).view(np.float32)
        bits = bits[np.isfinite(bits)]
        want = torch.from_numpy(bits).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return np.array_equal(R.f32_to_bf16_bits(bits), want)
    pin("bf16 rounding", bf16)

    # IEEE minimum/maximum on signed zeros and NaN
    def minmax():
        a = np.array([0.0, -0.0, np.nan, 1.0], np.float32)
        b = np.array([-0.0, 0.0, 1.0, np.nan], np.float32)
        mn = R.reduce_op("min", "f32", a, b)
        mx = R.reduce_op("max", "f32", a, b)
        return (np.signbit(mn[:2]).all() and not np.signbit(mx[:2]).any()
                and np.isnan(mn[2:]).all() and np.isnan(mx[2:]).all())
    pin("ieee min/max", minmax)

    # int32 sum wraps; avg truncates toward zero
    def int_closed_forms():
        xs = [np.array([2**31 - 1, -7, 5], np.int32), np.array([1, 0, 0], np.int32), np.array([0, 0, 0], np.int32)]
        out, _ = R.ring_allreduce(xs, "sum", "i32")
        avg, _ = R.ring_allreduce(xs, "avg", "i32")
        return (out[0].tolist() == [-(2**31), -7, 5]) and avg[0].tolist() == [-(2**31) // 3 + 1, -2, 1]
    pin("int32 wrap and avg", int_closed_forms)

    # bf16 with float32 partials keeps what per-step rounding loses: 256 + 1 + 1 is 258 exactly,
    # while per-step bf16 rounds 257 to 256 (ties to even) twice
    def acc32():
        xs = [R.f32_to_bf16_bits(np.array([v], np.float32)) for v in (256.0, 1.0, 1.0)]
        per_step, _ = R.ring_allreduce(xs, "sum", "bf16")
        acc, _ = R.ring_allreduce(xs, "sum", "bf16acc32")
        return int(per_step[0][0]) == 0x4380 and int(acc[0][0]) == 0x4381
    pin("bf16 with float32 partials", acc32)

    # binary16: 1 + 2^-11 is a tie between 1 and 1 + 2^-10 and rounds to even (1), twice
    def f16():
        import torch
        xs = [np.array([v], np.float16).view(np.uint16) for v in (1.0, 2.0 ** -11, 2.0 ** -11)]
        out, _ = R.ring_allreduce(xs, "sum", "f16")
        rng = np.random.default_rng(4)
        vals = (rng.standard_normal(5000) * 2.0 ** rng.integers(-20, 16, 5000)).astype(np.float32)
        want = torch.from_numpy(vals).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        return int(out[0][0]) == 0x3C00 and np.array_equal(R.f32_to_f16_bits(vals), want)
    pin("binary16", f16)

    # float avg: the sum divided by N once, correctly rounded (7/3 in float32)
    def avg_f32():
        xs = [np.array([v], np.float32) for v in (1.0, 2.0, 4.0)]
        out, _ = R.ring_allreduce(xs, "avg", "f32")
        return float(out[0][0]) == float(np.float32(7.0) / np.float32(3.0))
    pin("float avg", avg_f32)

    return out


RING_MUTANTS = [
    ("ceil chunks", ("return (c * length) // n, ((c + 1) * length) // n",
                     "return -(-c * length // n), -(-(c + 1) * length // n)")),
    ("send the wrong chunk", ("            c = (r - s) % n\n            a, b = chunk(c, n, length)\n            msg = buf[r][a:b].copy()\n            mailbox[(r + 1) % n].append((c, msg))\n            stats.sent[r] += msg.size * esz\n        for r in range(n):                                  # ... then every rank receives and adds",
                              "            c = (r - s - 1) % n\n            a, b = chunk(c, n, length)\n            msg = buf[r][a:b].copy()\n            mailbox[(r + 1) % n].append((c, msg))\n            stats.sent[r] += msg.size * esz\n        for r in range(n):                                  # ... then every rank receives and adds")),
    ("overwrite instead of add", ("            buf[r][a:b] = reduce_op(op, dtype, buf[r][a:b], msg)\n        stats.rs_steps += 1",
                                  "            buf[r][a:b] = msg\n        stats.rs_steps += 1")),
    ("bf16 ties away", ("rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)",
                        "rounded = ((bits + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)")),
    ("min tie picks +0", ("    out = np.where(tie, np.where(np.signbit(a), a, b), out)\n    return np.where(np.isnan(a) | np.isnan(b), np.float32(np.nan), out).astype(np.float32)\n\n\ndef _ieee_maximum",
                          "    out = np.where(tie, np.where(np.signbit(a), b, a), out)\n    return np.where(np.isnan(a) | np.isnan(b), np.float32(np.nan), out).astype(np.float32)\n\n\ndef _ieee_maximum")),
    ("int avg floors", ("q = np.where(w >= 0, w // n, -((-w) // n))", "q = w // n")),
    ("int sum saturates", ("return np.add(a.view(np.uint32), b.view(np.uint32), dtype=np.uint32).view(np.int32)",
                           "return np.clip(a.astype(np.int64) + b, -2**31, 2**31 - 1).astype(np.int32)")),
    ("shard taken from rank c", ("shards.append(buf[(c - 1) % n][a:b].copy())", "shards.append(buf[c][a:b].copy())")),
    ("bf16acc32 rounds every step", ('"i32": "i32", "f16": "f16", "bf16acc32": "f32"}', '"i32": "i32", "f16": "f16", "bf16acc32": "bf16"}')),
    ("f16 widened as bf16", ("return f32_to_f16_bits(_f32_op(op, f16_bits_to_f32(a), f16_bits_to_f32(b)))",
                             "return f32_to_f16_bits(_f32_op(op, bf16_bits_to_f32(a), bf16_bits_to_f32(b)))")),
    ("float avg multiplies", ("v = np.divide(np.asarray(v, np.float32), np.float32(n), dtype=np.float32)",
                              "v = np.multiply(np.asarray(v, np.float32), np.float32(n), dtype=np.float32)")),
    ("avg divides by N - 1", ("def finish(op: str, dtype: str, v: np.ndarray, n: int) -> np.ndarray:",
                              "def finish(op: str, dtype: str, v: np.ndarray, n: int) -> np.ndarray:\n    n = max(1, n - 1)")),
    ("fold starts one rank late", ("        acc = to_work(xs[c][a:b], dtype)\n        for k in range(1, n):\n            acc = reduce_op(op, wd, acc, to_work(xs[(c + k) % n][a:b], dtype))",
                                   "        acc = to_work(xs[(c + 1) % n][a:b], dtype)\n        for k in range(2, n + 1):\n            acc = reduce_op(op, wd, acc, to_work(xs[(c + k) % n][a:b], dtype))")),
]


def test_ring_oracle_passes_every_pin():
    R = _load("oracle/ring.py", name="ring_unmutated")
    bad = [(name, ok) for name, ok in _ring_pins(R) if ok is not True]
    assert not bad, bad


@pytest.mark.parametrize("label,mutation", RING_MUTANTS, ids=[m[0] for m in RING_MUTANTS])
def test_ring_mutant_fails_a_pin(label, mutation):
    R = _load("oracle/ring.py", mutation, name="ring_mutant")
    results = _ring_pins(R)
    assert any(ok is not True for _, ok in results), f"mutant {label!r} passed every pin"


# --------------------------------------------------------------------------
# pins against oracle/orders.py
# --------------------------------------------------------------------------

TREE = {3: ((0, 1), 2), 4: ((0, 1), (2, 3)), 5: (((0, 1), (2, 3)), 4), 8: (((0, 1), (2, 3)), ((4, 5), (6, 7)))}
HALVING = {4: ((0, 2), (1, 3)), 8: (((0, 4), (2, 6)), ((1, 5), (3, 7)))}


def _orders_pins(O):
    from oracle.explore import evaluate
    from oracle.ring import same_bits

    out = []

    def pin(name, fn):
        try:
            out.append((name, bool(fn())))
        except Exception as e:  # noqa: BLE001
            out.append((name, e))

    def spread(n, m, seed):
        rng = np.random.default_rng(seed)
        return [(rng.choice([-1.0, 1.0], m) * rng.uniform(1, 2, m) * np.exp2(rng.integers(-20, 21, m)))
                .astype(np.float32) for _ in range(n)]

    def bracket(fn, trees):
        for n, t in trees.items():
            xs = spread(n, 256, n)
            got, _ = fn(xs)
            if not all(same_bits(g, evaluate(t, xs), "f32") for g in got):
                return False
        return True
    pin("tree bracketing", lambda: bracket(O.tree_allreduce, TREE))
    pin("recursive doubling bracketing", lambda: bracket(O.recursive_doubling_allreduce, {4: TREE[4], 8: TREE[8]}))
    pin("halving bracketing", lambda: bracket(O.halving_doubling_allreduce, HALVING))
    pin("definitions", lambda: O.binomial_tree(5) == TREE[5] and O.halving_tree(8) == HALVING[8])

    def exact(fn, ns):
        rng = np.random.default_rng(9)
        for n in ns:
            for length in (1, 5, 3 * n + 2):
                ints = [rng.integers(-8, 9, size=length) for _ in range(n)]
                got, _ = fn([x.astype(np.float32) for x in ints])
                if not all(np.array_equal(g, np.sum(ints, axis=0).astype(np.float32)) for g in got):
                    return False
                got, _ = fn([x.astype(np.int32) for x in ints], "avg", "i32")
                s = np.sum(ints, axis=0)
                if not all(np.array_equal(g, (np.sign(s) * (np.abs(s) // n)).astype(np.int32)) for g in got):
                    return False
        return True
    pin("tree exact", lambda: exact(O.tree_allreduce, (2, 3, 5, 6, 7)))
    pin("recursive doubling exact", lambda: exact(O.recursive_doubling_allreduce, (2, 4, 8)))
    pin("halving exact", lambda: exact(O.halving_doubling_allreduce, (2, 4, 8, 16)))

    def counts():
        S = 64 * 8 * 4
        xs = [np.ones(64 * 8, np.float32) for _ in range(8)]
        _, a = O.recursive_doubling_allreduce(xs)
        _, b = O.halving_doubling_allreduce(xs)
        _, c = O.tree_allreduce(xs)
        return (a.stages == 3 and a.sent == [3 * S] * 8 and b.stages == 6 and b.sent == [2 * 7 * S // 8] * 8
                and c.stages == 6 and sum(c.sent) == 2 * 7 * S)
    pin("stages and bytes", counts)
    return out


ORDER_MUTANTS = [
    ("recursive doubling from the largest distance", [
        ("    d = 1\n    while d < n:\n        for r in range(n):\n            _deliver(mailbox, stats, _ITEMSIZE[wd], r, r ^ d, (buf[r].copy(),))",
         "    d = n // 2\n    while d >= 1:\n        for r in range(n):\n            _deliver(mailbox, stats, _ITEMSIZE[wd], r, r ^ d, (buf[r].copy(),))"),
        ("        stats.stages += 1\n        d *= 2\n    out = [finish(op, dtype, b, n) for b in buf]",
         "        stats.stages += 1\n        d //= 2\n    out = [finish(op, dtype, b, n) for b in buf]")]),
    ("tree drops a partial subtree", ("            if r % (2 * d) == 0 and r + d < n:\n                (msg,) = _take(",
                                      "            if r % (2 * d) == 0 and r + 2 * d <= n:\n                (msg,) = _take(")),
    ("recursive doubling forgets to add", ("            (msg,) = _take(mailbox, stats, _ITEMSIZE[wd], r, r ^ d)\n            buf[r] = reduce_op(op, wd, buf[r], msg)",
                                           "            (msg,) = _take(mailbox, stats, _ITEMSIZE[wd], r, r ^ d)\n            buf[r] = msg")),
    ("halving from distance 1", [
        ("    d = n // 2\n    while d >= 1:\n        for r in range(n):\n            (_, (g0, g1)) = halves(r, d)",
         "    d = 1\n    while d < n:\n        for r in range(n):\n            (_, (g0, g1)) = halves(r, d)"),
        ("        stats.stages += 1\n        d //= 2\n    out = []",
         "        stats.stages += 1\n        d *= 2\n    out = []")]),
    ("halving keeps the wrong half", ("return (low, high) if r & d == 0 else (high, low)", "return (high, low) if r & d == 0 else (low, high)")),
    ("avg divides by 2", ("    out = [finish(op, dtype, b, n) for b in buf]", "    out = [finish(op, dtype, b, 2) for b in buf]")),
    ("chunk span ends early", ("return chunk(lo, n, length)[0], chunk(hi - 1, n, length)[1]", "return chunk(lo, n, length)[0], chunk(lo, n, length)[1]")),
    ("halving tree splits on the top bit", ("        return (t([r for r in ranks if not r & bit], bit * 2), t([r for r in ranks if r & bit], bit * 2))\n\n    return t(list(range(n)), 1)",
                                            "        return (t([r for r in ranks if not r & bit], bit // 2), t([r for r in ranks if r & bit], bit // 2))\n\n    return t(list(range(n)), n // 2)")),
]


def test_orders_oracle_passes_every_pin():
    O = _load("oracle/orders.py", name="orders_unmutated")
    bad = [(name, ok) for name, ok in _orders_pins(O) if ok is not True]
    assert not bad, bad


@pytest.mark.parametrize("label,mutation", ORDER_MUTANTS, ids=[m[0] for m in ORDER_MUTANTS])
def test_orders_mutant_fails_a_pin(label, mutation):
    O = _load("oracle/orders.py", mutation, name="orders_mutant")
    results = _orders_pins(O)
    assert any(ok is not True for _, ok in results), f"mutant {label!r} passed every pin"


# --------------------------------------------------------------------------
# pins against oracle/staged.py
# --------------------------------------------------------------------------

def _staged_pins(S):
    """(name, ok) for each pin of the reduce-then-broadcast oracle."""
    out = []

    def pin(name, fn):
        try:
            out.append((name, bool(fn())))
        except Exception as e:  # noqa: BLE001 - a raising mutant is a caught mutant
            out.append((name, e))

    with open(os.path.join(GOLDEN, "p4_worked_examples.json")) as f:
        gold = json.load(f)

    # the Reduce example of "2.1 ..." section 3.3: GPU0 gets the sum, the others keep their vectors
    def reduce_example():
        ex = gold["reduce_sum_3_4_onto_gpu0"]
        xs = [np.array(v, np.float32) for v in ex["inputs"]]
        got, _ = S.reduce_to_root(xs, root=ex["root"])
        return all(np.array_equal(g, np.array(w, np.float32)) for g, w in zip(got, ex["expected"]))
    pin("reduce example", reduce_example)

    # the AllReduce example of section 3.4 from every root
    def allreduce_example():
        ex = gold["allreduce_sum_3_4"]
        xs = [np.array(v, np.float32) for v in ex["inputs"]]
        for root in range(4):
            got, _ = S.reduce_then_broadcast(xs, root=root)
            if not all(np.array_equal(g, np.array(ex["expected"], np.float32)) for g in got):
                return False
        return True
    pin("allreduce example", allreduce_example)

    # the ring's bracketing, typed by hand for 4 ranks x 4 elements: element i starts at rank i
    def ring_order():
        base = np.array([1e8, 1.0, -1e8, 1.0], np.float32)
        xs = [np.roll(base, -r) for r in range(4)]
        want = []
        for i in range(4):
            acc = xs[i][i]
            for k in range(1, 4):
                acc = np.float32(acc + xs[(i + k) % 4][i])
            want.append(acc)
        got, _ = S.reduce_then_broadcast(xs, root=2)
        return all(np.array_equal(g, np.array(want, np.float32)) for g in got)
    pin("ring order", ring_order)

    # ragged chunks and avg, against integer closed forms: sum, then one truncating division
    def ragged_avg():
        rng = np.random.default_rng(7)
        xs = [rng.integers(-1000, 1000, size=1003).astype(np.int32) for _ in range(5)]
        got, _ = S.reduce_then_broadcast(xs, op="avg", dtype="i32", root=1)
        tot = np.sum(np.stack(xs).astype(np.int64), axis=0)
        want = np.where(tot >= 0, tot // 5, -((-tot) // 5)).astype(np.int32)
        return all(np.array_equal(g, want) for g in got)
    pin("ragged avg", ragged_avg)

    # bytes: the root receives and sends N-1 buffers, every other rank one each way
    def traffic():
        xs = [np.ones(10, np.float32) for _ in range(4)]
        _, st = S.reduce_then_broadcast(xs, root=3)
        return st.received == [40, 40, 40, 120] and st.sent == [40, 40, 40, 120]
    pin("traffic", traffic)
    return out


STAGED_MUTANTS = [
    ("root folds every chunk from rank 0",
     ("acc = to_work(have[c][a:b], dtype)", "acc = to_work(have[0][a:b], dtype)")),
    ("root folds from its own rank",
     ("acc = reduce_op(op, wd, acc, to_work(have[(c + k) % n][a:b], dtype))",
      "acc = reduce_op(op, wd, acc, to_work(have[(root + k) % n][a:b], dtype))")),
    ("avg left undivided", ("out[a:b] = finish(op, dtype, acc, n)", "out[a:b] = acc.astype(_STORAGE[dtype])")),
    ("broadcast skips the last rank", ("    for r in range(n):\n        if r != root:\n            msg = mailbox[r].popleft()",
                                       "    for r in range(n - 1):\n        if r != root:\n            msg = mailbox[r].popleft()")),
    ("other ranks' buffers taken from the result", ("bufs = [np.array(x, dtype=_STORAGE[dtype], copy=True) for x in xs]",
                                                    "bufs = [out.copy() for x in xs]")),
    ("root's sends not counted", ("            stats.sent[root] += length * esz\n", "")),
]


def test_staged_oracle_passes_every_pin():
    S = _load("oracle/staged.py", name="staged_unmutated")
    bad = [(name, ok) for name, ok in _staged_pins(S) if ok is not True]
    assert not bad, bad


@pytest.mark.parametrize("label,mutation", STAGED_MUTANTS, ids=[m[0] for m in STAGED_MUTANTS])
def test_staged_mutant_fails_a_pin(label, mutation):
    S = _load("oracle/staged.py", mutation, name="staged_mutant")
    results = _staged_pins(S)
    assert any(ok is not True for _, ok in results), f"mutant {label!r} passed every pin"


# --------------------------------------------------------------------------
# pins against oracle/dbt.py
# --------------------------------------------------------------------------

# the two trees typed by hand from the construction (as in test_oracle_dbt.py)
DBT0 = {4: (((0, 1), 2), 3), 6: ((((0, 1), 2), 3), (4, 5)), 8: (((((0, 1), 2), 3), ((4, 5), 6)), 7)}
DBT1 = {4: (((1, 2), 3), 0), 6: ((((1, 2), 3), 4), (5, 0)), 8: (((((1, 2), 3), 4), ((5, 6), 7)), 0)}


def _dbt_pins(D):
    from oracle.explore import evaluate
    from oracle.ring import same_bits

    out = []

    def pin(name, fn):
        try:
            out.append((name, bool(fn())))
        except Exception as e:  # noqa: BLE001
            out.append((name, e))

    def spread(n, m, seed):
        rng = np.random.default_rng(seed)
        return [(rng.choice([-1.0, 1.0], m) * rng.uniform(1, 2, m) * np.exp2(rng.integers(-20, 21, m)))
                .astype(np.float32) for _ in range(n)]

    def bracket():
        for n in DBT0:
            m = 257                                   # odd: the halves are 128 and 129 elements
            xs = spread(n, m, n)
            got, _ = D.double_binary_tree_allreduce(xs)
            want = np.concatenate([evaluate(DBT0[n], [x[:128] for x in xs]),
                                   evaluate(DBT1[n], [x[128:] for x in xs])])
            if not all(same_bits(g, want, "f32") for g in got):
                return False
        return True
    pin("hand-typed trees on each half", bracket)
    pin("definitions", lambda: all(D.double_binary_trees(n) == (DBT0[n], DBT1[n]) for n in DBT0))

    def exact():
        rng = np.random.default_rng(11)
        for n in (2, 3, 5, 6, 7, 9, 16):
            for length in (1, 5, 3 * n + 2):
                ints = [rng.integers(-8, 9, size=length) for _ in range(n)]
                got, _ = D.double_binary_tree_allreduce([x.astype(np.float32) for x in ints])
                if not all(np.array_equal(g, np.sum(ints, axis=0).astype(np.float32)) for g in got):
                    return False
                got, _ = D.double_binary_tree_allreduce([x.astype(np.int32) for x in ints], "avg", "i32")
                s = np.sum(ints, axis=0)
                if not all(np.array_equal(g, (np.sign(s) * (np.abs(s) // n)).astype(np.int32)) for g in got):
                    return False
        return True
    pin("exact sums and int avg", exact)

    def cost():
        for n in (5, 8, 13):
            length = 64 * n
            S = 4 * length
            _, st = D.double_binary_tree_allreduce([np.ones(length, np.float32) for _ in range(n)])
            if st.stages != 2 * (n.bit_length() - 1) or sum(st.sent) != 2 * (n - 1) * S or max(st.sent) > 2 * S + 8:
                return False
        return True
    pin("stages and bytes", cost)
    return out


DBT_MUTANTS = [
    ("second tree not moved on", ("    return (p - 1 + tree) % n", "    return (p - 1) % n")),
    ("right child takes the smallest step", ("    for j in range(h - 1, -1, -1):", "    for j in range(0, h):")),
    ("own value joins after both children", [
        ("                v = reduce_op(op, wd, mail.take(me, rank_of(left, t, n), (t, \"up\", left), _ITEMSIZE[wd]),\n                              val[t][p])",
         "                v = mail.take(me, rank_of(left, t, n), (t, \"up\", left), _ITEMSIZE[wd])"),
        ("                val[t][p] = v\n                up(t, p, v)",
         "                v = reduce_op(op, wd, v, val[t][p])\n                val[t][p] = v\n                up(t, p, v)")]),
    ("halves split by ceiling", ("    return chunk(0, 2, length), chunk(1, 2, length)",
                                 "    return (0, (length + 1) // 2), ((length + 1) // 2, length)")),
    ("root left unfinished", ("        final[t][top] = finish(op, dtype, val[t][top], n)",
                              "        final[t][top] = finish(op, dtype, val[t][top], 1)")),
    ("distribution skips right children", ("                    for c in children(p, n):\n                        if c is not None:\n                            mail.send(",
                                           "                    for c in children(p, n)[:1]:\n                        if c is not None:\n                            mail.send(")),
    ("root one level too low", ("    while 2 * r <= n:", "    while 2 * r < n:")),
]


def test_dbt_oracle_passes_every_pin():
    D = _load("oracle/dbt.py", name="dbt_unmutated")
    bad = [(name, ok) for name, ok in _dbt_pins(D) if ok is not True]
    assert not bad, bad


@pytest.mark.parametrize("label,mutation", DBT_MUTANTS, ids=[m[0] for m in DBT_MUTANTS])
def test_dbt_mutant_fails_a_pin(label, mutation):
    D = _load("oracle/dbt.py", mutation, name="dbt_mutant")
    results = _dbt_pins(D)
    assert any(ok is not True for _, ok in results), f"mutant {label!r} passed every pin"
