"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print for worked examples (fixtures under ``tests/golden/``), closed
forms, invariants the pages state, special cases that reduce to a library
routine, and exact arithmetic.  None of them re-derives the oracle's own
formula.
"""

import json
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ring as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(rows):
    return [np.array(r, dtype=np.float32) for r in rows]


# --------------------------------------------------------------------------
# chunk plan
# --------------------------------------------------------------------------

def test_chunk_bounds_of_the_rust_main_example():
    # 1003 elements over 5 ranks, worked out by hand: 200.6 per chunk, floored bounds
    bounds = [R.chunk(c, 5, 1003) for c in range(5)]
    assert bounds == [(0, 200), (200, 401), (401, 601), (601, 802), (802, 1003)]


def test_chunk_bounds_partition_and_balance():
    for n in (1, 2, 3, 4, 5, 7, 8, 16, 64):
        for length in (0, 1, 2, n - 1, n, n + 1, 2 * n + 3, 1000, 4099):
            if length < 0:
                continue
            b = [R.chunk(c, n, length) for c in range(n)]
            assert b[0][0] == 0 and b[-1][1] == length
            for c in range(1, n):
                assert b[c][0] == b[c - 1][1]
            sizes = [e - s for s, e in b]
            assert min(sizes) >= 0 and max(sizes) - min(sizes) <= 1
            assert sum(sizes) == length


def test_chunk_sizes_of_the_64_rank_uneven_workload():
    # 2^26 + 7 elements over 64 ranks: 2^20 each, plus one extra element in the
    # chunks where floor(7c/64) steps up, i.e. c = 9, 18, 27, 36, 45, 54, 63
    n, length = 64, (1 << 26) + 7
    sizes = {c: R.chunk(c, n, length)[1] - R.chunk(c, n, length)[0] for c in range(n)}
    longer = sorted(c for c, s in sizes.items() if s == (1 << 20) + 1)
    assert longer == [9, 18, 27, 36, 45, 54, 63]
    assert all(s == 1 << 20 for c, s in sizes.items() if c not in longer)
    # 64-bit arithmetic: the last chunk's end, (c+1) * len, exceeds 2^32 before the division
    assert 64 * length > 1 << 32 and R.chunk(63, n, length)[1] == length


def test_chunk_owner_against_scan():
    for n in (1, 3, 4, 5, 8):
        for length in (0, 1, 3, n, n + 1, 37):
            want = []
            for i in range(length):
                want.append(next(c for c in range(n)
                                 if R.chunk(c, n, length)[0] <= i < R.chunk(c, n, length)[1]))
            got = R.chunk_owner(np.arange(length), n, length)
            assert list(got) == want


# --------------------------------------------------------------------------
# worked examples printed on the pages
# --------------------------------------------------------------------------

def test_rust_main_every_rank_gets_the_plain_sum():
    g = _golden_json("p4_worked_examples.json")["rust_main"]
    n, length = g["nranks"], g["length"]
    xs = [np.array([r * length + i for i in range(length)], dtype=np.float32) for r in range(n)]
    out, stats = oracle.ring_allreduce(xs)
    # closed form in exact integers: sum over r of (r*len + i) = len*n(n-1)/2 + n*i
    want = np.array([length * n * (n - 1) // 2 + n * i for i in range(length)], dtype=np.float64)
    for r in range(n):
        assert np.array_equal(out[r].astype(np.float64), want)
    assert stats.rs_steps == n - 1 and stats.ag_steps == n - 1


def test_infra_guide_allreduce_example():
    g = _golden_json("p4_worked_examples.json")["allreduce_sum_3_4"]
    out, _ = oracle.ring_allreduce(_f32(g["inputs"]))   # 3 elements on 4 ranks: chunk 0 is empty
    for o in out:
        assert o.tolist() == g["expected"]


def test_p3_allreduce_example():
    g = _golden_json("p4_worked_examples.json")["allreduce_p3_example"]
    xs = [np.ones(g["length"], np.float32) * s for s in g["inputs_scale"]]
    out, _ = oracle.ring_allreduce(xs)
    for o in out:
        assert np.all(o == g["expected_value"])


def test_infra_guide_reduce_scatter_example():
    g = _golden_json("p4_worked_examples.json")["reduce_scatter_sum_4x4"]
    shards, _ = oracle.reduce_scatter(_f32(g["inputs"]))
    assert [s.tolist() for s in shards] == g["expected_shards"]


@pytest.mark.parametrize("key", ["all_gather_letters", "all_gather_p3_example"])
def test_all_gather_examples(key):
    g = _golden_json("p4_worked_examples.json")[key]
    shards = _f32(g["shards"])
    out, _ = oracle.all_gather(shards, length=sum(len(s) for s in shards))
    for o in out:
        assert o.tolist() == g["expected"]


def test_lab_values():
    g = _golden_json("p4_worked_examples.json")
    n = g["lab_allreduce"]["nranks"]
    out, _ = oracle.ring_allreduce([np.array([r], np.float32) for r in range(n)])
    assert all(o.tolist() == [g["lab_allreduce"]["expected"]] for o in out)
    out, _ = oracle.all_gather([np.array([r], np.float32) for r in range(n)], length=n)
    assert all(o.tolist() == g["lab_allgather"]["expected"] for o in out)
    shards, _ = oracle.reduce_scatter([np.array([10 * r + i for i in range(n)], np.float32)
                                       for r in range(n)])
    assert [s.tolist() for s in shards] == [[60 + 4 * r] for r in range(n)]


# --------------------------------------------------------------------------
# the per-step state tables (tagged inputs decode who contributed)
# --------------------------------------------------------------------------

def _parse_table(name):
    steps = {}
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            m = re.match(r"step (\d+)$", line)
            if m:
                cur = int(m.group(1))
                steps[cur] = {}
                continue
            m = re.match(r"GPU_(\d+): \[(.*)\]$", line)
            steps[cur][int(m.group(1))] = [c.strip() for c in m.group(2).split(",")]
    return steps


def test_reduce_scatter_state_table():
    table = _parse_table("p3_reduce_scatter_states.txt")
    n = 4
    # rank r's value in chunk c is 2^(4c + r): a partial sum's bits name its contributors
    xs = [np.array([2.0 ** (4 * c + r) for c in range(n)], np.float32) for r in range(n)]
    states = {}

    def grab(phase, s, bufs):
        if phase == "reduce_scatter":
            states[s + 1] = [b.copy() for b in bufs]

    oracle.ring_allreduce(xs, on_step=grab)
    for step, rows in table.items():
        for gpu, cells in rows.items():
            for c, cell in enumerate(cells):
                letters = re.findall(r"([A-D])(\d)", cell)
                assert all(ord(L) - ord("A") == c for L, _ in letters)
                want = {int(d) for _, d in letters}
                v = int(states[step][gpu][c])
                got = {r for r in range(n) if (v >> (4 * c + r)) & 1}
                assert got == want, (step, gpu, c)


def test_all_gather_state_table():
    table = _parse_table("p3_all_gather_states.txt")
    n = 4
    shards = [np.array([float(r + 1)], np.float32) for r in range(n)]
    states = {}

    def grab(phase, s, bufs):
        states[s + 1] = [b.copy() for b in bufs]      # the start arrives as step -1

    out, _ = oracle.all_gather(shards, length=n, on_step=grab)
    assert sorted(states) == sorted(table)
    for step, rows in table.items():
        for gpu, cells in rows.items():
            for c, cell in enumerate(cells):
                v = states[step][gpu][c]
                if cell == "_":
                    assert np.isnan(v), (step, gpu, c)
                else:
                    assert v == ord(cell) - ord("A") + 1, (step, gpu, c)
    assert all(o.tolist() == [1, 2, 3, 4] for o in out)


def test_chunk0_journey_and_its_association_order():
    n = 4
    stages = []
    with open(os.path.join(GOLDEN, "p1_chunk0_journey.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                st, rank, content = line.split()
                stages.append((int(st), int(rank[1:]), content))
    # one element per chunk; rank r's chunk-0 value is 2^r (letters A-D = ranks 0-3)
    xs = [np.array([2.0 ** r] + [0.0] * (n - 1), np.float32) for r in range(n)]
    snaps = {0: [x.copy() for x in xs]}

    def grab(phase, s, bufs):
        snaps[(s + 1) if phase == "reduce_scatter" else (n + s)] = [b.copy() for b in bufs]

    oracle.ring_allreduce(xs, on_step=grab)
    for st, rank, content in stages:
        if content == "S0":
            want = set(range(n))
        else:
            want = {ord(t[0]) - ord("A") for t in content.split("+")}
        v = int(snaps[st][rank][0])
        assert {r for r in range(n) if v >> r & 1} == want, (st, rank)

    # the left fold of the figure: (((A0 + B0) + C0) + D0), rounding at each step.
    # 2^24 + 1 rounds back to 2^24 in float32, so only this order gives 0.
    vals = [2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]
    xs = [np.array([vals[r]] + [0.0] * (n - 1), np.float32) for r in range(n)]
    out, _ = oracle.ring_allreduce(xs)
    assert all(o[0] == 0.0 for o in out)
    # chunk c starts on rank c: the same four values rotated so rank c holds 2^24
    for c in range(n):
        xs = [np.zeros(n, np.float32) for _ in range(n)]
        for k in range(n):
            xs[(c + k) % n][c] = vals[k]
        out, _ = oracle.ring_allreduce(xs)
        assert out[0][c] == 0.0
        # any other starting rank gives a non-zero result
        for start in range(1, n):
            acc = np.float32(vals[start])
            for k in range(1, n):
                acc = np.float32(acc + np.float32(vals[(start + k) % n]))
            assert acc != 0.0


# --------------------------------------------------------------------------
# invariants the pages state
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,length", [(2, 10), (3, 10), (4, 16), (5, 1003), (8, 999), (16, 5)])
def test_finished_chunk_after_reduce_scatter(n, length):
    rng = np.random.default_rng(7)
    xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
    last = {}

    def grab(phase, s, bufs):
        if phase == "reduce_scatter" and s == n - 2:
            last["bufs"] = [b.copy() for b in bufs]

    oracle.ring_allreduce(xs, on_step=grab, check=False)
    exact = np.sum(np.stack(xs).astype(np.float64), axis=0)
    for r in range(n):
        a, b = R.chunk((r + 1) % n, n, length)
        got = last["bufs"][r][a:b].astype(np.float64)
        bound = (n - 1) * 2.0 ** -24 * np.sum(np.abs(np.stack(xs)[:, a:b]).astype(np.float64), axis=0)
        assert np.all(np.abs(got - exact[a:b]) <= bound + 1e-45)
        # and it is the complete sum: no rank's terms are missing
        if b > a and n > 2:
            other = (r + 2) % n
            a2, b2 = R.chunk(other, n, length)
            if b2 > a2:
                assert not np.allclose(last["bufs"][r][a2:b2], exact[a2:b2], rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("n,length", [(2, 8), (4, 1024), (5, 1003), (8, 4096), (7, 10), (64, 64 * 3 + 7)])
def test_bytes_sent_per_rank(n, length):
    rng = np.random.default_rng(3)
    xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
    _, st = oracle.ring_allreduce(xs)
    size = [R.chunk(c, n, length)[1] - R.chunk(c, n, length)[0] for c in range(n)]
    for r in range(n):
        # each phase sends every chunk but one: reduce-scatter skips r+1, all-gather r+2
        assert st.sent[r] == 4 * (2 * length - size[(r + 1) % n] - size[(r + 2) % n])
        assert st.received[(r + 1) % n] == st.sent[r]
    assert sum(st.sent) == 2 * (n - 1) * length * 4
    if length % n == 0:
        assert all(s == 2 * (n - 1) * (length // n) * 4 for s in st.sent)


def test_summation_order_differs_from_a_pairwise_sum():
    n, length = 8, 1 << 14
    rng = np.random.default_rng(11)
    xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
    out, _ = oracle.ring_allreduce(xs)
    pairwise = np.sum(np.stack(xs), axis=0, dtype=np.float32)
    assert not np.array_equal(out[0], pairwise)
    # chunk 0 starts on rank 0, so there the ring order is the rank-order left fold
    a, b = R.chunk(0, n, length)
    acc = xs[0][a:b].copy()
    for r in range(1, n):
        acc = np.add(acc, xs[r][a:b], dtype=np.float32)
    assert np.array_equal(out[3][a:b], acc)


# --------------------------------------------------------------------------
# closed forms for exact arithmetic
# --------------------------------------------------------------------------

def test_small_integer_workload_is_the_exact_sum():
    from inputs import WORKLOADS, make_inputs

    xs = make_inputs(WORKLOADS["c1"])
    out, _ = oracle.ring_allreduce(xs)
    exact = np.sum(np.stack(xs).astype(np.int64), axis=0)
    for o in out:
        assert np.array_equal(o.astype(np.int64), exact)


@pytest.mark.parametrize("op", ["sum", "min", "max", "prod"])
def test_int32_matches_closed_forms(op):
    from inputs import WORKLOADS, make_inputs

    xs = make_inputs(WORKLOADS["c4"], count=4099)
    out, _ = oracle.ring_allreduce(xs, op=op, dtype="i32")
    st = np.stack(xs).astype(np.int64)
    if op == "sum":
        want = (np.sum(st, axis=0) % (1 << 32)).astype(np.uint32).view(np.int32)
    elif op == "min":
        want = np.min(np.stack(xs), axis=0)
    elif op == "max":
        want = np.max(np.stack(xs), axis=0)
    else:
        want = np.ones(st.shape[1], dtype=object)
        for row in st:
            want = (want * row.astype(object)) % (1 << 32)
        want = np.array([int(v) for v in want], dtype=np.uint64).astype(np.uint32).view(np.int32)
    for o in out:
        assert np.array_equal(o, want)


def test_int32_wraps():
    a = np.array([2**31 - 1, -(2**31), 65536, -1], np.int32)
    b = np.array([1, -1, 65536, -1], np.int32)
    assert R.reduce_op("sum", "i32", a, b).tolist() == [-(2**31), 2**31 - 1, 131072, -2]
    assert R.reduce_op("prod", "i32", a, b).tolist() == [2**31 - 1, -(2**31), 0, 1]


def test_float32_error_bound_against_exact_sums():
    from inputs import WORKLOADS, make_inputs

    for name, n_override in (("c2", None), ("c5", 16)):
        xs = make_inputs(WORKLOADS[name], count=2048, nranks=n_override)
        n = len(xs)
        out, _ = oracle.ring_allreduce(xs)
        for i in range(0, 2048, 7):
            col = [float(x[i]) for x in xs]
            exact = math.fsum(col)
            bound = (n - 1) * 2.0 ** -24 * math.fsum(abs(v) for v in col)
            assert abs(float(out[0][i]) - exact) <= bound


def test_ieee_min_max_special_cases():
    a = np.array([0.0, -0.0, 1.0, np.nan, 2.0, -np.inf], np.float32)
    b = np.array([-0.0, 0.0, np.nan, 1.0, 3.0, 5.0], np.float32)
    mn = R.reduce_op("min", "f32", a, b)
    mx = R.reduce_op("max", "f32", a, b)
    assert np.signbit(mn[0]) and np.signbit(mn[1])
    assert not np.signbit(mx[0]) and not np.signbit(mx[1])
    assert np.isnan(mn[2]) and np.isnan(mn[3]) and np.isnan(mx[2]) and np.isnan(mx[3])
    assert mn[4] == 2.0 and mx[4] == 3.0 and mn[5] == -np.inf and mx[5] == 5.0


def test_float_min_max_match_numpy_without_nan_or_signed_zero():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(10000).astype(np.float32)
    b = rng.standard_normal(10000).astype(np.float32)
    assert np.array_equal(R.reduce_op("min", "f32", a, b), np.minimum(a, b))
    assert np.array_equal(R.reduce_op("max", "f32", a, b), np.maximum(a, b))


# --------------------------------------------------------------------------
# bfloat16: the rounding helper against torch, the add against exact rounding
# --------------------------------------------------------------------------

def _torch_bf16_bits(f):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_ties_and_random_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(0)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)])
    f = pats.view(np.float32)
    mine = R.f32_to_bf16_bits(f)
    ref = _torch_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all(np.isnan(R.bf16_bits_to_f32(mine[nan])))
    # widening is exact: torch's bf16 -> f32 of every pattern
    import torch

    allbits = np.arange(1 << 16, dtype=np.uint16)
    tw = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    mw = R.bf16_bits_to_f32(allbits)
    ok = ~np.isnan(tw)
    assert np.array_equal(mw[ok].view(np.uint32), tw[ok].view(np.uint32))
    assert np.array_equal(np.isnan(mw), np.isnan(tw))


def _round_fraction_to_bf16(q: Fraction) -> Fraction | float:
    """Nearest bf16 value to the exact rational q, ties to even (8-bit significand)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # below the normal range the spacing stays 2^-133
    quantum = Fraction(2) ** (e - 7)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * v


def test_bf16_add_is_the_correctly_rounded_sum():
    rng = np.random.default_rng(9)
    m = 20000
    sign = rng.integers(0, 2, size=(2, m)).astype(np.uint32)
    expo = rng.integers(1, 255, size=(2, m)).astype(np.uint32)
    # bias half the pairs to nearby exponents, where rounding happens most
    expo[1, : m // 2] = np.clip(expo[0, : m // 2] + rng.integers(-9, 10, size=m // 2), 1, 254).astype(np.uint32)
    frac = rng.integers(0, 128, size=(2, m)).astype(np.uint32)
    bits = ((sign << 15) | (expo << 7) | frac).astype(np.uint16)
    got = R.reduce_op("sum", "bf16", bits[0], bits[1])
    va, vb = R.bf16_bits_to_f32(bits[0]), R.bf16_bits_to_f32(bits[1])
    gv = R.bf16_bits_to_f32(got)
    for i in range(m):
        want = _round_fraction_to_bf16(Fraction(float(va[i])) + Fraction(float(vb[i])))
        if isinstance(want, float):
            assert gv[i] == want
        else:
            assert Fraction(float(gv[i])) == want, (hex(bits[0][i]), hex(bits[1][i]))


def test_bf16_add_sign_of_zero_and_denormals():
    z, nz = np.uint16(0x0000), np.uint16(0x8000)
    one, mone = np.uint16(0x3F80), np.uint16(0xBF80)
    tiny = np.uint16(0x0001)                      # smallest bf16 denormal, 2^-133
    got = R.reduce_op("sum", "bf16", np.array([z, nz, one, tiny, tiny]), np.array([nz, nz, mone, tiny, np.uint16(0x8001)]))
    assert got.tolist() == [0x0000, 0x8000, 0x0000, 0x0002, 0x0000]


# --------------------------------------------------------------------------
# the schedule against the closed definition, and the phases against each other
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "prod"), ("f32", "min"), ("f32", "max"),
                                      ("bf16", "sum"), ("bf16", "prod"), ("bf16", "max"),
                                      ("i32", "sum"), ("i32", "prod"), ("i32", "min")])
@pytest.mark.parametrize("n,length", [(1, 5), (2, 3), (3, 2), (5, 1003), (8, 4103), (16, 31)])
def test_schedule_equals_definition(dtype, op, n, length):
    rng = np.random.default_rng(n * 1000 + length)
    if dtype == "f32":
        xs = [(rng.standard_normal(length) * 10.0 ** rng.integers(-3, 4, length)).astype(np.float32) for _ in range(n)]
    elif dtype == "bf16":
        xs = [R.f32_to_bf16_bits(rng.standard_normal(length).astype(np.float32)) for _ in range(n)]
    else:
        xs = [rng.integers(-(2**31), 2**31, size=length, dtype=np.int32) for _ in range(n)]
    out, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    want = oracle.ring_order_fold(xs, op=op, dtype=dtype)
    for o in out:
        assert R.same_bits(o, want, dtype)
    # reduce-scatter followed by all-gather is AllReduce, bit for bit
    shards, _ = oracle.reduce_scatter(xs, op=op, dtype=dtype)
    for c in range(n):                     # shard c is chunk c of the AllReduce result
        assert R.same_bits(shards[c], want[slice(*R.chunk(c, n, length))], dtype)
    again, _ = oracle.all_gather(shards, length, dtype=dtype)
    for o in again:
        assert R.same_bits(o, want, dtype)
    # and the fold at chosen positions agrees with the whole fold
    if length:
        pos = np.unique(rng.integers(0, length, size=min(length, 64)))
        cols = np.stack([np.asarray(x)[pos] for x in xs])
        got = oracle.ring_order_fold_columns(cols, R.chunk_owner(pos, n, length), op=op, dtype=dtype)
        assert R.same_bits(got, want[pos], dtype)


def test_all_gather_standalone_is_the_concatenation():
    rng = np.random.default_rng(2)
    for n, length in ((1, 4), (3, 10), (5, 1003), (8, 5), (64, 64 * 2 + 7)):
        full = rng.standard_normal(length).astype(np.float32)
        shards = [full[slice(*R.chunk(r, n, length))] for r in range(n)]
        out, st = oracle.all_gather(shards, length)
        for o in out:
            assert np.array_equal(o, full)
        size = [len(s) for s in shards]
        for r in range(n):
            assert st.sent[r] == 4 * (length - size[(r + 1) % n])   # every shard but r+1's


def test_degenerate_lengths_and_single_rank():
    out, st = oracle.ring_allreduce([np.zeros(0, np.float32)] * 4)
    assert all(o.size == 0 for o in out) and sum(st.sent) == 0
    x = np.arange(7, dtype=np.float32)
    out, st = oracle.ring_allreduce([x])
    assert np.array_equal(out[0], x) and st.rs_steps == 0 and st.ag_steps == 0
    shards, _ = oracle.reduce_scatter([x])
    assert np.array_equal(shards[0], x)
