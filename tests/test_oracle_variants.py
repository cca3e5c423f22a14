"""Pins for the oracle's precision and operator variants: IEEE binary16 buffers,
``avg`` (ring sum, then one division by N), and bf16 buffers whose partial sums
travel in float32 (``bf16acc32``)."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ring as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _round_fraction(q: Fraction, mant_bits: int, emin: int, emax: int):
    """Nearest binary floating-point value to the exact rational q, ties to even.

    mant_bits counts the significand bits including the leading one; below
    2^emin the spacing stays 2^(emin - mant_bits + 1) (subnormals); at or
    beyond the overflow threshold the result is infinite.
    """
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant_bits + 1)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * v


def _to_f32_exact(q):
    return _round_fraction(q, 24, -126, 127)


def _to_f16_exact(q):
    return _round_fraction(q, 11, -14, 15)


def _to_bf16_exact(q):
    return _round_fraction(q, 8, -126, 127)


# --------------------------------------------------------------------------
# binary16
# --------------------------------------------------------------------------

def test_f16_rounding_matches_torch_on_ties_and_random_patterns():
    import torch

    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    # f32 bits whose discarded part is 0, tiny, just under/at/over one half
    lows = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(1)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, size=3_000_000, dtype=np.uint64).astype(np.uint32)])
    f = pats.view(np.float32)
    mine = R.f32_to_f16_bits(f)
    ref = torch.from_numpy(f.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all(np.isnan(R.f16_bits_to_f32(mine[nan])))
    allbits = np.arange(1 << 16, dtype=np.uint16)
    tw = torch.from_numpy(allbits.view(np.int16)).view(torch.float16).to(torch.float32).numpy()
    mw = R.f16_bits_to_f32(allbits)
    ok = ~np.isnan(tw)
    assert np.array_equal(mw[ok].view(np.uint32), tw[ok].view(np.uint32))


def test_f16_add_is_the_correctly_rounded_sum():
    rng = np.random.default_rng(2)
    m = 20000
    sign = rng.integers(0, 2, size=(2, m)).astype(np.uint16)
    expo = rng.integers(0, 31, size=(2, m)).astype(np.uint16)          # includes subnormals (0)
    expo[1, : m // 2] = np.clip(expo[0, : m // 2].astype(int) + rng.integers(-6, 7, size=m // 2), 0, 30)
    frac = rng.integers(0, 1024, size=(2, m)).astype(np.uint16)
    bits = ((sign << 15) | (expo << 10) | frac).astype(np.uint16)
    got = R.f16_bits_to_f32(R.reduce_op("sum", "f16", bits[0], bits[1]))
    va, vb = R.f16_bits_to_f32(bits[0]), R.f16_bits_to_f32(bits[1])
    for i in range(m):
        want = _to_f16_exact(Fraction(float(va[i])) + Fraction(float(vb[i])))
        if isinstance(want, float):
            assert got[i] == want
        else:
            assert Fraction(float(got[i])) == want, (hex(bits[0][i]), hex(bits[1][i]))


def test_f16_integer_sums_are_exact():
    xs = [np.array([r + 1.0, -2.0 * r, 1000.0], np.float16).view(np.uint16) for r in range(6)]
    out, _ = oracle.ring_allreduce(xs, dtype="f16")
    assert R.f16_bits_to_f32(out[0]).tolist() == [21.0, -30.0, 6000.0]


# --------------------------------------------------------------------------
# avg
# --------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "p4_worked_examples.json")) as f:
        return json.load(f)


def test_avg_of_the_page_examples():
    g = _golden()
    xs = [np.array(r, np.float32) for r in g["allreduce_sum_3_4"]["inputs"]]
    out, _ = oracle.ring_allreduce(xs, op="avg")
    # the mean of the page's example: its sums [10, 20, 30] divided by 4 ranks
    assert all(o.tolist() == [2.5, 5.0, 7.5] for o in out)
    out, _ = oracle.ring_allreduce([np.array([r], np.float32) for r in range(4)], op="avg")
    assert all(o.tolist() == [1.5] for o in out)


@pytest.mark.parametrize("n", [3, 5, 7, 8])
def test_avg_float32_is_the_correctly_rounded_mean_of_exact_sums(n):
    rng = np.random.default_rng(n)
    length = 3001
    xs = [rng.integers(-(1 << 20), 1 << 20, size=length).astype(np.float32) for _ in range(n)]
    out, _ = oracle.ring_allreduce(xs, op="avg")
    for i in range(0, length, 13):
        exact_sum = sum(int(x[i]) for x in xs)                  # every partial is exact in float32
        want = _to_f32_exact(Fraction(exact_sum, n))
        assert Fraction(float(out[0][i])) == want


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_avg_16bit_rounds_the_quotient_once(dtype):
    n = 3
    vals = np.array([1.0, 3.0, 5.0, 7.0, 11.0, 100.0, -2.0], np.float32)
    to_bits = R.f32_to_bf16_bits if dtype == "bf16" else R.f32_to_f16_bits
    widen = R.bf16_bits_to_f32 if dtype == "bf16" else R.f16_bits_to_f32
    exact_round = _to_bf16_exact if dtype == "bf16" else _to_f16_exact
    xs = [to_bits(vals * np.float32(r + 1)) for r in range(n)]     # sums 6*vals: exact in both types
    out, _ = oracle.ring_allreduce(xs, op="avg", dtype=dtype)
    got = widen(out[0])
    for i, v in enumerate(vals):
        assert Fraction(float(got[i])) == exact_round(Fraction(float(v)) * 6 / n)


def test_avg_int32_truncates_the_wrapped_sum():
    xs = [np.array([7, -7, 2**31 - 1, 5], np.int32), np.array([1, -1, 1, -6], np.int32),
          np.array([0, 0, 0, 0], np.int32)]
    out, _ = oracle.ring_allreduce(xs, op="avg", dtype="i32")
    # sums 8, -8, 2^31 (wraps to -2^31), -1; divided by 3 toward zero
    assert out[0].tolist() == [2, -2, -(2**31) // 3 + 1, 0]


def test_avg_reduce_scatter_and_single_rank():
    xs = [np.full(8, float(r), np.float32) for r in range(4)]
    shards, _ = oracle.reduce_scatter(xs, op="avg")
    assert all(np.all(s == 1.5) for s in shards)
    out, _ = oracle.ring_allreduce([np.arange(5, dtype=np.float32)], op="avg")
    assert out[0].tolist() == [0, 1, 2, 3, 4]


# --------------------------------------------------------------------------
# bf16 with float32 partial sums
# --------------------------------------------------------------------------

def test_bf16acc32_keeps_what_per_step_rounding_loses():
    # rank 0 holds 1.0, 64 ranks hold 2^-9: bf16 has 8 significand bits, so
    # adding 2^-9 to 1.0 in bf16 is lost, while float32 partials keep every
    # term and round once: 1 + 64 * 2^-9 = 1.125, a bf16 value
    n = 65
    xs = [R.f32_to_bf16_bits(np.array([1.0 if r == 0 else 2.0 ** -9], np.float32)) for r in range(n)]
    acc, _ = oracle.ring_allreduce(xs, dtype="bf16acc32")
    step, _ = oracle.ring_allreduce(xs, dtype="bf16")
    assert R.bf16_bits_to_f32(acc[0]).tolist() == [1.125]
    assert R.bf16_bits_to_f32(step[0]).tolist() != [1.125]


@pytest.mark.parametrize("n", [4, 8, 16])
def test_bf16acc32_rounds_the_exact_sum_once(n):
    # bf16 integers: every float32 partial is exact, so the result is the exact
    # sum rounded once to bf16
    rng = np.random.default_rng(n)
    length = 2000
    xs = [R.f32_to_bf16_bits(rng.integers(-255, 256, size=length).astype(np.float32) * np.float32(64))
          for _ in range(n)]
    out, st = oracle.ring_allreduce(xs, dtype="bf16acc32")
    vals = [R.bf16_bits_to_f32(x) for x in xs]
    got = R.bf16_bits_to_f32(out[0])
    for i in range(0, length, 7):
        exact = sum(int(v[i]) for v in vals)
        assert Fraction(float(got[i])) == _to_bf16_exact(Fraction(exact))
    # partial sums travel as float32 in reduce-scatter (4 bytes), results as bf16 in all-gather (2 bytes)
    size = [R.chunk(c, n, length)[1] - R.chunk(c, n, length)[0] for c in range(n)]
    for r in range(n):
        assert st.sent[r] == 4 * (length - size[(r + 1) % n]) + 2 * (length - size[(r + 2) % n])


def test_bf16acc32_error_bound():
    # one final rounding plus the float32 accumulation error of N-1 additions
    rng = np.random.default_rng(5)
    n, length = 8, 5000
    xs = [R.f32_to_bf16_bits(rng.standard_normal(length).astype(np.float32)) for _ in range(n)]
    out, _ = oracle.ring_allreduce(xs, dtype="bf16acc32")
    vals = np.stack([R.bf16_bits_to_f32(x).astype(np.float64) for x in xs])
    exact = vals.sum(axis=0)                                   # exact: 8 bf16 terms fit in a double
    got = R.bf16_bits_to_f32(out[0]).astype(np.float64)
    half_ulp = np.maximum(np.abs(exact), 2.0 ** -126) * 2.0 ** -8
    bound = half_ulp * (1 + 2.0 ** -8) + (n - 1) * 2.0 ** -24 * np.abs(vals).sum(axis=0) * 1.01
    assert np.all(np.abs(got - exact) <= bound)


@pytest.mark.parametrize("dtype,op", [("f16", "sum"), ("f16", "max"), ("f16", "prod"), ("f16", "avg"),
                                      ("bf16acc32", "sum"), ("bf16acc32", "avg"), ("bf16acc32", "min"),
                                      ("f32", "avg"), ("bf16", "avg"), ("i32", "avg")])
@pytest.mark.parametrize("n,length", [(1, 5), (2, 3), (3, 2), (5, 1003), (8, 4103), (16, 31)])
def test_variants_schedule_equals_definition(dtype, op, n, length):
    rng = np.random.default_rng(n * 100 + length)
    if dtype == "i32":
        xs = [rng.integers(-(2**31), 2**31, size=length, dtype=np.int32) for _ in range(n)]
    elif dtype == "f32":
        xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
    elif dtype == "f16":
        xs = [R.f32_to_f16_bits(rng.standard_normal(length).astype(np.float32) * np.float32(30)) for _ in range(n)]
    else:
        xs = [R.f32_to_bf16_bits(rng.standard_normal(length).astype(np.float32)) for _ in range(n)]
    out, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    want = oracle.ring_order_fold(xs, op=op, dtype=dtype)
    for o in out:
        assert R.same_bits(o, want, dtype)
    shards, _ = oracle.reduce_scatter(xs, op=op, dtype=dtype)
    again, _ = oracle.all_gather(shards, length, dtype=dtype)
    for o in again:
        assert R.same_bits(o, want, dtype)
    if length:
        pos = np.unique(rng.integers(0, length, size=min(length, 64)))
        cols = np.stack([np.asarray(x)[pos] for x in xs])
        got = oracle.ring_order_fold_columns(cols, R.chunk_owner(pos, n, length), op=op, dtype=dtype)
        assert R.same_bits(got, want[pos], dtype)
