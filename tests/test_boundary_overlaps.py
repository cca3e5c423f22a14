"""The host's aliasing rules, checked against their statement on random layouts.

include/ar.h allows exactly these overlaps: send buffers among themselves
(read only), and one in-place layout per collective (AllReduce: recv[r] ==
send[r]; reduce-scatter: recv[r] == send[r] + start(r) elements; all-gather:
send[r] == recv[r] + start(r) elements).  Any other overlap is an
AR_ERR_INVALID_ARGUMENT.  Hypothesis draws layouts of fake, element-aligned
device addresses crowded into a small window so that overlaps are common; the
library's verdict is compared with the rule written out below.  A layout that
passes validation goes on to the launch, which fails without a GPU
(AR_ERR_HIP), so no device memory is ever touched.
"""

import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.ring import chunk

BASE = 0x7F0000000000
ESZ = 4            # float32


@pytest.fixture(scope="module")
def lib():
    import os

    from ring_allreduce_reduction_virtual_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return _lib.lib()


def _ptrs(vals):
    arr = (ctypes.c_void_p * len(vals))()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


def _expected_valid(coll, sends, recvs, count, n):
    ivs = []
    for r in range(n):
        a, b = chunk(r, n, count)
        slen = (b - a) if coll == "all_gather" else count
        rlen = (b - a) if coll == "reduce_scatter" else count
        if slen:
            ivs.append(("send", r, sends[r], sends[r] + ESZ * slen))
        if rlen:
            ivs.append(("recv", r, recvs[r], recvs[r] + ESZ * rlen))
    for i in range(len(ivs)):
        for j in range(i + 1, len(ivs)):
            x, y = ivs[i], ivs[j]
            if not (x[2] < y[3] and y[2] < x[3]):
                continue
            if x[0] == "send" and y[0] == "send":
                continue
            if x[0] == y[0]:
                return False                      # two receive buffers overlap
            s, d = (x, y) if x[0] == "send" else (y, x)
            if s[1] != d[1]:
                return False                      # another rank's buffer
            start = chunk(s[1], n, count)[0] * ESZ
            if coll == "allreduce" and d[2] == s[2]:
                continue
            if coll == "reduce_scatter" and d[2] == s[2] + start:
                continue
            if coll == "all_gather" and s[2] == d[2] + start:
                continue
            return False
    return True


@st.composite
def layouts(draw):
    coll = draw(st.sampled_from(["allreduce", "reduce_scatter", "all_gather"]))
    n = draw(st.integers(1, 6))
    count = draw(st.integers(1, 40))
    window = 6 * count                                 # elements: crowded, so overlaps are common
    slot = st.integers(0, window)
    sends, recvs = [], []
    for r in range(n):
        start = chunk(r, n, count)[0]
        kind = draw(st.sampled_from(["free", "free", "in_place", "shifted"]))
        s = BASE + ESZ * draw(slot)
        if kind == "free":
            d = BASE + ESZ * draw(slot)
        elif kind == "in_place":
            d = {"allreduce": s, "reduce_scatter": s + ESZ * start, "all_gather": s - ESZ * start}[coll]
        else:
            d = s + ESZ * draw(st.integers(-3, 3))
        if coll == "all_gather" and kind == "in_place":
            s, d = d + ESZ * start, d                  # send[r] is the shard inside recv[r]
        sends.append(s)
        recvs.append(d)
    return coll, n, count, sends, recvs


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts())
def test_overlap_rules_match_their_statement(lib, layout):
    coll, n, count, sends, recvs = layout
    if coll == "allreduce":
        rc = lib.ar_allreduce(_ptrs(sends), _ptrs(recvs), count, 0, 0, n, None)
    elif coll == "reduce_scatter":
        rc = lib.ar_reduce_scatter(_ptrs(sends), _ptrs(recvs), count, 0, 0, n, None)
    else:
        rc = lib.ar_all_gather(_ptrs(sends), _ptrs(recvs), count, 0, n, None)
    valid = _expected_valid(coll, sends, recvs, count, n)
    detail = lib.ar_get_last_error_detail()
    if valid:
        assert rc in (0, 3), (coll, n, count, rc, detail)          # passed validation, then no device
        if rc == 3:
            assert b"overlaps" not in detail
    else:
        assert rc == 1 and b"overlaps" in detail, (coll, n, count, rc, detail)
