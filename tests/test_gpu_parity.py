"""GPU parity on the five workloads and the 8 x 2^26 float32 headline workload.

Every check calls the HIP library through its C ABI (ctypes) and compares
with the CPU oracle on the same seeded inputs, bit for bit: the library folds
in the ring's association order, so float sums must match exactly, and
integer work and min/max are exact anyway.

* at sizes the oracle finishes in seconds: the whole output of every rank
  against the oracle's executed ring schedule;
* at the full sizes (the launch configurations the benchmark times): every
  element of every rank's output, for every ring-order algorithm (the
  library's default, fused, staged, phases, the ring's launches, the
  pipelined ring) against the oracle's whole result.  The oracle runs on the
  host (the executed ring schedule for the headline workload; elsewhere
  ``ring_order_fold``, which the CPU tests pin bit for bit to the executed
  schedule); its result is copied to the device once and compared there,
  and one rank's output is also copied back and compared on the host with
  the oracle's NaN rule.  Outputs are poisoned with NaN before each call, so
  an element a kernel fails to write cannot pass.  int32 results also equal
  their closed forms.
"""

import numpy as np
import pytest

import oracle
from inputs import WORKLOADS, make_inputs
from oracle.ring import chunk, chunk_owner, same_bits

from gpu_util import (assert_every_rank_equals, bits, from_dev, poison, require_gpu, tdtype, to_dev,
                      want_on_device)

pytestmark = pytest.mark.gpu


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _alloc(n, length, dtype):
    import torch

    return [torch.empty(length, dtype=tdtype(dtype), device="cuda:0") for _ in range(n)]


def _run_allreduce(xs, dtype, op, algo):
    import torch

    ar = _ar()
    sends = [to_dev(x, dtype) for x in xs]
    recvs = _alloc(len(xs), len(xs[0]), dtype)
    ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo)
    torch.cuda.synchronize()
    return sends, recvs


def _check_whole(xs, dtype, op, algo):
    want, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    _, recvs = _run_allreduce(xs, dtype, op, algo)
    for r, t in enumerate(recvs):
        assert same_bits(from_dev(t, dtype), want[r], dtype), f"rank {r}"


# --------------------------------------------------------------------------
# workloads at sizes the executed schedule finishes in seconds
# --------------------------------------------------------------------------

@pytest.mark.parametrize("algo", ["fused", "ring", "phases", "ring_pipelined", "staged"])
def test_c1_small_integers_exact(algo):
    w = WORKLOADS["c1"]
    xs = make_inputs(w)
    _check_whole(xs, "f32", "sum", algo)
    _, recvs = _run_allreduce(xs, "f32", "sum", algo)
    exact = np.sum(np.stack(xs).astype(np.int64), axis=0)
    for t in recvs:
        assert np.array_equal(from_dev(t, "f32").astype(np.int64), exact)


@pytest.mark.parametrize("algo", ["fused", "ring", "phases", "ring_pipelined", "staged"])
def test_c2_gradient_bucket(algo):
    _check_whole(make_inputs(WORKLOADS["c2"]), "f32", "sum", algo)


@pytest.mark.parametrize("algo", ["fused", "ring", "phases", "ring_pipelined", "staged"])
def test_c3_bf16_reduced_length(algo):
    _check_whole(make_inputs(WORKLOADS["c3"], count=(1 << 18) + 13), "bf16", "sum", algo)


@pytest.mark.parametrize("op", ["sum", "min", "max", "prod"])
@pytest.mark.parametrize("algo", ["fused", "ring", "phases", "ring_pipelined", "staged"])
def test_c4_int32_reduced_length(op, algo):
    _check_whole(make_inputs(WORKLOADS["c4"], count=(1 << 16) + 5), "i32", op, algo)


@pytest.mark.parametrize("algo", ["fused", "ring", "phases", "ring_pipelined", "staged"])
def test_c5_uneven_64_ranks_reduced_length(algo):
    _check_whole(make_inputs(WORKLOADS["c5"], count=64 * 1024 + 7), "f32", "sum", algo)


@pytest.mark.parametrize("algo", ["fused", "ring", "phases", "ring_pipelined"])
def test_c5_reduce_scatter_and_all_gather_reduced_length(algo):
    import torch

    ar = _ar()
    n, length = 64, 64 * 1024 + 7
    xs = make_inputs(WORKLOADS["c5"], count=length)
    shards_want, _ = oracle.reduce_scatter(xs)
    sends = [to_dev(x, "f32") for x in xs]
    shards = [torch.empty(len(s), dtype=torch.float32, device="cuda:0") for s in shards_want]
    ar.ar_reduce_scatter_ex(sends, shards, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(from_dev(shards[r], "f32"), shards_want[r], "f32"), f"shard {r}"
    # all-gather of the shards: the concatenation, and AllReduce bit for bit
    gathered_want, _ = oracle.all_gather(shards_want, length)
    outs = _alloc(n, length, "f32")
    ar.ar_all_gather_ex(shards, outs, algo=algo)
    torch.cuda.synchronize()
    allreduce_want, _ = oracle.ring_allreduce(xs)
    for r in range(n):
        got = from_dev(outs[r], "f32")
        assert same_bits(got, gathered_want[r], "f32") and same_bits(got, allreduce_want[r], "f32")


# --------------------------------------------------------------------------
# full sizes, every element
# --------------------------------------------------------------------------

RING_ORDER = ("auto", "fused", "staged", "phases", "ring", "ring_pipelined")


def _allreduce_algo(ar, sends, recvs, algo, op="sum"):
    if algo == "auto":
        ar.ar_allreduce(sends, recvs, op=op)
    else:
        ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo)


def _every_algo_every_element(sends, want_host, dtype, op, label, algos=RING_ORDER):
    """Run each algorithm into poisoned outputs and compare every element of every
    rank with the oracle's result; rank 0 of the default also on the host."""
    import torch

    ar = _ar()
    n, length = len(sends), sends[0].numel()
    want_dev = want_on_device(want_host, dtype)
    recvs = _alloc(n, length, dtype)
    for algo in algos:
        print(f"[parity] {label} {op} {algo}", flush=True)
        poison(recvs)
        _allreduce_algo(ar, sends, recvs, algo, op)
        torch.cuda.synchronize()
        assert_every_rank_equals(recvs, want_dev, f"{label} {op} {algo}")
        if algo == "auto":
            assert same_bits(from_dev(recvs[0], dtype), want_host, dtype), f"{label} {op}: rank 0 on the host"
    del recvs
    return want_dev


def test_headline_8_ranks_2p26_float32_full_size_every_element():
    """The benchmark's workload: the oracle's executed ring schedule on the whole
    2 GiB of inputs, against every element of every algorithm's output, then in
    place over the inputs (the fused kernel here reads with nontemporal loads)."""
    import torch

    ar = _ar()
    w = WORKLOADS["headline"]
    xs = make_inputs(w)
    want, _ = oracle.ring_allreduce(xs)          # every rank the same bits (checked inside)
    sends = [to_dev(x, "f32") for x in xs]
    want_dev = _every_algo_every_element(sends, want[0], "f32", "sum", "headline")
    ar.ar_allreduce(sends)
    torch.cuda.synchronize()
    assert_every_rank_equals(sends, want_dev, "headline in place")


# The fused AllReduce reads inputs of up to 256 MiB in total (N * S) with
# cache-allocating loads and larger ones with nontemporal loads.
CACHED_LOADS_MAX_BYTES = 256 << 20


@pytest.mark.parametrize("count", [CACHED_LOADS_MAX_BYTES // 32, CACHED_LOADS_MAX_BYTES // 32 + 4])
def test_fused_loads_either_side_of_the_cache_bound(count):
    """8 ranks of float32 at exactly 256 MiB of inputs and just above: both load
    forms give the oracle's bits everywhere, call after call."""
    import torch

    ar = _ar()
    xs = make_inputs(WORKLOADS["c2"], count=count)
    want_dev = want_on_device(oracle.ring_order_fold(xs), "f32")
    sends = [to_dev(x, "f32") for x in xs]
    recvs = _alloc(len(xs), count, "f32")
    for call in range(3):                  # again, with the inputs now possibly cached
        poison(recvs)
        ar.ar_allreduce_ex(sends, recvs, algo="fused")
        torch.cuda.synchronize()
        assert_every_rank_equals(recvs, want_dev, f"call {call}")


def test_c3_bf16_full_size_every_element():
    w = WORKLOADS["c3"]
    xs = make_inputs(w)
    want = oracle.ring_order_fold(xs, "sum", "bf16")
    sends = [to_dev(x, "bf16") for x in xs]
    _every_algo_every_element(sends, want, "bf16", "sum", "c3")


@pytest.mark.parametrize("op", ["sum", "min", "max"])
def test_c4_int32_full_size_closed_forms_every_element(op):
    w = WORKLOADS["c4"]
    xs = make_inputs(w)
    st = np.stack(xs)
    if op == "sum":
        want = np.zeros(w.count, np.uint32)
        for x in xs:
            np.add(want, x.view(np.uint32), out=want)      # wrapping sum: any order gives these bits
        want = want.view(np.int32)
    elif op == "min":
        want = st.min(axis=0)
    else:
        want = st.max(axis=0)
    # the closed form is the ring's result too (order plays no part in these operators)
    assert np.array_equal(oracle.ring_order_fold(xs, op, "i32"), want)
    sends = [to_dev(x, "i32") for x in xs]
    _every_algo_every_element(sends, want, "i32", op, "c4")


@pytest.fixture(scope="module")
def c5_data():
    """The 64-rank workload's inputs (16 GiB on the host) and the oracle's AllReduce result."""
    w = WORKLOADS["c5"]
    xs = make_inputs(w)
    return w, xs, oracle.ring_order_fold(xs)


def test_c5_full_size_allreduce_every_element(c5_data):
    w, xs, want = c5_data
    sends = [to_dev(x, "f32") for x in xs]
    _every_algo_every_element(sends, want, "f32", "sum", "c5")


def test_c5_full_size_reduce_scatter_every_element(c5_data):
    """Shard c of the reduce-scatter is chunk c of the oracle's AllReduce result
    (the CPU tests pin the oracle's reduce-scatter to exactly that)."""
    import torch

    ar = _ar()
    w, xs, want = c5_data
    n, length = w.nranks, w.count
    sends = [to_dev(x, "f32") for x in xs]
    shards = []
    for c in range(n):
        s, e = chunk(c, n, length)
        shards.append(torch.empty(e - s, dtype=torch.float32, device="cuda:0"))
    wants = [want_on_device(want[slice(*chunk(c, n, length))], "f32") for c in range(n)]
    for algo in ("auto", "fused", "ring", "ring_pipelined"):
        print(f"[parity] c5 reduce-scatter {algo}", flush=True)
        poison(shards)
        if algo == "auto":
            ar.ar_reduce_scatter(sends, shards)
        else:
            ar.ar_reduce_scatter_ex(sends, shards, algo=algo)
        torch.cuda.synchronize()
        for c in range(n):
            assert torch.equal(bits(shards[c]), bits(wants[c])), (algo, c)
    host = np.concatenate([from_dev(t, "f32") for t in shards])
    assert same_bits(host, want, "f32")


def test_c5_full_size_all_gather_every_element(c5_data):
    """All-gather of seeded shards (rank c holds chunk c of its own input): every
    rank receives their concatenation, which is what the oracle's all-gather
    gives (pinned on the CPU)."""
    import torch

    ar = _ar()
    w, xs, _ = c5_data
    n, length = w.nranks, w.count
    shards_host = [xs[c][slice(*chunk(c, n, length))] for c in range(n)]
    want = np.concatenate(shards_host)
    want_dev = want_on_device(want, "f32")
    shards = [to_dev(s, "f32") for s in shards_host]
    outs = _alloc(n, length, "f32")
    for algo in ("auto", "fused", "ring", "ring_pipelined"):
        print(f"[parity] c5 all-gather {algo}", flush=True)
        poison(outs)
        if algo == "auto":
            ar.ar_all_gather(shards, outs)
        else:
            ar.ar_all_gather_ex(shards, outs, algo=algo)
        torch.cuda.synchronize()
        assert_every_rank_equals(outs, want_dev, f"c5 all-gather {algo}")
    assert same_bits(from_dev(outs[n - 1], "f32"), want, "f32")
