"""GPU parity on the five workloads and the 8 x 2^26 float32 headline workload.

Every check calls the HIP library through its C ABI (ctypes) and compares
with the CPU oracle on the same seeded inputs, bit for bit: the library folds
in the ring's association order, so float sums must match exactly, and
integer work and min/max are exact anyway.

* at sizes the oracle finishes in seconds: the whole output of every rank
  against the oracle's executed ring schedule;
* at the full sizes (launch configuration as in the benchmark): sampled
  positions against the oracle's fold at those positions (random positions
  plus every chunk's edges), and properties that hold at any size: all ranks
  bit-identical, every ring-order algorithm (fused, phases, the ring's
  launches, the pipelined ring, the staged reduce-then-broadcast) bit for
  bit equal to the fused result, int32
  results equal to their closed forms.
"""

import numpy as np
import pytest

import oracle
from inputs import WORKLOADS, make_inputs
from oracle.ring import chunk, chunk_owner, same_bits

from gpu_util import bits, from_dev, require_gpu, sample_positions, tdtype, to_dev

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
# full sizes, sampled
# --------------------------------------------------------------------------

def _sampled_check(xs, recvs, dtype, op, seed):
    import torch

    n, length = len(xs), len(xs[0])
    pos = sample_positions(length, n, seed)
    cols = np.stack([x[pos] for x in xs])
    want = oracle.ring_order_fold_columns(cols, chunk_owner(pos, n, length), op=op, dtype=dtype)
    idx = torch.from_numpy(pos).to("cuda:0")
    for r, t in enumerate(recvs):
        got = from_dev(t[idx], dtype)
        assert same_bits(got, want, dtype), f"rank {r}"
    ref = bits(recvs[0])
    for r in range(1, n):
        assert torch.equal(bits(recvs[r]), ref), f"rank {r} differs from rank 0"


def test_headline_8_ranks_2p26_float32_full_size():
    import torch

    ar = _ar()
    w = WORKLOADS["headline"]
    xs = make_inputs(w)
    sends, fused = _run_allreduce(xs, "f32", "sum", "fused")
    _sampled_check(xs, fused, "f32", "sum", seed=101)
    for algo in ("ring", "phases", "staged"):
        other = _alloc(w.nranks, w.count, "f32")
        ar.ar_allreduce_ex(sends, other, algo=algo)
        torch.cuda.synchronize()
        for r in range(w.nranks):
            assert torch.equal(bits(other[r]), bits(fused[0])), (algo, r)
        del other
    # in place over the inputs gives the same bits
    ar.ar_allreduce(sends)
    torch.cuda.synchronize()
    for t in sends:
        assert torch.equal(bits(t), bits(fused[0]))


# The fused AllReduce reads inputs of up to 256 MiB in total (N * S) with
# cache-allocating loads and larger ones with nontemporal loads.
CACHED_LOADS_MAX_BYTES = 256 << 20


@pytest.mark.parametrize("count", [CACHED_LOADS_MAX_BYTES // 32, CACHED_LOADS_MAX_BYTES // 32 + 4])
def test_fused_loads_either_side_of_the_cache_bound(count):
    """8 ranks of float32 at exactly 256 MiB of inputs and just above: both load
    forms give the oracle's bits at the sampled positions, call after call."""
    import torch

    ar = _ar()
    xs = make_inputs(WORKLOADS["c2"], count=count)
    sends, recvs = _run_allreduce(xs, "f32", "sum", "fused")
    _sampled_check(xs, recvs, "f32", "sum", seed=105)
    first = bits(recvs[0]).clone()
    for t in recvs:
        t.fill_(-1.0)
    for _ in range(2):                     # again, with the inputs now possibly cached
        ar.ar_allreduce_ex(sends, recvs, algo="fused")
    torch.cuda.synchronize()
    for r in range(len(recvs)):
        assert torch.equal(bits(recvs[r]), first), f"rank {r}"


def _same_as(reference, sends, dtype, op, algos):
    """Each algorithm's AllReduce of `sends`, bit for bit equal to `reference` on every rank."""
    import torch

    ar = _ar()
    for algo in algos:
        other = _alloc(len(sends), sends[0].numel(), dtype)
        ar.ar_allreduce_ex(sends, other, op=op, algo=algo)
        torch.cuda.synchronize()
        for r in range(len(sends)):
            assert torch.equal(bits(other[r]), bits(reference[0])), (algo, r)
        del other


def test_c3_bf16_full_size():
    w = WORKLOADS["c3"]
    xs = make_inputs(w)
    sends, recvs = _run_allreduce(xs, "bf16", "sum", "fused")
    _sampled_check(xs, recvs, "bf16", "sum", seed=102)
    _same_as(recvs, sends, "bf16", "sum", ("ring", "ring_pipelined", "staged"))


@pytest.mark.parametrize("op", ["sum", "min", "max"])
def test_c4_int32_full_size_closed_forms(op):
    import torch

    w = WORKLOADS["c4"]
    xs = make_inputs(w)
    sends, recvs = _run_allreduce(xs, "i32", op, "fused")
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
    got = from_dev(recvs[0], "i32")
    assert np.array_equal(got, want)
    for r in range(1, w.nranks):
        assert torch.equal(recvs[r], recvs[0])
    _sampled_check(xs, recvs, "i32", op, seed=103)
    _same_as(recvs, sends, "i32", op, ("ring", "ring_pipelined", "staged"))


def test_c5_full_size_allreduce_reduce_scatter_all_gather():
    import torch

    ar = _ar()
    w = WORKLOADS["c5"]
    n, length = w.nranks, w.count
    xs = make_inputs(w)
    sends = [to_dev(x, "f32") for x in xs]
    recvs = _alloc(n, length, "f32")
    ar.ar_allreduce(sends, recvs)          # 64 ranks x 256 MiB: the default runs the staged form
    torch.cuda.synchronize()
    _sampled_check(xs, recvs, "f32", "sum", seed=104)
    one_pass = _alloc(n, length, "f32")
    ar.ar_allreduce_ex(sends, one_pass, algo="fused")
    torch.cuda.synchronize()
    for r in range(n):
        assert torch.equal(bits(one_pass[r]), bits(recvs[0])), f"one-pass rank {r}"
    del one_pass
    _same_as(recvs, sends, "f32", "sum", ("ring", "ring_pipelined", "phases"))
    # reduce-scatter: shard c equals chunk c of the AllReduce, bit for bit
    shards = []
    for c in range(n):
        s, e = chunk(c, n, length)
        shards.append(torch.empty(e - s, dtype=torch.float32, device="cuda:0"))
    ar.ar_reduce_scatter(sends, shards)
    torch.cuda.synchronize()
    for c in range(n):
        s, e = chunk(c, n, length)
        assert torch.equal(bits(shards[c]), bits(recvs[0][s:e])), f"shard {c}"
    for algo in ("ring", "ring_pipelined"):
        other = [torch.empty_like(t) for t in shards]
        ar.ar_reduce_scatter_ex(sends, other, algo=algo)
        torch.cuda.synchronize()
        for c in range(n):
            assert torch.equal(bits(other[c]), bits(shards[c])), (algo, c)
        del other
    del sends
    # all-gather of those shards reproduces the AllReduce on every rank
    outs = recvs          # overwrite the AllReduce outputs after keeping one copy
    keep = recvs[0].clone()
    for t in outs:
        t.zero_()
    ar.ar_all_gather(shards, outs)
    torch.cuda.synchronize()
    for r in range(n):
        assert torch.equal(bits(outs[r]), bits(keep)), f"rank {r}"
    for algo in ("ring", "ring_pipelined"):
        for t in outs:
            t.zero_()
        ar.ar_all_gather_ex(shards, outs, algo=algo)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(bits(outs[r]), bits(keep)), (algo, r)
