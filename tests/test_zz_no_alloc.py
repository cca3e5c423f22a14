"""The reduce-scatter entry point that allocates nothing (ar_reduce_scatter_noalloc).

Its results are checked against ar_reduce_scatter_ex with a caller-owned
workspace, bit for bit, on two calls in a row (the second with a smaller
input, so it runs over what the first left in the library's fixed scratch
array), and against the oracle.  Sizes whose workspace would not fit the
array are refused before anything is launched.
"""

import ctypes

import numpy as np
import pytest

import oracle
from oracle.ring import chunk, f32_to_bf16_bits, same_bits

from gpu_util import from_dev, poison, require_gpu, to_dev

pytestmark = pytest.mark.gpu

TORCH_OF = {"f32": "float32", "bf16": "bfloat16", "bf16acc32": "bfloat16", "i32": "int32"}
HOST_AS = {"f32": "f32", "bf16": "bf16", "bf16acc32": "bf16", "i32": "i32"}


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _draw(dtype, n, length, seed):
    rng = np.random.default_rng(seed)
    if dtype == "i32":
        return [rng.integers(-(2**31), 2**31, size=length, dtype=np.int32) for _ in range(n)]
    xs = [(rng.standard_normal(length) * 2.0 ** rng.integers(-8, 8, size=length)).astype(np.float32)
          for _ in range(n)]
    return [f32_to_bf16_bits(x) for x in xs] if dtype in ("bf16", "bf16acc32") else xs


def _shards(n, length, dtype):
    import torch

    return [torch.empty(chunk(c, n, length)[1] - chunk(c, n, length)[0], dtype=getattr(torch, TORCH_OF[dtype]),
                        device="cuda:0") for c in range(n)]


# (ranks, elements per rank) of the first call, then of the second, smaller one
CALLS = [(8, (1 << 20) + 13), (5, 1003)]


@pytest.mark.parametrize("algo", ["ring", "ring_pipelined", "fused"])
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "sum"), ("bf16acc32", "avg"), ("i32", "max"),
                                      ("f32", "prod")])
def test_noalloc_equals_the_workspace_call_twice_in_a_row(algo, dtype, op):
    import torch

    ar = _ar()
    for call, (n, length) in enumerate(CALLS):
        print(f"[noalloc] {algo} {dtype} {op} call {call}: {n} x {length}", flush=True)
        xs = _draw(dtype, n, length, seed=1000 * call + n)
        sends = [to_dev(x, HOST_AS[dtype]) for x in xs]
        got = _shards(n, length, dtype)
        ref = _shards(n, length, dtype)
        poison(got)
        poison(ref)
        ar.ar_reduce_scatter_noalloc(sends, got, op=op, algo=algo, dtype=dtype)
        ar.ar_reduce_scatter_ex(sends, ref, op=op, algo=algo, dtype=dtype)
        torch.cuda.synchronize()
        want, _ = oracle.reduce_scatter(xs, op=op, dtype=dtype)
        for c in range(n):
            g = got[c].view(torch.int16) if got[c].element_size() == 2 else got[c].view(torch.int32)
            r = ref[c].view(torch.int16) if ref[c].element_size() == 2 else ref[c].view(torch.int32)
            assert torch.equal(g, r), (call, c)
            assert same_bits(from_dev(got[c], HOST_AS[dtype]), want[c], dtype), (call, c)


def test_noalloc_refuses_a_workspace_beyond_its_array():
    """A float32 ring reduce-scatter one element per rank too long for the array:
    refused with AR_ERR_INVALID_ARGUMENT, the outputs left untouched."""
    import torch

    ar = _ar()
    from ring_allreduce_reduction_virtual_amd import _lib

    n = 3
    count = (_lib.NOALLOC_SCRATCH_BYTES - 1024) // 4 + 1
    assert ar.ar_workspace_bytes("reduce_scatter", "ring", count, "f32", n) > _lib.NOALLOC_SCRATCH_BYTES
    assert ar.ar_workspace_bytes("reduce_scatter", "ring", count - 1, "f32", n) <= _lib.NOALLOC_SCRATCH_BYTES
    sends = [torch.zeros(count, device="cuda:0") for _ in range(n)]
    shards = _shards(n, count, "f32")
    for t in shards:
        t.fill_(7.0)
    with pytest.raises(_lib.ArError) as e:
        ar.ar_reduce_scatter_noalloc(sends, shards, algo="ring")
    assert e.value.code == 1 and "scratch" in e.value.detail
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in shards)
    # the largest size that fits runs, and matches the fused kernel
    sends = [torch.randn(count - 1, device="cuda:0") for _ in range(n)]
    got, ref = _shards(n, count - 1, "f32"), _shards(n, count - 1, "f32")
    ar.ar_reduce_scatter_noalloc(sends, got, algo="ring")
    ar.ar_reduce_scatter_ex(sends, ref, algo="fused")
    torch.cuda.synchronize()
    for c in range(n):
        assert torch.equal(got[c].view(torch.int32), ref[c].view(torch.int32)), c


def test_noalloc_through_the_c_abi_with_a_raw_stream():
    """The C function itself, called with ctypes on a side stream's raw handle."""
    import torch

    _ar()
    from ring_allreduce_reduction_virtual_amd import _lib

    n, length = 6, 6 * 4096 + 5
    xs = _draw("f32", n, length, seed=77)
    sends = [to_dev(x, "f32") for x in xs]
    shards = _shards(n, length, "f32")
    poison(shards)
    sp = _lib.ptr_array([t.data_ptr() for t in sends])
    rp = _lib.ptr_array([t.data_ptr() for t in shards])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    rc = _lib.lib().ar_reduce_scatter_noalloc(sp, rp, length, _lib.DTYPES["f32"], _lib.OPS["sum"], n,
                                              _lib.ALGOS["ring"], ctypes.c_void_p(side.cuda_stream))
    assert rc == 0
    side.synchronize()
    want, _ = oracle.reduce_scatter(xs)
    for c in range(n):
        assert same_bits(from_dev(shards[c], "f32"), want[c], "f32"), c


@pytest.mark.parametrize("algo", ["ring", "ring_pipelined"])
def test_noalloc_replays_from_a_graph(algo):
    """What the entry point is for: captured into a HIP graph, where nothing may
    be allocated, then replayed with eager work between the replays (new
    inputs, poisoned outputs), every replay giving the oracle's bits."""
    import torch

    ar = _ar()
    n, length = 8, 8 * 4096 + 5
    xs = _draw("f32", n, length, seed=5)
    sends = [to_dev(x, "f32") for x in xs]
    got = _shards(n, length, "f32")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ar.ar_reduce_scatter_noalloc(sends, got, algo=algo)     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ar.ar_reduce_scatter_noalloc(sends, got, algo=algo)
    for rep in range(3):
        print(f"[noalloc graph] {algo} replay {rep}", flush=True)
        xs = [x + np.float32(rep + 1) * np.float32(0.5) for x in xs]
        for r in range(n):
            sends[r].copy_(to_dev(xs[r], "f32"))
        poison(got)
        g.replay()
        torch.cuda.synchronize()
        want, _ = oracle.reduce_scatter(xs)
        for c in range(n):
            assert same_bits(from_dev(got[c], "f32"), want[c], "f32"), (rep, c)
