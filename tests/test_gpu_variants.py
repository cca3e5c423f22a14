"""GPU parity for the precision and operator variants: IEEE binary16 buffers,
``avg``, and bf16 buffers whose partial sums are kept in float32
(``bf16acc32``), with every algorithm, against the oracle bit for bit."""

import zlib

import numpy as np
import pytest

import oracle
from oracle.ring import chunk, f32_to_bf16_bits, f32_to_f16_bits, same_bits

from gpu_util import from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

TORCH_OF = {"f16": "float16", "bf16acc32": "bfloat16", "bf16": "bfloat16", "f32": "float32", "i32": "int32"}
STORE_AS = {"bf16acc32": "bf16"}          # how the buffers are moved to and from the device


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _draw(dtype, n, length, seed, special=False):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(n):
        if dtype == "i32":
            xs.append(rng.integers(-(2**31), 2**31, size=length, dtype=np.int32))
            continue
        f = (rng.standard_normal(length) * 2.0 ** rng.integers(-12, 12, size=length)).astype(np.float32)
        if special and length:
            sp = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 6.0e-8, -3.0e-5, 65504.0, 70000.0, 1e-40, 3e38],
                          np.float32)
            where = rng.integers(0, length, size=max(1, length // 5))
            f[where] = sp[rng.integers(0, len(sp), size=len(where))]
        if dtype == "f16":
            xs.append(f32_to_f16_bits(f))
        elif dtype in ("bf16", "bf16acc32"):
            xs.append(f32_to_bf16_bits(f))
        else:
            xs.append(f)
    return xs


def _dev(x, dtype):
    import torch

    if dtype in ("f16", "bf16", "bf16acc32"):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0").view(getattr(torch, TORCH_OF[dtype]))
    return to_dev(x, dtype)


def _host(t, dtype):
    import torch

    if dtype in ("f16", "bf16", "bf16acc32"):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return from_dev(t, dtype)


def _empty(n, length, dtype):
    import torch

    return [torch.empty(length, dtype=getattr(torch, TORCH_OF[dtype]), device="cuda:0") for _ in range(n)]


CASES = [(d, o) for d in ("f16", "bf16acc32") for o in ("sum", "prod", "min", "max", "avg")] + \
        [("f32", "avg"), ("bf16", "avg"), ("i32", "avg")]


@pytest.mark.parametrize("algo", ["fused", "phases", "ring", "ring_pipelined", "staged"])
@pytest.mark.parametrize("dtype,op", CASES)
@pytest.mark.parametrize("n,length", [(1, 9), (2, 1001), (3, 7), (5, 1003), (8, 8 * 512 + 13), (17, 4099)])
def test_allreduce_variants(n, length, dtype, op, algo):
    import torch

    ar = _ar()
    xs = _draw(dtype, n, length, seed=zlib.crc32(f"{dtype}{op}{n}".encode()))
    want, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    sends = [_dev(x, dtype) for x in xs]
    recvs = _empty(n, length, dtype)
    ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), f"rank {r}"


@pytest.mark.parametrize("algo", ["fused", "ring", "ring_pipelined"])
@pytest.mark.parametrize("dtype,op", [("f16", "sum"), ("f16", "avg"), ("bf16acc32", "sum"), ("bf16acc32", "avg"),
                                      ("bf16acc32", "max"), ("i32", "avg")])
@pytest.mark.parametrize("n,length", [(2, 33), (4, 4), (5, 1003), (64, 64 * 9 + 5)])
def test_reduce_scatter_and_all_gather_variants(n, length, dtype, op, algo):
    import torch

    ar = _ar()
    xs = _draw(dtype, n, length, seed=n * 31 + length)
    shards_want, _ = oracle.reduce_scatter(xs, op=op, dtype=dtype)
    sends = [_dev(x, dtype) for x in xs]
    tdt = getattr(torch, TORCH_OF[dtype])
    shards = [torch.empty(len(s), dtype=tdt, device="cuda:0") for s in shards_want]
    ar.ar_reduce_scatter_ex(sends, shards, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(shards[r], dtype), shards_want[r], dtype), f"shard {r}"
    outs = _empty(n, length, dtype)
    ar.ar_all_gather_ex(shards, outs, algo=algo)
    torch.cuda.synchronize()
    want, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    for r in range(n):
        assert same_bits(_host(outs[r], dtype), want[r], dtype), f"rank {r}"


@pytest.mark.parametrize("algo", ["fused", "phases", "ring", "ring_pipelined", "staged"])
@pytest.mark.parametrize("dtype,op", [("f16", "sum"), ("f16", "prod"), ("f16", "min"), ("f16", "avg"),
                                      ("bf16acc32", "sum"), ("bf16acc32", "avg"), ("f32", "avg")])
def test_special_values_variants(dtype, op, algo):
    import torch

    ar = _ar()
    n, length = 6, 3001
    xs = _draw(dtype, n, length, seed=17, special=True)
    want, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    sends = [_dev(x, dtype) for x in xs]
    recvs = _empty(n, length, dtype)
    ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), f"rank {r}"


@pytest.mark.parametrize("algo", ["fused", "phases", "ring", "ring_pipelined", "staged"])
@pytest.mark.parametrize("layout", ["in_place", "common_offset", "mixed_offsets"])
def test_bf16acc32_layouts(layout, algo):
    """Float32 partials with in-place buffers and views 1..3 elements into allocations."""
    import torch

    ar = _ar()
    n, length = 5, 4096 + 11
    dtype = "bf16acc32"
    xs = _draw(dtype, n, length, seed=23)
    want, _ = oracle.ring_allreduce(xs, op="sum", dtype=dtype)
    if layout == "in_place":
        sends = [_dev(x, dtype) for x in xs]
        recvs = sends
    else:
        sends, recvs = [], []
        for r in range(n):
            off = 1 if layout == "common_offset" else r % 4
            base = torch.empty(length + 8, dtype=torch.bfloat16, device="cuda:0")
            v = base[off:off + length]
            v.copy_(_dev(xs[r], dtype))
            sends.append(v)
            off2 = 1 if layout == "common_offset" else (r + 1) % 3
            rb = torch.empty(length + 8, dtype=torch.bfloat16, device="cuda:0")
            recvs.append(rb[off2:off2 + length])
    ar.ar_allreduce_ex(sends, recvs, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), f"rank {r}"


def test_c3_workload_full_size_with_float32_partials_and_avg():
    """8 x 2^26 bf16 (the c3 workload) with float32 partials, and its average:
    every element of every rank, for the default and every ring-order algorithm."""
    import torch

    from gpu_util import assert_every_rank_equals, poison, want_on_device
    from inputs import WORKLOADS, make_inputs

    ar = _ar()
    w = WORKLOADS["c3"]
    xs = make_inputs(w)
    sends = [_dev(x, "bf16") for x in xs]
    recvs = _empty(w.nranks, w.count, "bf16")
    for dtype, op in (("bf16acc32", "sum"), ("bf16acc32", "avg"), ("bf16", "avg")):
        want = want_on_device(oracle.ring_order_fold(xs, op=op, dtype=dtype), dtype)
        for algo in ("auto", "fused", "ring", "ring_pipelined", "staged", "phases"):
            print(f"[full size] c3 {dtype} {op} {algo}", flush=True)
            poison(recvs)
            if algo == "auto":
                ar.ar_allreduce(sends, recvs, op=op, dtype=dtype)
            else:
                ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
            torch.cuda.synchronize()
            assert_every_rank_equals(recvs, want, f"{dtype} {op} {algo}")
