"""GPU parity for the tree-shaped AllReduce orders: the binomial tree (fused and
staged), recursive doubling, recursive halving/doubling (fused and staged) and
the double binary tree (fused and level by level), against the oracle's
schedules (oracle/orders.py, oracle/dbt.py) bit for bit, over every
dtype and operator, in-place and offset layouts, special values, persistent
plans and HIP graph replays, and every element at the full workload sizes."""

import zlib

import numpy as np
import pytest

from oracle import dbt
from oracle.orders import order_allreduce as _order_allreduce
from oracle.orders import order_bracketing, tree_order_fold
from oracle.ring import f32_to_bf16_bits, f32_to_f16_bits, ring_order_fold, same_bits

from gpu_util import assert_every_rank_equals, from_dev, poison, require_gpu, to_dev, want_on_device

pytestmark = pytest.mark.gpu

ORDER_OF = {"tree": "tree", "tree_steps": "tree", "recursive_doubling": "recursive_doubling",
            "halving_doubling": "halving_doubling", "halving_doubling_steps": "halving_doubling",
            "double_binary_tree": "double_binary_tree", "double_binary_tree_steps": "double_binary_tree"}
POW2 = ("recursive_doubling", "halving_doubling", "halving_doubling_steps")
TORCH_OF = {"f16": "float16", "bf16acc32": "bfloat16", "bf16": "bfloat16", "f32": "float32", "i32": "int32"}


def order_allreduce(order, xs, op="sum", dtype="f32"):
    """The oracle's executed schedule of an order: (outputs, stats)."""
    if order == "double_binary_tree":
        return dbt.double_binary_tree_allreduce(xs, op, dtype)
    return _order_allreduce(order, xs, op, dtype)


def order_fold(order, xs, op="sum", dtype="f32"):
    """The order's result as a definition: its bracketing evaluated on the whole buffers."""
    if order == "double_binary_tree":
        return dbt.double_binary_tree_fold(xs, op, dtype)
    return tree_order_fold(xs, order_bracketing(order, len(xs)), op, dtype)


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

    return [torch.full((length,), 0x5A, dtype=getattr(torch, TORCH_OF[dtype]), device="cuda:0") for _ in range(n)]


CASES = [("f32", "sum"), ("f32", "prod"), ("f32", "min"), ("f32", "max"), ("f32", "avg"), ("bf16", "sum"),
         ("bf16", "max"), ("f16", "sum"), ("f16", "avg"), ("i32", "sum"), ("i32", "max"), ("i32", "avg"),
         ("bf16acc32", "sum"), ("bf16acc32", "avg")]
SHAPES = [(1, 9), (2, 1001), (3, 7), (4, 4), (5, 1003), (8, 8 * 4096 + 13), (16, 16 * 700 + 9), (17, 4099),
          (64, 64 * 300 + 5)]


# every (algorithm, shape) pair the library accepts: the power-of-two schedules
# only at power-of-two rank counts (their refusal elsewhere is a host test)
VALID = [(algo, n, length) for algo in ORDER_OF for n, length in SHAPES if algo not in POW2 or not n & (n - 1)]


@pytest.mark.parametrize("dtype,op", CASES)
@pytest.mark.parametrize("algo,n,length", VALID)
def test_tree_orders_match_the_oracle(algo, n, length, dtype, op):
    import torch

    ar = _ar()
    xs = _draw(dtype, n, length, seed=zlib.crc32(f"{dtype}{op}{n}{length}".encode()))
    want, _ = order_allreduce(ORDER_OF[algo], xs, op, dtype)
    sends = [_dev(x, dtype) for x in xs]
    recvs = _empty(n, length, dtype)
    ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), f"rank {r}"


@pytest.mark.parametrize("algo", list(ORDER_OF))
def test_tree_orders_are_not_the_ring(algo):
    """On spread inputs the tree orders give other bits than the ring (and the oracle says which)."""
    import torch

    ar = _ar()
    n, length = 8, 8 * 1024
    xs = _draw("f32", n, length, seed=99)
    sends = [_dev(x, "f32") for x in xs]
    recvs = _empty(n, length, "f32")
    ar.ar_allreduce_ex(sends, recvs, algo=algo)
    torch.cuda.synchronize()
    got = _host(recvs[0], "f32")
    assert not same_bits(got, ring_order_fold(xs), "f32")
    assert same_bits(got, order_allreduce(ORDER_OF[algo], xs)[0][0], "f32")


@pytest.mark.parametrize("algo", list(ORDER_OF))
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "min"), ("f32", "prod"), ("f16", "sum"),
                                      ("f16", "avg"), ("bf16acc32", "sum")])
def test_tree_orders_special_values(dtype, op, algo):
    import torch

    ar = _ar()
    n, length = 8, 3001
    xs = _draw(dtype, n, length, seed=17, special=True)
    want, _ = order_allreduce(ORDER_OF[algo], xs, op, dtype)
    sends = [_dev(x, dtype) for x in xs]
    recvs = _empty(n, length, dtype)
    ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), f"rank {r}"


@pytest.mark.parametrize("algo", list(ORDER_OF))
@pytest.mark.parametrize("dtype", ["f32", "bf16acc32"])
@pytest.mark.parametrize("layout", ["in_place", "common_offset", "mixed_offsets"])
def test_tree_orders_layouts(layout, dtype, algo):
    """In place, views one element into their allocations (vector path at a residue),
    and views at different residues (element path)."""
    import torch

    ar = _ar()
    n, length = 8, 8 * 2048 + 11
    xs = _draw(dtype, n, length, seed=23)
    want, _ = order_allreduce(ORDER_OF[algo], xs, "sum", dtype)
    tdt = getattr(torch, TORCH_OF[dtype])
    if layout == "in_place":
        sends = [_dev(x, dtype) for x in xs]
        recvs = sends
    else:
        sends, recvs = [], []
        for r in range(n):
            off = 1 if layout == "common_offset" else r % 4
            base = torch.empty(length + 8, dtype=tdt, device="cuda:0")
            v = base[off:off + length]
            v.copy_(_dev(xs[r], dtype))
            sends.append(v)
            off2 = 1 if layout == "common_offset" else (r + 1) % 3
            rb = torch.empty(length + 8, dtype=tdt, device="cuda:0")
            recvs.append(rb[off2:off2 + length])
    ar.ar_allreduce_ex(sends, recvs, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), f"rank {r}"


LAUNCHES = {"tree": lambda n: 1, "halving_doubling": lambda n: 1, "double_binary_tree": lambda n: 1,
            "tree_steps": lambda n: 2 * (n - 1).bit_length(), "recursive_doubling": lambda n: (n - 1).bit_length(),
            "halving_doubling_steps": lambda n: 2 * (n - 1).bit_length(),
            "double_binary_tree_steps": lambda n: 2 * (n.bit_length() - 1)}


@pytest.mark.parametrize("n,algo", [(n, algo) for n in (4, 8, 13, 16) for algo in ORDER_OF
                                    if algo not in POW2 or not n & (n - 1)])
def test_tree_order_plans_and_launch_counts(n, algo):
    """Stage counts of the pages' cost statements: 2 ceil(log2 N) for the tree and for
    halving/doubling, log2 N for recursive doubling, 2 floor(log2 N) for the double
    binary tree; one launch for the fused forms."""
    import torch

    ar = _ar()
    length = n * 1000 + 3
    xs = _draw("bf16acc32", n, length, seed=n)
    sends = [_dev(x, "bf16acc32") for x in xs]
    recvs = _empty(n, length, "bf16acc32")
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo, dtype="bf16acc32")
    assert plan.num_launches == LAUNCHES[algo](n)
    for rep in range(2):
        want, _ = order_allreduce(ORDER_OF[algo], xs, "sum", "bf16acc32")
        plan.start()
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(recvs[r], "bf16acc32"), want[r], "bf16acc32"), (rep, r)
        xs = [f32_to_bf16_bits(np.float32(0.5) * ((x.astype(np.uint32) << 16).view(np.float32))) for x in xs]
        for r in range(n):
            sends[r].copy_(_dev(xs[r], "bf16acc32"))
    plan.close()


@pytest.mark.parametrize("algo", ["tree_steps", "recursive_doubling", "halving_doubling_steps",
                                  "double_binary_tree_steps"])
def test_tree_order_graph_replays(algo):
    """Staged schedules captured in a HIP graph: 4 replays with eager input changes between."""
    import torch

    ar = _ar()
    n, length = 8, 8 * 2048 + 3
    xs = _draw("f32", n, length, seed=11)
    sends = [_dev(x, "f32") for x in xs]
    recvs = _empty(n, length, "f32")
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.start(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(2):
            plan.start()
    for rep in range(4):
        xs = [x + np.float32(rep + 1) * np.float32(0.25) for x in xs]
        for r in range(n):
            sends[r].copy_(_dev(xs[r], "f32"))
        for r in range(n):
            recvs[r].fill_(-7.0)
        g.replay()
        torch.cuda.synchronize()
        want, _ = order_allreduce(ORDER_OF[algo], xs)
        for r in range(n):
            assert same_bits(_host(recvs[r], "f32"), want[r], "f32"), (rep, r)


@pytest.mark.parametrize("workload,algos", [
    ("headline", ["tree", "halving_doubling", "tree_steps", "recursive_doubling", "halving_doubling_steps",
                  "double_binary_tree", "double_binary_tree_steps"]),
    ("c5", ["tree", "halving_doubling", "double_binary_tree", "double_binary_tree_steps"]),
    ("c3", ["tree", "halving_doubling_steps", "double_binary_tree"]),
    ("c4", ["double_binary_tree_steps"]),
])
def test_tree_orders_full_size_every_element(workload, algos):
    """The full workloads: every element of every rank against the order's
    bracketing evaluated over the whole buffers on the host."""
    import torch

    from inputs import WORKLOADS, make_inputs

    ar = _ar()
    w = WORKLOADS[workload]
    dtype = w.dtype
    xs = make_inputs(w)
    sends = [_dev(x, dtype) for x in xs]
    recvs = _empty(w.nranks, w.count, dtype)
    wants = {}
    for algo in algos:
        print(f"[full size] {workload} {algo}", flush=True)
        order = ORDER_OF[algo]
        if order not in wants:
            wants[order] = want_on_device(order_fold(order, xs, "sum", dtype), dtype)
        poison(recvs)
        ar.ar_allreduce_ex(sends, recvs, algo=algo, dtype=dtype)
        torch.cuda.synchronize()
        assert_every_rank_equals(recvs, wants[order], f"{workload} {algo}")
