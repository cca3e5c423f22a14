"""The slab tile order of the launches that stream every rank's buffer at once
(the fused AllReduce, the staged reduce, the phases' and the standalone fused
reduce-scatter, the fused binomial-tree and double-binary-tree AllReduces)
against the oracle.

In that order the launch's tiles are cut into eight contiguous slabs, one per
XCD, and the blocks of one XCD walk one slab; blocks past the last whole group
of eight walk nothing, and a grid of fewer than eight blocks walks the tiles in
the plain order.  The library takes it from 64 ranks; the AR_TILE_XCD
environment variable (read at every call) moves that bound, so these tests
force it on from 2 ranks and compare every rank's whole output with the
executed ring of the oracle: ragged shapes, several tiles per chunk, segments
of the staged form that start inside a chunk, grids capped at sizes that are
and are not multiples of eight, and capped below eight.
"""

import pytest

import oracle
from oracle.dbt import double_binary_tree_allreduce
from oracle.orders import order_allreduce
from oracle.ring import same_bits

from gpu_util import require_gpu
from test_gpu_random import _draw, _empty, _host, _offsets, _tensor

pytestmark = pytest.mark.gpu

SHAPES = [(2, 1, "f32", "sum"), (3, 1000, "f32", "sum"), (5, 5 * 3 * 4096 + 7, "f32", "sum"),
          (8, 8 * 8192 + 5, "bf16", "sum"), (17, 17 * 4099, "i32", "max"), (64, 64 * 333 + 7, "f32", "sum"),
          (7, 7 * 3000 + 5, "bf16acc32", "avg"), (9, 9 * 4096 * 3 + 1, "f16", "min")]


@pytest.fixture
def slab_order(monkeypatch):
    monkeypatch.setenv("AR_TILE_XCD", "2")
    monkeypatch.setenv("AR_STAGE_BYTES", str(3 * 8192))   # segments that start inside chunks


@pytest.mark.parametrize("algo", ["fused", "staged", "phases"])
@pytest.mark.parametrize("n,length,dtype,op", SHAPES)
def test_slab_order_allreduce(n, length, dtype, op, algo, slab_order):
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    print(f"[tile order] slabs {algo} n={n} len={length} {dtype} {op}", flush=True)
    xs = _draw(dtype, n, length, seed=n * 7 + length)
    want = oracle.ring_allreduce(xs, op=op, dtype=dtype)[0]
    for layout in ("fresh", "mixed"):
        so, ro = _offsets(layout, n)
        sends = [_tensor(x, dtype, so[r]) for r, x in enumerate(xs)]
        recvs = [_empty(length, dtype, ro[r]) for r in range(n)]
        ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(recvs[r], dtype), want[r], dtype), (layout, r)


@pytest.mark.parametrize("n,length,dtype,op", SHAPES)
def test_slab_order_reduce_scatter(n, length, dtype, op, slab_order):
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    print(f"[tile order] slabs reduce-scatter n={n} len={length} {dtype} {op}", flush=True)
    xs = _draw(dtype, n, length, seed=n * 11 + length)
    shards_want, _ = oracle.reduce_scatter(xs, op=op, dtype=dtype)
    sends = [_tensor(x, dtype) for x in xs]
    shards = [_empty(len(shards_want[r]), dtype) for r in range(n)]
    ar.ar_reduce_scatter_ex(sends, shards, op=op, algo="fused", dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(shards[r], dtype), shards_want[r], dtype), r


@pytest.mark.parametrize("cap", [1, 5, 8, 13, 24, 0])
@pytest.mark.parametrize("algo", ["fused", "staged", "phases"])
def test_slab_order_capped_grids(algo, cap, slab_order):
    """Plans whose grids are capped after planning (ar_plan_limit_blocks): a
    multiple of eight blocks, a remainder of idle blocks, and fewer than eight
    (the plain order); 0 puts the planned grid back."""
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    n, length = 6, 6 * 5 * 4096 + 3
    xs = _draw("f32", n, length, seed=cap + 100)
    want = oracle.ring_allreduce(xs, op="sum", dtype="f32")[0]
    sends = [_tensor(x, "f32") for x in xs]
    recvs = [_empty(length, "f32") for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    plan.limit_blocks(cap)
    for _ in range(2):
        for r in range(n):
            recvs[r].fill_(-7.0)
        plan.start()
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(recvs[r], "f32"), want[r], "f32"), (cap, r)
    plan.close()


@pytest.mark.parametrize("n,length,algo", [
    (8, (1 << 21) + 13, "auto"),    # 64 MiB of inputs, read through the last-level cache: slabs
    (16, 1 << 22, "auto"),          # 256 MiB, the cached-load bound: slabs
    (8, 1 << 20, "auto"),           # 32 MiB: the plain order
    (32, (1 << 18) + 5, "fused"),   # 32 ranks: slabs at any size
    (12, 3 * (1 << 21) + 1, "fused"),  # 288 MiB, streamed from HBM: the plain order
])
def test_default_tile_order_of_the_fused_allreduce(n, length, algo, monkeypatch):
    """The library's own rule, with no override: the fused AllReduce walks slabs
    from 32 ranks and whenever its inputs hold 64-256 MiB in all; whole outputs
    against the oracle on both sides of each bound."""
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    monkeypatch.delenv("AR_TILE_XCD", raising=False)
    print(f"[tile order] default rule {algo} n={n} len={length}", flush=True)
    xs = _draw("f32", n, length, seed=n * 13 + length)
    want = oracle.ring_allreduce(xs, op="sum", dtype="f32")[0]
    sends = [_tensor(x, "f32") for x in xs]
    recvs = [_empty(length, "f32") for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    assert plan.algo == "fused"
    plan.close()
    ar.ar_allreduce_ex(sends, recvs, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], "f32"), want[r], "f32"), r


# longer than the tree orders' small-message bound (2^16 elements per rank), so
# the tiled kernels run
TREE_SHAPES = [(3, 65537 + 1000, "f32", "sum"), (5, 5 * 3 * 8192 + 7, "f32", "sum"),
               (8, 8 * 16384 + 5, "bf16", "sum"), (17, 17 * 4099, "i32", "max"), (64, 64 * 1100 + 7, "f32", "sum"),
               (7, 7 * 10000 + 5, "bf16acc32", "avg"), (9, 9 * 8192 + 1, "f16", "min"), (16, 16 * 8192 + 3, "f32", "prod")]
TREE_CASES = [(algo,) + shape for algo in ("tree", "halving_doubling", "double_binary_tree") for shape in TREE_SHAPES
              if algo != "halving_doubling" or not shape[0] & (shape[0] - 1)]


@pytest.mark.parametrize("algo,n,length,dtype,op", TREE_CASES)
def test_slab_order_tree_orders(algo, n, length, dtype, op, slab_order):
    """The fused tree-order kernels in the slab order, against their own
    orders' oracles (halving/doubling: power-of-two rank counts only)."""
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    print(f"[tile order] slabs {algo} n={n} len={length} {dtype} {op}", flush=True)
    xs = _draw(dtype, n, length, seed=n * 17 + length)
    if algo == "double_binary_tree":
        want, _ = double_binary_tree_allreduce(xs, op, dtype)
    else:
        want, _ = order_allreduce(algo, xs, op, dtype)
    sends = [_tensor(x, dtype) for x in xs]
    recvs = [_empty(length, dtype) for _ in range(n)]
    ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], dtype), want[r], dtype), r


@pytest.mark.parametrize("algo", ["tree", "halving_doubling", "double_binary_tree"])
@pytest.mark.parametrize("n,length", [(8, (1 << 21) + 13), (16, (1 << 20) + 5)])
def test_default_rule_of_the_tree_orders(algo, n, length, monkeypatch):
    """The tree orders' one-pass kernels under the library's own rule: 64-128
    MiB of inputs, read through the last-level cache and walked in per-XCD
    slabs; whole outputs against each order's oracle."""
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    monkeypatch.delenv("AR_TILE_XCD", raising=False)
    print(f"[tile order] default rule {algo} n={n} len={length}", flush=True)
    xs = _draw("f32", n, length, seed=n * 19 + length)
    if algo == "double_binary_tree":
        want, _ = double_binary_tree_allreduce(xs, "sum", "f32")
    else:
        want, _ = order_allreduce(algo, xs, "sum", "f32")
    sends = [_tensor(x, "f32") for x in xs]
    recvs = [_empty(length, "f32") for _ in range(n)]
    ar.ar_allreduce_ex(sends, recvs, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], "f32"), want[r], "f32"), r
