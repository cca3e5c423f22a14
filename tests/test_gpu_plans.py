"""Persistent collectives (``*_init`` / ``ar_plan_start``) and HIP graph capture.

A plan must give the same bits as the one-shot call, follow its buffers'
current contents on every start, launch the expected number of kernels, and
replay correctly from a captured graph, replay after replay, with eager work
changing the inputs in between.
"""

import numpy as np
import pytest

import oracle
from oracle import dbt
from oracle.ring import chunk, same_bits

from gpu_util import from_dev, require_gpu, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _draw(n, length, seed, dtype="f32"):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal(length).astype(np.float32) for _ in range(n)]
    if dtype == "bf16":
        xs = [oracle.f32_to_bf16_bits(x) for x in xs]
    return xs


def _small(n, length):
    # the library's rule for the ring order's small-message kernel: count <= 2^16 and N * count <= 2^21
    return length <= (1 << 16) and n * length <= (1 << 21)


@pytest.mark.parametrize("algo,launches", [("fused", lambda n, m: 1), ("phases", lambda n, m: 2),
                                           ("ring", lambda n, m: 2 * (n - 1)), ("ring_pipelined", lambda n, m: 1),
                                           ("auto", lambda n, m: 1 if n < 24 or _small(n, m) or m * 4 < (4 << 20)
                                            or n * m * 4 <= (256 << 20) else 2)])
@pytest.mark.parametrize("n,length", [(5, 1003), (8, 8 * 4096 + 5), (32, 32 * 257 + 3), (32, 32 * 4100 + 3),
                                      (24, (1 << 20) + 3)])
def test_allreduce_plan_matches_and_follows_inputs(n, length, algo, launches):
    import torch

    ar = _ar()
    xs = _draw(n, length, seed=n)
    sends = [to_dev(x, "f32") for x in xs]
    recvs = [torch.empty(length, device="cuda:0") for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    assert plan.num_launches == launches(n, length)
    for rep in range(3):
        want, _ = oracle.ring_allreduce(xs)
        plan.start()
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(from_dev(recvs[r], "f32"), want[r], "f32"), (rep, r)
        # new contents in the same buffers: the next start must see them
        xs = [x * np.float32(1.5) + np.float32(rep) for x in xs]
        for r in range(n):
            sends[r].copy_(to_dev(xs[r], "f32"))
    plan.close()
    plan.close()


@pytest.mark.parametrize("algo", ["fused", "ring", "ring_pipelined"])
def test_phase_plans(algo):
    import torch

    ar = _ar()
    n, length = 7, 7 * 1000 + 6
    xs = _draw(n, length, seed=3, dtype="bf16")
    sends = [to_dev(x, "bf16") for x in xs]
    shards = [torch.empty(chunk(r, n, length)[1] - chunk(r, n, length)[0], dtype=torch.bfloat16, device="cuda:0")
              for r in range(n)]
    outs = [torch.empty(length, dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
    rs = ar.ar_reduce_scatter_init(sends, shards, algo=algo)
    ag = ar.ar_all_gather_init(shards, outs, algo=algo)
    assert rs.num_launches == (n - 1 if algo == "ring" else 1)
    assert ag.num_launches == (n if algo == "ring" else 1)
    ar.ar_plan_start(rs)
    ar.ar_plan_start(ag)
    torch.cuda.synchronize()
    want, _ = oracle.ring_allreduce(xs, dtype="bf16")
    for r in range(n):
        assert same_bits(from_dev(outs[r], "bf16"), want[r], "bf16")
    ar.ar_plan_free(rs)
    ar.ar_plan_free(ag)


RING_ORDER = ("fused", "phases", "ring", "ring_pipelined", "staged")
TREE_ORDER = {"tree": "tree", "tree_steps": "tree", "recursive_doubling": "recursive_doubling",
              "halving_doubling": "halving_doubling", "halving_doubling_steps": "halving_doubling"}


def _want(algo, xs):
    """The oracle's float32 sum for an algorithm: the ring's order, a tree order's
    executed schedule, or the double binary tree's."""
    from oracle.orders import order_allreduce

    if algo in RING_ORDER:
        return oracle.ring_allreduce(xs)[0]
    if algo.startswith("double_binary_tree"):
        return dbt.double_binary_tree_allreduce(xs, "sum", "f32")[0]
    return order_allreduce(TREE_ORDER[algo], xs)[0]


@pytest.mark.parametrize("algo", RING_ORDER + ("tree", "tree_steps", "halving_doubling_steps", "double_binary_tree",
                                               "double_binary_tree_steps"))
def test_graph_capture_replays(algo, monkeypatch):
    """Capture 3 starts of a plan in a HIP graph; replay it 4 times with eager input
    changes in between, checking every replay against the oracle.  The staged form
    runs with one tile of results per segment (8 segments, 16 launches per start)."""
    import torch

    if algo == "staged":
        monkeypatch.setenv("AR_STAGE_BYTES", "8192")
    ar = _ar()
    n, length = 8, 8 * 2048 + 3
    xs = _draw(n, length, seed=11)
    sends = [to_dev(x, "f32") for x in xs]
    recvs = [torch.empty(length, device="cuda:0") for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.start(side)                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            plan.start()
    for rep in range(4):
        xs = [x + np.float32(rep + 1) * np.float32(0.25) for x in xs]
        for r in range(n):
            sends[r].copy_(to_dev(xs[r], "f32"))       # eager work between replays
        for r in range(n):
            recvs[r].fill_(-7.0)
        g.replay()
        torch.cuda.synchronize()
        want = _want(algo, xs)
        for r in range(n):
            assert same_bits(from_dev(recvs[r], "f32"), want[r], "f32"), (rep, r)


@pytest.mark.parametrize("algo", ["fused", "phases", "ring", "ring_pipelined", "staged", "tree", "tree_steps",
                                  "recursive_doubling", "halving_doubling_steps", "double_binary_tree",
                                  "double_binary_tree_steps"])
def test_block_limits_keep_the_bits(algo, monkeypatch):
    """A plan capped at 1, 3, 64 blocks (the kernels stride over their tiles), then
    uncapped again, gives the oracle's bits every time.  The staged form runs with
    one tile of results per segment (16 segments)."""
    import torch

    if algo == "staged":
        monkeypatch.setenv("AR_STAGE_BYTES", "8192")
    ar = _ar()
    n, length = 8, 8 * 4096 + 5
    xs = _draw(n, length, seed=21)
    sends = [to_dev(x, "f32") for x in xs]
    recvs = [torch.empty(length, device="cuda:0") for _ in range(n)]
    want = _want(algo, xs)
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    if algo == "staged":
        assert plan.num_launches == 2 * 16
    for cap in (1, 3, 64, 0):
        plan.limit_blocks(cap)
        for r in range(n):
            recvs[r].fill_(-3.0)
        plan.start()
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(from_dev(recvs[r], "f32"), want[r], "f32"), (cap, r)
    plan.close()


@pytest.mark.parametrize("n,count,dtype,want,launches", [
    (8, 1 << 26, "float32", "staged", 4),     # the headline, 8 x 256 MiB: staged, 2 segments of 128 MiB
    (8, 24 << 20, "float32", "fused", 1),     # 96 MiB per rank, 768 MiB in all: below the staged total
    (8, 8 << 20, "float32", "fused", 1),      # 32 MiB per rank, 256 MiB in all: fused
    (16, 1 << 24, "float32", "staged", 2),    # 16 x 64 MiB, 1 GiB in all: staged, one segment
    (16, 1 << 26, "float32", "phases", 2),    # 16 x 256 MiB, 4 GiB in all: the two phases
    (64, 1 << 24, "float32", "phases", 2),    # 64 x 64 MiB, 4 GiB in all: the two phases
    (32, 1 << 26, "float32", "phases", 2),    # 32 x 256 MiB, 8 GiB in all: the two phases (upper bound)
    (16, 1 << 27, "float32", "staged", 8),    # 16 x 512 MiB: above the per-rank bound, staged, 4 segments
    (48, 1 << 26, "float32", "staged", 12),   # 48 x 256 MiB, 12 GiB in all: staged, 6 segments of 42.7 MiB
    (64, (1 << 26) + 7, "float32", "staged", 16),  # the 64-rank workload, 16 GiB in all: staged, 8 segments
    (128, 1 << 25, "float32", "staged", 8),   # 128 x 128 MiB, 16 GiB in all: staged, 4 segments of 32 MiB
    (16, 8 << 20, "float32", "fused", 1),     # 16 x 32 MiB, 512 MiB in all: fused
    (8, 48 << 20, "bfloat16", "staged", 2),   # 96 MiB per rank of bf16 at 8 ranks: staged (16-bit total)
    (8, 1 << 26, "bfloat16", "staged", 2),    # the bf16 workload (128 MiB per rank): staged, one segment
    (16, 1 << 25, "bfloat16", "staged", 2),   # bf16, 16 x 64 MiB: staged
    (8, 1 << 24, "bfloat16", "fused", 1),     # 32 MiB per rank, 256 MiB in all: below the 16-bit total
    (4, 1 << 27, "float32", "fused", 1),      # 4 ranks: below the staged rank bound
    (6, 1 << 26, "float32", "staged", 4),     # 6 ranks x 256 MiB: staged, 2 segments of 128 MiB
    (64, 1 << 20, "float32", "fused", 1),     # 64 ranks x 4 MiB, 256 MiB in all: fused (read through the cache)
    (64, (1 << 20) + 1024, "float32", "phases", 2),  # just over 256 MiB in all: the two phases (many ranks)
    (24, 2 << 20, "float32", "fused", 1),     # 24 x 8 MiB, 192 MiB in all: fused
    (24, 3 << 20, "float32", "phases", 2),    # 24 x 12 MiB, 288 MiB in all: the two phases
])
def test_auto_choice(n, count, dtype, want, launches):
    """Which form AR_ALGO_AUTO plans at shapes on both sides of its bounds
    (validation and planning only: nothing is launched)."""
    import torch

    ar = _ar()
    tdt = getattr(torch, dtype)
    sends = [torch.empty(count, dtype=tdt, device="cuda:0") for _ in range(n)]
    recvs = [torch.empty(count, dtype=tdt, device="cuda:0") for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo="auto")
    assert plan.algo == want
    assert plan.num_launches == launches
    plan.close()


def _raw_init(fn, sends, recvs, count, algo="fused", ws=None, ws_bytes=0):
    """One of the ``*_init`` calls on raw addresses: (result code, plan handle, error detail)."""
    import ctypes

    from ring_allreduce_reduction_virtual_amd import _lib

    lib = _lib.lib()
    n = len(sends)
    table = ctypes.c_void_p * n
    plan = ctypes.c_void_p()
    head = (table(*sends), table(*recvs), count, _lib.DTYPES["f32"])
    if fn == "ar_all_gather_init":
        rc = lib.ar_all_gather_init(*head, n, _lib.ALGOS[algo], ws, ws_bytes, ctypes.byref(plan))
    else:
        rc = getattr(lib, fn)(*head, _lib.OPS["sum"], n, _lib.ALGOS[algo], ws, ws_bytes, ctypes.byref(plan))
    return rc, plan, lib.ar_get_last_error_detail().decode()


def test_plans_refuse_buffers_the_kernels_cannot_reach():
    """*_init asks the runtime where every buffer lives: plain and pinned host
    memory and buffers (or a workspace) that run past the end of their
    allocation are refused before anything is planned.  No refused plan
    exists, so nothing is ever launched on those addresses."""
    import ctypes

    import torch

    ar = _ar()
    from ring_allreduce_reduction_virtual_amd import _lib

    lib = _lib.lib()
    hip = ctypes.CDLL("libamdhip64.so")
    n, count = 4, 1 << 18                      # 1 MiB per rank
    xs = _draw(n, count, seed=77)
    sends = [to_dev(x, "f32") for x in xs]
    recvs = [torch.empty(count, device="cuda:0") for _ in range(n)]
    sp = [t.data_ptr() for t in sends]
    rp = [t.data_ptr() for t in recvs]

    rc, plan, _ = _raw_init("ar_allreduce_init", sp, rp, count)      # torch's own buffers pass
    assert rc == 0 and plan.value
    lib.ar_plan_free(plan)

    host = ctypes.create_string_buffer(count * 4 + 256)
    haddr = (ctypes.addressof(host) + 255) // 256 * 256
    rc, plan, detail = _raw_init("ar_allreduce_init", [haddr] + sp[1:], rp, count)
    assert rc == 1 and plan.value is None and "sendbufs[0] is host memory" in detail, detail
    shard = count // n
    rc, plan, detail = _raw_init("ar_all_gather_init", [sp[0], haddr] + sp[2:], rp, count)
    assert rc == 1 and plan.value is None and "sendbufs[1] is host memory" in detail, detail

    pinned = torch.empty(count, pin_memory=True)
    rc, plan, detail = _raw_init("ar_allreduce_init", sp, rp[:3] + [pinned.data_ptr()], count)
    assert rc == 1 and plan.value is None and "recvbufs[3] is host memory" in detail, detail

    dev = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(dev), ctypes.c_size_t(count * 4)) == 0
    wsp = ctypes.c_void_p()
    need = ar.ar_workspace_bytes("reduce_scatter", "ring", count, "f32", n)
    assert hip.hipMalloc(ctypes.byref(wsp), ctypes.c_size_t(need - 4096)) == 0
    try:
        rc, plan, _ = _raw_init("ar_allreduce_init", sp, rp[:2] + [dev.value] + rp[3:], count)   # fits exactly
        assert rc == 0 and plan.value
        lib.ar_plan_free(plan)
        rc, plan, detail = _raw_init("ar_allreduce_init", sp, rp[:2] + [dev.value + 4096] + rp[3:], count)
        assert rc == 1 and plan.value is None and "recvbufs[2] runs 4096 bytes past" in detail, detail
        # a reduce-scatter shard at the allocation's end fits; one element further does not
        tail = dev.value + count * 4 - shard * 4
        rc, plan, _ = _raw_init("ar_reduce_scatter_init", sp, [tail] + rp[1:], count)
        assert rc == 0 and plan.value
        lib.ar_plan_free(plan)
        rc, plan, detail = _raw_init("ar_reduce_scatter_init", sp, [tail + 4] + rp[1:], count)
        assert rc == 1 and plan.value is None and "recvbufs[0] runs 4 bytes past" in detail, detail
        # a workspace whose claimed size exceeds its allocation
        rc, plan, detail = _raw_init("ar_reduce_scatter_init", sp, rp, count, algo="ring", ws=wsp.value,
                                     ws_bytes=need)
        assert rc == 1 and plan.value is None and "workspace runs 4096 bytes past" in detail, detail
    finally:
        torch.cuda.synchronize()
        assert hip.hipFree(dev) == 0 and hip.hipFree(wsp) == 0

    # the refusals leave no runtime error behind for the next launch to report
    ar.ar_allreduce(sends, recvs)
    torch.cuda.synchronize()
    want, _ = oracle.ring_allreduce(xs)
    for r in range(n):
        assert same_bits(from_dev(recvs[r], "f32"), want[r], "f32"), r


def test_binding_refuses_a_workspace_off_the_buffers_gpu():
    """A workspace tensor must be contiguous memory of the buffers' GPU: the
    binding refuses a host tensor or a strided view before calling the library."""
    import torch

    ar = _ar()
    n, count = 4, 4096
    sends = [torch.randn(count, device="cuda:0") for _ in range(n)]
    shards = [torch.empty(count // n, device="cuda:0") for _ in range(n)]
    need = ar.ar_workspace_bytes("reduce_scatter", "ring", count, "f32", n)
    for ws, msg in ((torch.empty(need, dtype=torch.uint8), "on the buffers' GPU"),
                    (torch.empty(2 * need, dtype=torch.uint8, device="cuda:0")[::2], "contiguous")):
        with pytest.raises(ValueError, match=msg):
            ar.ar_reduce_scatter_ex(sends, shards, algo="ring", workspace=ws)
        with pytest.raises(ValueError, match=msg):
            ar.ar_reduce_scatter_init(sends, shards, algo="ring", workspace=ws)
    # a proper workspace still works, with the oracle's bits
    xs = [from_dev(t, "f32") for t in sends]
    ar.ar_reduce_scatter_ex(sends, shards, algo="ring",
                            workspace=torch.empty(need, dtype=torch.uint8, device="cuda:0"))
    torch.cuda.synchronize()
    want, _ = oracle.reduce_scatter(xs)
    for r in range(n):
        assert same_bits(from_dev(shards[r], "f32"), want[r], "f32"), r
