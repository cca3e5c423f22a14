"""GPU parity for the ring in one launch, in both forms: the persistent ring
(all 2(N-1) steps in one cooperative launch with grid barriers) and the
pipelined ring (each slice of each chunk carried through all steps by one
workgroup, no barrier).  The ring's bits for every dtype and operator, rank
counts up to 128, layouts, persistent plans with workgroup caps, the full
headline workload (every element); the persistent ring refuses graph capture, the
pipelined ring replays from a graph.

Every launch here runs alone on the device, as the grid barrier requires."""

import zlib

import numpy as np
import pytest

import oracle
from oracle.ring import f32_to_bf16_bits, f32_to_f16_bits, same_bits

from gpu_util import assert_every_rank_equals, from_dev, poison, require_gpu, to_dev, want_on_device

pytestmark = pytest.mark.gpu

ONE_LAUNCH = ["ring_persistent", "ring_pipelined"]

TORCH_OF = {"f16": "float16", "bf16": "bfloat16", "f32": "float32", "i32": "int32"}


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _draw(dtype, n, length, seed):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(n):
        if dtype == "i32":
            xs.append(rng.integers(-(2**31), 2**31, size=length, dtype=np.int32))
            continue
        f = (rng.standard_normal(length) * 2.0 ** rng.integers(-12, 12, size=length)).astype(np.float32)
        xs.append(f32_to_f16_bits(f) if dtype == "f16" else f32_to_bf16_bits(f) if dtype == "bf16" else f)
    return xs


def _dev(x, dtype):
    import torch

    if dtype in ("f16", "bf16"):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0").view(getattr(torch, TORCH_OF[dtype]))
    return to_dev(x, dtype)


def _host(t, dtype):
    import torch

    if dtype in ("f16", "bf16"):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return from_dev(t, dtype)


def _empty(n, length, dtype):
    import torch

    return [torch.full((length,), 0x5A, dtype=getattr(torch, TORCH_OF[dtype]), device="cuda:0") for _ in range(n)]


@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "prod"), ("f32", "min"), ("f32", "avg"),
                                      ("bf16", "sum"), ("bf16", "max"), ("f16", "sum"), ("f16", "avg"),
                                      ("i32", "sum"), ("i32", "max"), ("i32", "avg")])
@pytest.mark.parametrize("n,length", [(1, 9), (2, 1001), (3, 7), (5, 1003), (8, 8 * 4096 + 13), (17, 4099),
                                      (64, 64 * 300 + 5), (128, 128 * 40 + 3)])
@pytest.mark.parametrize("algo", ONE_LAUNCH)
def test_one_launch_ring_matches_the_oracle(algo, n, length, dtype, op):
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


@pytest.mark.parametrize("layout", ["in_place", "common_offset", "mixed_offsets"])
@pytest.mark.parametrize("algo", ONE_LAUNCH)
def test_one_launch_ring_layouts(algo, layout):
    import torch

    ar = _ar()
    n, length = 6, 6 * 2048 + 11
    xs = _draw("f32", n, length, seed=31)
    want, _ = oracle.ring_allreduce(xs)
    if layout == "in_place":
        sends = [_dev(x, "f32") for x in xs]
        recvs = sends
    else:
        sends, recvs = [], []
        for r in range(n):
            off = 1 if layout == "common_offset" else r % 4
            base = torch.empty(length + 8, device="cuda:0")
            v = base[off:off + length]
            v.copy_(_dev(xs[r], "f32"))
            sends.append(v)
            off2 = 1 if layout == "common_offset" else (r + 1) % 3
            recvs.append(torch.empty(length + 8, device="cuda:0")[off2:off2 + length])
    ar.ar_allreduce_ex(sends, recvs, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(recvs[r], "f32"), want[r], "f32"), f"rank {r}"


@pytest.mark.parametrize("algo", ONE_LAUNCH)
def test_one_launch_ring_plan_and_caps(algo):
    import torch

    ar = _ar()
    n, length = 8, 8 * 4096 + 5
    xs = _draw("bf16", n, length, seed=41)
    want, _ = oracle.ring_allreduce(xs, dtype="bf16")
    sends = [_dev(x, "bf16") for x in xs]
    recvs = _empty(n, length, "bf16")
    plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
    assert plan.num_launches == 1
    for cap in (0, 1, 5, 64, 0):
        plan.limit_blocks(cap)
        for t in recvs:
            t.zero_()
        plan.start()
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(recvs[r], "bf16"), want[r], "bf16"), (cap, r)
    plan.close()


def test_persistent_ring_refuses_graph_capture():
    import torch

    ar = _ar()
    n, length = 4, 4096
    sends = [torch.randn(length, device="cuda:0") for _ in range(n)]
    recvs = [torch.empty(length, device="cuda:0") for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo="ring_persistent")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(ar.ArError) as err:
        with torch.cuda.graph(g):
            plan.start()
    assert "captured" in str(err.value)
    torch.cuda.synchronize()
    plan.start()           # still usable outside a capture
    torch.cuda.synchronize()
    want, _ = oracle.ring_allreduce([s.cpu().numpy() for s in sends])
    assert same_bits(recvs[0].cpu().numpy(), want[0], "f32")
    plan.close()


def test_pipelined_ring_replays_from_a_graph():
    """Capture 3 starts of a pipelined-ring plan; replay 4 times with eager input
    changes in between, checking every replay against the oracle."""
    import torch

    ar = _ar()
    n, length = 8, 8 * 2048 + 3
    xs = _draw("f32", n, length, seed=51)
    sends = [_dev(x, "f32") for x in xs]
    recvs = _empty(n, length, "f32")
    plan = ar.ar_allreduce_init(sends, recvs, algo="ring_pipelined")
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
        xs = [x + np.float32(rep + 1) * np.float32(0.5) for x in xs]
        for r in range(n):
            sends[r].copy_(_dev(xs[r], "f32"))   # eager work between replays
        for t in recvs:
            t.fill_(-3.0)
        g.replay()
        torch.cuda.synchronize()
        want, _ = oracle.ring_allreduce(xs)
        for r in range(n):
            assert same_bits(_host(recvs[r], "f32"), want[r], "f32"), (rep, r)
    plan.close()


@pytest.mark.parametrize("algo", ONE_LAUNCH)
def test_one_launch_ring_headline_full_size_every_element(algo):
    import torch

    from inputs import WORKLOADS, make_inputs

    ar = _ar()
    w = WORKLOADS["headline"]
    xs = make_inputs(w)
    want = want_on_device(oracle.ring_order_fold(xs), "f32")
    sends = [_dev(x, "f32") for x in xs]
    recvs = _empty(w.nranks, w.count, "f32")
    poison(recvs)
    ar.ar_allreduce_ex(sends, recvs, algo=algo)
    torch.cuda.synchronize()
    assert_every_rank_equals(recvs, want, algo)
