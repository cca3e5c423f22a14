"""AR_ALGO_STAGED (reduce into rank 0, then broadcast, segment by segment)
against the oracle's reduce-then-broadcast schedule (oracle/staged.py).

The staged AllReduce gives the ring's bits: its reducing launch folds in the
ring's association order, its broadcasting launch copies.  These tests cut
the buffers into segments of a few tiles (the AR_STAGE_BYTES environment
variable, read at every call), so that segment edges fall inside chunks and
between them, and check every rank's whole output against the executed
schedule, over dtypes, operators, ragged shapes, both address paths and in
place.  The full-size check at the headline shape is in test_gpu_parity.py.
"""

import zlib

import numpy as np
import pytest

import oracle
from oracle.ring import same_bits

from gpu_util import require_gpu
from test_gpu_random import _draw, _empty, _host, _offsets, _tensor

pytestmark = pytest.mark.gpu

# 8 KiB is one tile of 16-byte vectors (256 threads x 2 vectors) on the vector path
STAGE_SIZES = (8192, 3 * 8192, 40000, 1 << 20)


def _run(n, length, dtype, op, layout, stage, seed):
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    xs = _draw(dtype, n, length, seed=seed)
    # the staged form's own oracle (reduce onto rank 0, then broadcast, in the ring's
    # association order); its equality with the executed ring is pinned on the CPU
    want, _ = oracle.reduce_then_broadcast(xs, op=op, dtype=dtype, root=0)
    so, ro = _offsets(layout, n)
    sends = [_tensor(x, dtype, so[r]) for r, x in enumerate(xs)]
    recvs = None if layout == "in_place" else [_empty(length, dtype, ro[r]) for r in range(n)]
    out = ar.ar_allreduce_ex(sends, recvs, op=op, algo="staged", dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(out[r], dtype), want[r], dtype), f"rank {r} (stage {stage} B, {layout})"


@pytest.fixture
def stage_env(monkeypatch):
    def set_stage(nbytes):
        monkeypatch.setenv("AR_STAGE_BYTES", str(nbytes))
    return set_stage


@pytest.mark.parametrize("stage", STAGE_SIZES)
@pytest.mark.parametrize("n,length", [(1, 7), (2, 1), (3, 1000), (5, 1003), (8, 8 * 4096 + 5), (8, 1 << 16),
                                      (16, 65541), (64, 64 * 333 + 7), (128, 128 * 40 + 3)])
def test_staged_shapes_f32_sum(n, length, stage, stage_env):
    require_gpu()
    stage_env(stage)
    print(f"[staged] f32 sum n={n} len={length} stage={stage}", flush=True)
    _run(n, length, "f32", "sum", "fresh", stage, seed=n * 31 + length)


@pytest.mark.parametrize("layout", ["fresh", "offset", "mixed", "in_place"])
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "avg"), ("f32", "min"), ("bf16", "sum"),
                                      ("bf16", "max"), ("f16", "sum"), ("f16", "avg"), ("i32", "sum"),
                                      ("i32", "prod"), ("i32", "min"), ("bf16acc32", "sum"),
                                      ("bf16acc32", "avg")])
def test_staged_dtypes_ops_layouts(dtype, op, layout, stage_env):
    require_gpu()
    stage_env(3 * 8192)
    n, length = 7, 7 * 3000 + 5
    print(f"[staged] {dtype} {op} {layout}", flush=True)
    _run(n, length, dtype, op, layout, 3 * 8192, seed=zlib.crc32(f"{dtype}{op}{layout}".encode()))


def _random_cases(seed=2026, count=80):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        n = int(rng.choice((2, 3, 4, 5, 8, 9, 16, 31, 64, 128)))
        length = min(max(0, n * int(rng.choice((0, 1, 7, 64, 255, 1000, 2048))) + int(rng.integers(-3, 4))),
                     1 << 15)
        cases.append((n, length, str(rng.choice(("f32", "bf16", "f16", "i32", "bf16acc32"))),
                      str(rng.choice(("sum", "prod", "min", "max", "avg"))),
                      str(rng.choice(("fresh", "offset", "mixed", "in_place"))),
                      int(rng.choice((512, 4096, 8192, 20000, 1 << 20)))))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: "{}x{}-{}-{}-{}-{}".format(*c))
def test_staged_random(case, stage_env):
    require_gpu()
    n, length, dtype, op, layout, stage = case
    stage_env(stage)
    print(f"[staged] random {case}", flush=True)
    _run(n, length, dtype, op, layout, stage, seed=zlib.crc32(repr(case).encode()))


def test_staged_equals_fused_bits_and_segments(stage_env):
    """Several segments at 8 ranks x 2^20 float32: the fused kernel's bits,
    and a plan of two launches per segment that replays in a HIP graph."""
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    n, length = 8, (1 << 20) + 3
    xs = _draw("f32", n, length, seed=77)
    sends = [_tensor(x, "f32") for x in xs]
    fused = [_empty(length, "f32") for _ in range(n)]
    ar.ar_allreduce_ex(sends, fused, algo="fused")
    stage_env(1 << 20)                            # 1 MiB of results per segment: 4 segments
    staged = [_empty(length, "f32") for _ in range(n)]
    ar.ar_allreduce_ex(sends, staged, algo="staged")
    torch.cuda.synchronize()
    for r in range(n):
        assert torch.equal(staged[r].view(torch.int32), fused[0].view(torch.int32)), f"rank {r}"
    plan = ar.ar_allreduce_init(sends, staged, algo="staged")
    # chunks of 131,072 or 131,073 elements: the longest whole-vector body is 32,768 vectors,
    # 64 tiles of 512 vectors (8 KiB) per chunk, 512 tiles; 128 tiles of results per 1 MiB
    # segment: 4 segments of two launches
    assert plan.num_launches == 2 * 4
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    for t in staged:
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        plan.start(stream=stream)
    for rep in range(3):
        for t in staged:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(staged[r].view(torch.int32), fused[0].view(torch.int32)), (rep, r)
    plan.close()


# the copy forms: one destination per block grouped on an XCD (the default), whole tiles to
# every rank per block, one unit row of a tile to every rank per block
COPY_FORMS = {"xcd": {}, "whole": {"AR_BCAST_FORM": "0", "AR_GATHER_FORM": "0", "AR_HALF_TILES": "0"},
              "half": {"AR_BCAST_FORM": "0", "AR_GATHER_FORM": "0", "AR_HALF_TILES": "1"}}


@pytest.mark.parametrize("form", sorted(COPY_FORMS))
@pytest.mark.parametrize("n,length,dtype,op", [(5, 1003, "f32", "sum"), (8, 8 * 4096 + 5, "bf16", "sum"),
                                               (17, 4099, "i32", "max"), (64, 64 * 333 + 7, "f32", "sum"),
                                               (7, 7 * 3000 + 5, "bf16acc32", "avg"), (2, 9000, "f16", "min")])
def test_staged_every_broadcast_form(n, length, dtype, op, form, stage_env, monkeypatch):
    """The broadcast with one destination rank per block grouped on an XCD (the
    default), with whole tiles per block and with one unit row per block
    (AR_BCAST_FORM=0 and AR_HALF_TILES force those), over several segments."""
    require_gpu()
    stage_env(3 * 8192)
    for k, v in COPY_FORMS[form].items():
        monkeypatch.setenv(k, v)
    print(f"[staged] broadcast form {form} n={n} len={length} {dtype} {op}", flush=True)
    for layout in ("fresh", "offset", "in_place"):
        _run(n, length, dtype, op, layout, 3 * 8192, seed=n + length)


@pytest.mark.parametrize("form", sorted(COPY_FORMS))
@pytest.mark.parametrize("n,length,dtype", [(1, 7, "f32"), (3, 1000, "i32"), (5, 1003, "f32"), (8, 8 * 4096 + 5, "bf16"),
                                            (64, 64 * 333 + 7, "f32"), (128, 300, "f16"), (9, 9 * 4096 * 3 + 1, "f32")])
def test_all_gather_every_form(n, length, dtype, form, monkeypatch):
    """The fused all-gather with one destination rank per block grouped on an XCD
    (the default), whole tiles and unit rows to every rank per block, out of
    place and in place, against the oracle; and the phases' AllReduce, whose
    all-gather runs in place."""
    import torch
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    for k, v in COPY_FORMS[form].items():
        monkeypatch.setenv(k, v)
    xs = _draw(dtype, n, length, seed=n * 5 + length)
    shards_want, _ = oracle.reduce_scatter(xs, dtype=dtype)
    want, _ = oracle.all_gather(shards_want, length, dtype=dtype)
    for layout in ("fresh", "offset", "in_place"):
        so = 1 if layout == "offset" else 0
        if layout == "in_place":
            outs = [_empty(length, dtype) for _ in range(n)]
            shards = []
            for r in range(n):
                b, e = ar.ar_chunk_range(r, length, n)
                outs[r][b:e].copy_(_tensor(shards_want[r], dtype))
                shards.append(outs[r][b:e])
        else:
            shards = [_tensor(sh, dtype, so) for sh in shards_want]
            outs = [_empty(length, dtype, so) for _ in range(n)]
        ar.ar_all_gather_ex(shards, outs, algo="fused")
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(outs[r], dtype), want[r], dtype), (layout, r)
    sends = [_tensor(x, dtype) for x in xs]
    outs = [_empty(length, dtype) for _ in range(n)]
    ar.ar_allreduce_ex(sends, outs, algo="phases")
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(outs[r], dtype), want[r], dtype), ("phases", r)


def test_staged_is_allreduce_only():
    import ring_allreduce_reduction_virtual_amd as ar

    require_gpu()
    xs = _draw("f32", 4, 64, seed=1)
    sends = [_tensor(x, "f32") for x in xs]
    shards = [_empty(16, "f32") for _ in range(4)]
    with pytest.raises(ar.ArError) as e:
        ar.ar_reduce_scatter_ex(sends, shards, algo="staged")
    assert "UNSUPPORTED" in str(e.value)
    with pytest.raises(ar.ArError) as e:
        ar.ar_all_gather_ex(shards, sends, algo="staged")
    assert "UNSUPPORTED" in str(e.value)
