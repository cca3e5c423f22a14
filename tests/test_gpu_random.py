"""Seeded random GPU cases against the oracle.

Rank counts from 1 to 128, lengths around multiples of the rank count (so
chunks are uneven, empty or one element long), every dtype and operator,
every algorithm each collective accepts, and four layouts: fresh
allocations, views one element into every allocation (a common address
residue), views at different offsets per rank (no common residue: the
element path) and in place.  The cases are drawn once from a fixed seed, so
a failure names a case that reruns exactly.
"""

import zlib

import numpy as np
import pytest

import oracle
from oracle.orders import order_allreduce
from oracle.ring import f32_to_bf16_bits, f32_to_f16_bits, same_bits

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "bf16", "f16", "i32", "bf16acc32")
OPS = ("sum", "prod", "min", "max", "avg")
RING_ORDER = ("fused", "phases", "auto", "ring", "ring_persistent", "ring_pipelined")
ORDER_OF = {"tree": "tree", "tree_steps": "tree", "recursive_doubling": "recursive_doubling",
            "halving_doubling": "halving_doubling", "halving_doubling_steps": "halving_doubling"}
POW2 = ("recursive_doubling", "halving_doubling", "halving_doubling_steps")
RANKS = (1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 32, 64, 100, 128)
BASES = (0, 1, 2, 7, 8, 63, 64, 255, 256, 1000, 2048)
LAYOUTS = ("fresh", "offset", "mixed", "in_place")
TORCH_OF = {"f32": "float32", "bf16": "bfloat16", "f16": "float16", "i32": "int32", "bf16acc32": "bfloat16"}


def _accepts(n, dtype, algo):
    if algo in POW2 and n & (n - 1):
        return False
    return not (algo == "ring_persistent" and dtype == "bf16acc32")


def _allreduce_cases(seed=2024, count=300):
    rng = np.random.default_rng(seed)
    algos = RING_ORDER + tuple(ORDER_OF)
    cases = []
    while len(cases) < count:
        n = int(rng.choice(RANKS))
        length = max(0, n * int(rng.choice(BASES)) + int(rng.integers(-3, 4)))
        length = min(length, 1 << 15)
        dtype, op = str(rng.choice(DTYPES)), str(rng.choice(OPS))
        algo, layout = str(rng.choice(algos)), str(rng.choice(LAYOUTS))
        if _accepts(n, dtype, algo):
            cases.append((n, length, dtype, op, algo, layout))
    return cases


def _collective_cases(seed=2025, count=100):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        n = int(rng.choice(RANKS))
        length = min(max(0, n * int(rng.choice(BASES)) + int(rng.integers(-3, 4))), 1 << 15)
        cases.append((n, length, str(rng.choice(DTYPES)), str(rng.choice(OPS)),
                      str(rng.choice(("fused", "ring", "ring_pipelined"))), str(rng.choice(("fresh", "in_place")))))
    return cases


def _draw(dtype, n, length, seed):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(n):
        if dtype == "i32":
            xs.append(rng.integers(-(2**31), 2**31, size=length, dtype=np.int32))
            continue
        f = (rng.standard_normal(length) * 2.0 ** rng.integers(-10, 10, size=length)).astype(np.float32)
        xs.append(f32_to_f16_bits(f) if dtype == "f16" else f32_to_bf16_bits(f) if dtype in ("bf16", "bf16acc32")
                  else f)
    return xs


def _tensor(x, dtype, offset=0):
    """A device tensor holding x, `offset` elements into a larger allocation."""
    import torch

    tdt = getattr(torch, TORCH_OF[dtype])
    base = torch.empty(len(x) + 8, dtype=tdt, device="cuda:0")
    view = base[offset:offset + len(x)]
    if len(x):
        host = torch.from_numpy(np.ascontiguousarray(x).view(np.int16 if x.dtype == np.uint16 else x.dtype))
        view.copy_(host.to("cuda:0").view(tdt))
    return view


def _empty(length, dtype, offset=0):
    import torch

    tdt = getattr(torch, TORCH_OF[dtype])
    base = torch.full((length + 8,), 0x5A, dtype=tdt, device="cuda:0")
    return base[offset:offset + length]


def _host(t, dtype):
    import torch

    t = t.detach().cpu()
    if dtype in ("f16", "bf16", "bf16acc32"):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _offsets(layout, n):
    if layout == "offset":
        return [1] * n, [1] * n
    if layout == "mixed":
        return [r % 4 for r in range(n)], [(r + 1) % 3 for r in range(n)]
    return [0] * n, [0] * n


def _case_id(case):
    return "{}x{}-{}-{}-{}-{}".format(*case)


@pytest.mark.parametrize("case", _allreduce_cases(), ids=_case_id)
def test_random_allreduce(case):
    import torch

    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    n, length, dtype, op, algo, layout = case
    print(f"[random] allreduce {_case_id(case)}", flush=True)
    xs = _draw(dtype, n, length, seed=zlib.crc32(_case_id(case).encode()))
    if algo in ORDER_OF:
        want, _ = order_allreduce(ORDER_OF[algo], xs, op, dtype)
    else:
        want, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
    so, ro = _offsets(layout, n)
    sends = [_tensor(x, dtype, so[r]) for r, x in enumerate(xs)]
    recvs = None if layout == "in_place" else [_empty(length, dtype, ro[r]) for r in range(n)]
    out = ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(out[r], dtype), want[r], dtype), f"rank {r}"


@pytest.mark.parametrize("case", _collective_cases(), ids=_case_id)
def test_random_reduce_scatter_then_all_gather(case):
    import torch

    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    n, length, dtype, op, algo, layout = case
    print(f"[random] reduce-scatter / all-gather {_case_id(case)}", flush=True)
    xs = _draw(dtype, n, length, seed=zlib.crc32(_case_id(case).encode()))
    shards_want, _ = oracle.reduce_scatter(xs, op=op, dtype=dtype)
    store = "bf16" if dtype == "bf16acc32" else dtype
    gathered_want, _ = oracle.all_gather(shards_want, length, dtype=store)
    sends = [_tensor(x, dtype) for x in xs]
    bounds = [ar.ar_chunk_range(r, length, n) for r in range(n)]
    if layout == "in_place":
        shards = [sends[r][b:e] for r, (b, e) in enumerate(bounds)]      # shard r inside send[r]
    else:
        shards = [_empty(e - b, dtype) for b, e in bounds]
    ar.ar_reduce_scatter_ex(sends, shards, op=op, algo=algo, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(shards[r], dtype), shards_want[r], dtype), f"shard {r}"
    if layout == "in_place":
        outs = sends                                                     # shard r already sits in chunk r
    else:
        outs = [_empty(length, dtype) for _ in range(n)]
    ar.ar_all_gather_ex(shards, outs, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert same_bits(_host(outs[r], store), gathered_want[r], store), f"rank {r}"
