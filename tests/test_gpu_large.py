"""GPU parity at the size limits: a rank buffer of more than 2^31 elements
(every element index past the 32-bit range), and the largest rank count at a
large size.

Inputs are drawn on the device from a seeded torch generator (N(0,1)
float32), so tens of GiB need no host copy.  The oracle sees the sampled
columns: random positions, every chunk's first and last element, and the
elements around 2^31, copied back to the host.
"""

import numpy as np
import pytest

import oracle
from oracle.ring import chunk, chunk_owner, same_bits

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _inputs(n, count, seed):
    import torch

    g = torch.Generator(device="cuda:0").manual_seed(seed)
    return [torch.randn(count, generator=g, device="cuda:0") for _ in range(n)]


def _positions(n, count, seed, extra=()):
    rng = np.random.default_rng(seed)
    edges = []
    for c in range(n):
        b, e = chunk(c, n, count)
        if e > b:
            edges += [b, e - 1]
    pos = np.concatenate([rng.integers(0, count, 2048), np.array(edges, dtype=np.int64),
                          np.array([p for p in extra if 0 <= p < count], dtype=np.int64)])
    return np.unique(pos)


def _check(sends, recvs, pos):
    import torch

    n, count = len(sends), sends[0].numel()
    idx = torch.from_numpy(pos).to("cuda:0")
    cols = np.stack([t[idx].cpu().numpy() for t in sends])
    want = oracle.ring_order_fold_columns(cols, chunk_owner(pos, n, count))
    for r, t in enumerate(recvs):
        assert same_bits(t[idx].cpu().numpy(), want, "f32"), f"rank {r}"


def test_rank_buffers_beyond_2p31_elements():
    """2 ranks x (2^31 + 37) float32 (8 GiB per buffer): every algorithm of the ring order."""
    import torch

    ar = _ar()
    n, count = 2, (1 << 31) + 37
    print(f"[large] {n} x {count} f32", flush=True)
    sends = _inputs(n, count, seed=31)
    recvs = [torch.empty(count, device="cuda:0") for _ in range(n)]
    edge = 1 << 31
    pos = _positions(n, count, seed=5, extra=range(edge - 5, edge + 5))
    for algo in ("fused", "phases", "ring", "ring_pipelined", "staged"):
        print(f"[large] {algo}", flush=True)
        for t in recvs:
            t.fill_(-1.0)
        ar.ar_allreduce_ex(sends, recvs, algo=algo)
        torch.cuda.synchronize()
        _check(sends, recvs, pos)
        assert torch.equal(recvs[0], recvs[1])


def test_128_ranks_at_a_large_size():
    """128 ranks x (2^25 + 3) float32 (128 MiB per buffer): the default (the staged form), the two
    phases and the one-pass kernel."""
    import torch

    ar = _ar()
    n, count = 128, (1 << 25) + 3
    print(f"[large] {n} x {count} f32", flush=True)
    sends = _inputs(n, count, seed=128)
    recvs = [torch.empty(count, device="cuda:0") for _ in range(n)]
    pos = _positions(n, count, seed=6)
    ar.ar_allreduce(sends, recvs)
    torch.cuda.synchronize()
    _check(sends, recvs, pos)
    first = recvs[0].clone()
    for algo in ("fused", "phases"):
        print(f"[large] {algo}", flush=True)
        ar.ar_allreduce_ex(sends, recvs, algo=algo)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(recvs[r], first), f"{algo} rank {r}"
