"""GPU parity at the size limits: a rank buffer of more than 2^31 elements
(every element index past the 32-bit range), and the largest rank count at a
large size.

Inputs are drawn on the device from a seeded torch generator (N(0,1)
float32), then copied to the host, where the oracle folds the whole buffers
in the ring's order.  Its result goes back to the device once, and every
element of every rank's output is compared with it there, bit for bit.
"""

import numpy as np
import pytest

import oracle
from oracle.ring import same_bits

from gpu_util import assert_every_rank_equals, poison, require_gpu, want_on_device

pytestmark = pytest.mark.gpu


def _ar():
    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    return ar


def _inputs(n, count, seed):
    import torch

    g = torch.Generator(device="cuda:0").manual_seed(seed)
    return [torch.randn(count, generator=g, device="cuda:0") for _ in range(n)]


def _oracle_whole(sends):
    """The oracle's AllReduce of the device inputs, on the host, back on the device."""
    xs = [t.cpu().numpy() for t in sends]
    want = oracle.ring_order_fold(xs)
    return want, want_on_device(want, "f32")


def test_rank_buffers_beyond_2p31_elements():
    """2 ranks x (2^31 + 37) float32 (8 GiB per buffer): every algorithm of the ring order."""
    import torch

    ar = _ar()
    n, count = 2, (1 << 31) + 37
    print(f"[large] {n} x {count} f32", flush=True)
    sends = _inputs(n, count, seed=31)
    want, want_dev = _oracle_whole(sends)
    recvs = [torch.empty(count, device="cuda:0") for _ in range(n)]
    for algo in ("fused", "phases", "ring", "ring_pipelined", "staged"):
        print(f"[large] {algo}", flush=True)
        poison(recvs)
        ar.ar_allreduce_ex(sends, recvs, algo=algo)
        torch.cuda.synchronize()
        assert_every_rank_equals(recvs, want_dev, algo)
    edge = 1 << 31                          # the elements around 2^31, also on the host
    assert same_bits(recvs[1][edge - 5:edge + 5].cpu().numpy(), want[edge - 5:edge + 5], "f32")


def test_128_ranks_at_a_large_size():
    """128 ranks x (2^25 + 3) float32 (128 MiB per buffer): the default (the staged form), the two
    phases and the one-pass kernel."""
    import torch

    ar = _ar()
    n, count = 128, (1 << 25) + 3
    print(f"[large] {n} x {count} f32", flush=True)
    sends = _inputs(n, count, seed=128)
    _, want_dev = _oracle_whole(sends)
    recvs = [torch.empty(count, device="cuda:0") for _ in range(n)]
    for algo in ("auto", "fused", "phases"):
        print(f"[large] {algo}", flush=True)
        poison(recvs)
        if algo == "auto":
            ar.ar_allreduce(sends, recvs)
        else:
            ar.ar_allreduce_ex(sends, recvs, algo=algo)
        torch.cuda.synchronize()
        assert_every_rank_equals(recvs, want_dev, algo)
