"""GPU parity for the small-message kernels (chunks shorter than the
small-message threshold: every rank's values of a few positions staged through
LDS), across the threshold, for the ring order, the tree orders and the double
binary tree, every dtype class and several operators, rank counts from 2 to
128."""

import zlib

import numpy as np
import pytest

import oracle
from oracle.dbt import double_binary_tree_allreduce
from oracle.orders import order_allreduce
from oracle.ring import f32_to_bf16_bits, f32_to_f16_bits, same_bits

from gpu_util import from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

TORCH_OF = {"f16": "float16", "bf16acc32": "bfloat16", "bf16": "bfloat16", "f32": "float32", "i32": "int32"}
# the library's bounds: for the ring's order, chunks shorter than 8192 elements with
# chunk * N^2 <= 2^19 take the small-message kernel; for the tree orders, every message
# with N * count <= 2^20 elements
def threshold(n):
    return min(8192, (1 << 19) // (n * n) + 1)


def lengths(algo, n):
    if algo == "fused":
        th = threshold(n)
        edge = [(th - 1) * n, th * n - 1, th * n + 5]
    else:
        last = (1 << 20) // n                  # the longest buffer the tree orders' small kernels take
        edge = [last - 1, last, last + 1]
    return [x for x in [1, n - 1, n + 1, 7 * n + 3] + edge if x > 0]


def _draw(dtype, n, length, seed):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(n):
        if dtype == "i32":
            xs.append(rng.integers(-(2**31), 2**31, size=length, dtype=np.int32))
            continue
        f = (rng.standard_normal(length) * 2.0 ** rng.integers(-12, 12, size=length)).astype(np.float32)
        xs.append(f32_to_f16_bits(f) if dtype == "f16" else
                  f32_to_bf16_bits(f) if dtype in ("bf16", "bf16acc32") else f)
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


# halving/doubling is defined for power-of-two rank counts only
VALID = [(algo, n) for algo in ("fused", "tree", "halving_doubling", "double_binary_tree")
         for n in (2, 3, 8, 16, 64, 128) if algo != "halving_doubling" or not n & (n - 1)]


@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "max"), ("bf16", "sum"), ("f16", "avg"),
                                      ("i32", "sum"), ("bf16acc32", "sum"), ("bf16acc32", "avg")])
@pytest.mark.parametrize("algo,n", VALID)
def test_small_messages_across_the_threshold(algo, n, dtype, op):
    import torch

    require_gpu()
    import ring_allreduce_reduction_virtual_amd as ar

    for length in lengths(algo, n):
        xs = _draw(dtype, n, length, seed=zlib.crc32(f"{dtype}{op}{n}{length}".encode()))
        if algo == "fused":
            want, _ = oracle.ring_allreduce(xs, op=op, dtype=dtype)
        elif algo == "double_binary_tree":
            want, _ = double_binary_tree_allreduce(xs, op, dtype)
        else:
            want, _ = order_allreduce(algo, xs, op, dtype)
        sends = [_dev(x, dtype) for x in xs]
        recvs = [torch.full((length,), 0x5A, dtype=getattr(torch, TORCH_OF[dtype]), device="cuda:0")
                 for _ in range(n)]
        ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(recvs[r], dtype), want[r], dtype), (length, r)
        # in place as well
        ar.ar_allreduce_ex(sends, None, op=op, algo=algo, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(n):
            assert same_bits(_host(sends[r], dtype), want[r], dtype), ("in place", length, r)
