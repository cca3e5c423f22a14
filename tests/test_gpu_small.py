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
# the library's bounds: a message takes the small-message kernel when each rank holds
# at most 2^16 elements and all ranks together at most 2^21 elements (the ring's
# order) or 8 MiB (the tree orders)
ESIZE = {"f32": 4, "i32": 4, "bf16": 2, "f16": 2, "bf16acc32": 2}


def last_small(algo, n, dtype):
    """The longest per-rank buffer the small-message kernel of `algo` takes at N = n."""
    work = (1 << 21) if algo == "fused" else (8 << 20) // ESIZE[dtype]
    return min(1 << 16, work // n)


def lengths(algo, n, dtype):
    last = last_small(algo, n, dtype)
    return [x for x in [1, n - 1, n + 1, 7 * n + 3, last - 1, last, last + 1] if x > 0]


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

    for length in lengths(algo, n, dtype):
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
