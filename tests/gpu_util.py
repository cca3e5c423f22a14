"""Helpers shared by the GPU tests: moving seeded host buffers to the device
and back, and choosing sample positions for full-size checks."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TORCH_DTYPE_NAMES = {"f32": "float32", "bf16": "bfloat16", "i32": "int32"}


def require_gpu():
    """Import torch and the library, building it if it was never built; fail without a GPU."""
    import torch

    from ring_allreduce_reduction_virtual_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


def tdtype(dtype):
    import torch

    return getattr(torch, TORCH_DTYPE_NAMES[dtype])


def to_dev(x: np.ndarray, dtype: str, device="cuda:0"):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def from_dev(t, dtype: str) -> np.ndarray:
    import torch

    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(t):
    """Device tensor reinterpreted as same-width integers (for bitwise comparison)."""
    import torch

    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def sample_positions(length: int, nranks: int, seed: int, k: int = 4096) -> np.ndarray:
    """Random positions plus every chunk's first and last few elements."""
    from oracle.ring import chunk

    rng = np.random.default_rng(seed)
    pos = [rng.integers(0, length, size=min(k, length))] if length else []
    for c in range(nranks):
        s, e = chunk(c, nranks, length)
        for d in range(4):
            for p in (s + d, e - 1 - d):
                if s <= p < e:
                    pos.append(np.array([p]))
    if not pos:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate(pos).astype(np.int64))


def has_nan(x: np.ndarray, dtype: str) -> bool:
    """Whether a host buffer (float32, int32 or 16-bit patterns) holds a NaN."""
    if dtype == "f32":
        return bool(np.isnan(x).any())
    if dtype in ("bf16", "bf16acc32"):
        return bool(((x & 0x7FFF) > 0x7F80).any())
    if dtype == "f16":
        return bool(((x & 0x7FFF) > 0x7C00).any())
    return False


def want_on_device(want: np.ndarray, dtype: str):
    """An oracle result copied to the device once, so that every element of every
    rank's output can be compared there.

    On the device the comparison is bitwise; that is the oracle's NaN-as-a-class
    rule only when the result holds no NaN, which is checked here.
    """
    assert not has_nan(want, dtype), "bitwise comparison needs a NaN-free oracle result"
    return to_dev(want, "bf16" if dtype in ("bf16acc32", "f16") else dtype)


def assert_every_rank_equals(recvs, want_dev, label=""):
    """Every element of every rank's output equals the oracle's result, bit for bit."""
    import torch

    w = bits(want_dev)
    for r, t in enumerate(recvs):
        assert t.numel() == want_dev.numel(), f"{label}: rank {r} has {t.numel()} elements"
        assert torch.equal(bits(t), w), f"{label}: rank {r} differs from the oracle"


def poison(tensors):
    """Fill outputs with a value no result here can take (NaN, or -1 for int32),
    so that an element a kernel fails to write cannot pass."""
    import torch

    for t in tensors:
        if t.dtype == torch.int32:
            t.fill_(-1)
        else:
            t.fill_(float("nan"))
