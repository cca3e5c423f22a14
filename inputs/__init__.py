"""Seeded synthetic inputs for the ring AllReduce workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and
the benchmark.  It only draws random numbers: it holds none of the
collective's arithmetic (no chunking, no reduction, no rounding of sums).

Each virtual rank ``r`` of a workload with seed ``s`` draws its values from
its own PCG64 stream ``numpy.random.default_rng([s, r])`` and (outlier
workload only) its outlier mask from a second stream ``default_rng([s, r, 1])``,
so a rank's data does not depend on how many ranks are generated or in which
order, and a shortened buffer is exactly the head of the full-length one.

Value recipes (the collective's pages name no dataset; gradient-like
synthetic values stand in for "a gradient buffer on each worker"):

* ``int_pm8``       integers drawn uniformly from [-8, 8] inclusive, stored
                    as float32 (every partial sum is exact);
* ``normal``        N(0, sigma^2) drawn in float32;
* ``normal_bf16``   N(0, sigma^2) drawn in float32, then converted to
                    bfloat16 by torch's CPU conversion; held as uint16 bit
                    patterns;
* ``int32_full``    int32 drawn uniformly over [-2^31, 2^31 - 1];
* ``normal_outlier`` N(0, 1) float32 where an independent 1% of elements
                    (Bernoulli(0.01) per element per rank) is multiplied by
                    1e4 in float32.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_rank", "make_inputs", "np_dtype"]


@dataclass(frozen=True)
class Workload:
    name: str
    nranks: int
    count: int          # elements per rank
    dtype: str          # "f32" | "bf16" | "i32"
    ops: tuple          # reduction operators exercised on this workload
    values: str         # value recipe, see module docstring
    seed: int
    sigma: float = 1.0
    phases: tuple = ("allreduce",)
    note: str = field(default="", compare=False)


WORKLOADS = {
    "c1": Workload("c1", 4, 1024, "f32", ("sum",), "int_pm8", 0,
                   note="N=4 x 1024 fp32, integers in [-8,8]: exact, closed-form sums"),
    "c2": Workload("c2", 8, 1 << 20, "f32", ("sum",), "normal", 1,
                   note="N=8 x 2^20 fp32 N(0,1): one gradient bucket"),
    "c3": Workload("c3", 8, 1 << 26, "bf16", ("sum",), "normal_bf16", 2, sigma=1e-2,
                   note="N=8 x 2^26 bf16 N(0,1e-2), rounded to bf16 after every ring add"),
    "c4": Workload("c4", 16, 1 << 24, "i32", ("sum", "min", "max"), "int32_full", 3,
                   note="N=16 x 2^24 int32 over the full range; wrapping sum, min, max"),
    "c5": Workload("c5", 64, (1 << 26) + 7, "f32", ("sum",), "normal_outlier", 4,
                   phases=("allreduce", "reduce_scatter", "all_gather"),
                   note="N=64 x (2^26+7) fp32 with 1% x1e4 outliers; uneven chunks"),
    "headline": Workload("headline", 8, 1 << 26, "f32", ("sum",), "normal", 1,
                         note="N=8 x 2^26 fp32 N(0,1): 256 MiB per rank"),
}


def np_dtype(dtype: str):
    """Host storage type of a buffer dtype (bf16 is held as raw uint16 bits)."""
    return {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}[dtype]


def _bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    import torch  # torch's CPU float32 -> bfloat16 conversion, used only to quantise inputs

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_rank(w: Workload, r: int, count: int | None = None) -> np.ndarray:
    """Draw rank ``r``'s buffer of workload ``w`` (``count`` overrides its length).

    Every recipe draws element by element from per-rank streams, so the
    first ``count`` elements equal the head of the full-length draw.
    """
    n = w.count if count is None else int(count)
    rng = np.random.default_rng([w.seed, r])
    if w.values == "int_pm8":
        return rng.integers(-8, 9, size=n, dtype=np.int64).astype(np.float32)
    if w.values == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
        return x
    if w.values == "normal_bf16":
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(w.sigma)
        return _bf16_bits_from_f32(x)
    if w.values == "int32_full":
        return rng.integers(-(1 << 31), 1 << 31, size=n, dtype=np.int32)
    if w.values == "normal_outlier":
        x = rng.standard_normal(n, dtype=np.float32)
        mask = np.random.default_rng([w.seed, r, 1]).random(n, dtype=np.float32) < np.float32(0.01)
        x[mask] *= np.float32(1e4)
        return x
    raise ValueError(f"unknown value recipe {w.values!r}")


def make_inputs(w: Workload | str, count: int | None = None, nranks: int | None = None,
                threads: int | None = None) -> list:
    """All ranks' buffers of a workload, drawn in parallel threads.

    ``nranks`` overrides the rank count (ranks keep their own streams).
    numpy's generators release the GIL, so the per-rank draws overlap.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    n = w.nranks if nranks is None else int(nranks)
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)), max(n, 1))
    if threads <= 1 or n <= 1:
        return [make_rank(w, r, count) for r in range(n)]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda r: make_rank(w, r, count), range(n)))
