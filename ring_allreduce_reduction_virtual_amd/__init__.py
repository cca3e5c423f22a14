"""Ring AllReduce over N virtual ranks in one MI355X's HBM.

The computation lives in libar.so (HIP kernels for gfx950 behind the C ABI of
include/ar.h); this package is its Python binding, with the C functions'
names, taking torch tensors.  Importing the package does not load the
library; the first call does, and fails loudly if it is not built.
"""

from ._lib import ArError, lib  # noqa: F401
from .binding import (  # noqa: F401
    Plan,
    ar_all_gather,
    ar_all_gather_ex,
    ar_all_gather_init,
    ar_allreduce,
    ar_allreduce_ex,
    ar_allreduce_init,
    ar_chunk_range,
    ar_dtype_size,
    ar_get_error_string,
    ar_get_last_error_detail,
    ar_plan_algo,
    ar_plan_free,
    ar_plan_limit_blocks,
    ar_plan_num_launches,
    ar_plan_start,
    ar_reduce_scatter,
    ar_reduce_scatter_ex,
    ar_reduce_scatter_init,
    ar_reduce_scatter_noalloc,
    ar_workspace_bytes,
)

__all__ = [
    "ArError", "lib", "Plan",
    "ar_allreduce", "ar_allreduce_ex", "ar_reduce_scatter", "ar_reduce_scatter_ex",
    "ar_all_gather", "ar_all_gather_ex", "ar_workspace_bytes", "ar_chunk_range",
    "ar_get_error_string", "ar_get_last_error_detail", "ar_dtype_size",
    "ar_allreduce_init", "ar_reduce_scatter_init", "ar_all_gather_init", "ar_plan_start", "ar_plan_free",
    "ar_plan_limit_blocks", "ar_plan_num_launches", "ar_reduce_scatter_noalloc", "ar_plan_algo",
]
