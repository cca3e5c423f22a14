"""ctypes view of libar.so: the C ABI of include/ar.h, one Python call per C symbol.

Loading fails loudly when the library has not been built: there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libar.so")

# values of the C enums in include/ar.h
AR_SUCCESS = 0
RESULT_NAMES = {0: "AR_SUCCESS", 1: "AR_ERR_INVALID_ARGUMENT", 2: "AR_ERR_UNSUPPORTED",
                3: "AR_ERR_HIP", 4: "AR_ERR_INTERNAL"}
DTYPES = {"f32": 0, "bf16": 1, "i32": 2, "f16": 3, "bf16acc32": 4}
OPS = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}
ALGOS = {"fused": 0, "ring": 1, "phases": 2, "auto": 3, "tree": 4, "tree_steps": 5, "recursive_doubling": 6,
         "halving_doubling": 7, "halving_doubling_steps": 8, "ring_persistent": 9, "ring_pipelined": 10,
         "staged": 11, "double_binary_tree": 12, "double_binary_tree_steps": 13}
# algorithms whose bracketing is a tree, not the ring's (AllReduce only)
TREE_ALGOS = ("tree", "tree_steps", "recursive_doubling", "halving_doubling", "halving_doubling_steps",
              "double_binary_tree", "double_binary_tree_steps")
COLLS = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2}
MAX_RANKS = 128

# every function include/ar.h declares
EXPORTS = (
    "ar_allreduce", "ar_reduce_scatter", "ar_all_gather",
    "ar_allreduce_ex", "ar_reduce_scatter_ex", "ar_all_gather_ex",
    "ar_workspace_bytes", "ar_chunk_range", "ar_get_error_string",
    "ar_get_last_error_detail", "ar_dtype_size",
    "ar_allreduce_init", "ar_reduce_scatter_init", "ar_all_gather_init",
    "ar_plan_start", "ar_plan_num_launches", "ar_plan_free", "ar_plan_limit_blocks",
    "ar_reduce_scatter_noalloc", "ar_plan_algo",
)
# bytes of the fixed device array behind ar_reduce_scatter_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None

_vp = ctypes.c_void_p
_vpp = ctypes.POINTER(ctypes.c_void_p)
_sz = ctypes.c_size_t
_int = ctypes.c_int


def _declare(lib):
    sig = {
        "ar_allreduce": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _vp]),
        "ar_reduce_scatter": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _vp]),
        "ar_all_gather": (_int, [_vpp, _vpp, _sz, _int, _int, _vp]),
        "ar_allreduce_ex": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _int, _vp, _sz, _vp]),
        "ar_reduce_scatter_ex": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _int, _vp, _sz, _vp]),
        "ar_all_gather_ex": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _vp, _sz, _vp]),
        "ar_workspace_bytes": (_sz, [_int, _int, _sz, _int, _int]),
        "ar_chunk_range": (_int, [_int, _sz, _int, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
        "ar_get_error_string": (ctypes.c_char_p, [_int]),
        "ar_get_last_error_detail": (ctypes.c_char_p, []),
        "ar_dtype_size": (_sz, [_int]),
        "ar_allreduce_init": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _int, _vp, _sz, _vpp]),
        "ar_reduce_scatter_init": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _int, _vp, _sz, _vpp]),
        "ar_all_gather_init": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _vp, _sz, _vpp]),
        "ar_plan_start": (_int, [_vp, _vp]),
        "ar_plan_num_launches": (_int, [_vp]),
        "ar_plan_algo": (_int, [_vp]),
        "ar_plan_free": (_int, [_vp]),
        "ar_plan_limit_blocks": (_int, [_vp, ctypes.c_uint]),
        "ar_reduce_scatter_noalloc": (_int, [_vpp, _vpp, _sz, _int, _int, _int, _int, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library; raises if libar.so is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; build it with "
                "`python -m ring_allreduce_reduction_virtual_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _lib = handle
    return _lib


class ArError(RuntimeError):
    """A call into libar.so returned an error code."""

    def __init__(self, fn: str, code: int):
        L = lib()
        detail = L.ar_get_last_error_detail().decode()
        msg = L.ar_get_error_string(code).decode()
        super().__init__(f"{fn}: {RESULT_NAMES.get(code, code)} ({msg}){': ' + detail if detail else ''}")
        self.code = code
        self.detail = detail


def check(fn: str, code: int):
    if code != AR_SUCCESS:
        raise ArError(fn, code)


def ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(len(ptrs), 1))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr
