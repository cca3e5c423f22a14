"""Python binding of libar.so with the C ABI's names, taking torch tensors.

Argument marshalling only: each function checks the tensors (same CUDA
device, contiguous, matching dtype and sizes), collects their device
addresses and the stream handle, and makes one call into the library.  All
arithmetic runs in the library's HIP kernels.  PyTorch provides the device
memory and the stream.

``sendbufs`` / ``recvbufs`` are sequences of one tensor per virtual rank.
``count`` is always the full per-rank length (see include/ar.h): for
reduce-scatter the receive tensors hold one chunk each, for all-gather the
send tensors do.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

_TORCH_DTYPES = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int32: "i32"}


def _stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_of(tensors):
    dt = tensors[0].dtype
    if dt not in _TORCH_DTYPES:
        raise TypeError(f"unsupported dtype {dt}; use float32, bfloat16 or int32")
    for t in tensors:
        if t.dtype != dt:
            raise TypeError("all buffers must have the same dtype")
    return _TORCH_DTYPES[dt]


def _check_tensors(sendbufs, recvbufs):
    if len(sendbufs) != len(recvbufs):
        raise ValueError("need one send and one receive buffer per rank")
    if not 1 <= len(sendbufs) <= _lib.MAX_RANKS:
        raise ValueError(f"nranks must be in [1, {_lib.MAX_RANKS}]")
    dev = sendbufs[0].device
    for t in list(sendbufs) + list(recvbufs):
        if not isinstance(t, torch.Tensor):
            raise TypeError("buffers must be torch tensors")
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all buffers must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("buffers must be contiguous")
    return dev


def ar_chunk_range(c: int, count: int, nranks: int):
    """(begin, end) of chunk c: [c*count/nranks, (c+1)*count/nranks)."""
    b, e = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check("ar_chunk_range", _lib.lib().ar_chunk_range(c, count, nranks, ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def ar_workspace_bytes(coll: str, algo: str, count: int, dtype: str, nranks: int) -> int:
    v = _lib.lib().ar_workspace_bytes(_lib.COLLS[coll], _lib.ALGOS[algo], count, _lib.DTYPES[dtype], nranks)
    if v == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments for ar_workspace_bytes")
    return v


def ar_get_error_string(code: int) -> str:
    return _lib.lib().ar_get_error_string(code).decode()


def ar_dtype_size(dtype: str) -> int:
    return _lib.lib().ar_dtype_size(_lib.DTYPES[dtype])


def _device_guard(dev):
    return torch.cuda.device(dev)


def ar_allreduce_ex(sendbufs, recvbufs=None, op: str = "sum", algo: str = "fused", workspace=None, stream=None):
    """AllReduce of the ranks' send tensors into every receive tensor (in place when recvbufs is None)."""
    recvbufs = sendbufs if recvbufs is None else recvbufs
    dev = _check_tensors(sendbufs, recvbufs)
    dtype = _dtype_of(list(sendbufs) + list(recvbufs))
    count = sendbufs[0].numel()
    if any(t.numel() != count for t in list(sendbufs) + list(recvbufs)):
        raise ValueError("every AllReduce buffer must hold count elements")
    with _device_guard(dev):
        L = _lib.lib()
        rc = L.ar_allreduce_ex(_lib.ptr_array([t.data_ptr() for t in sendbufs]),
                               _lib.ptr_array([t.data_ptr() for t in recvbufs]),
                               count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs), _lib.ALGOS[algo],
                               None if workspace is None else workspace.data_ptr(),
                               0 if workspace is None else workspace.numel() * workspace.element_size(),
                               _stream_handle(stream))
    _lib.check("ar_allreduce_ex", rc)
    return recvbufs


def ar_allreduce(sendbufs, recvbufs=None, op: str = "sum", stream=None):
    """AllReduce with the fused one-pass kernel."""
    recvbufs = sendbufs if recvbufs is None else recvbufs
    dev = _check_tensors(sendbufs, recvbufs)
    dtype = _dtype_of(list(sendbufs) + list(recvbufs))
    count = sendbufs[0].numel()
    if any(t.numel() != count for t in list(sendbufs) + list(recvbufs)):
        raise ValueError("every AllReduce buffer must hold count elements")
    with _device_guard(dev):
        rc = _lib.lib().ar_allreduce(_lib.ptr_array([t.data_ptr() for t in sendbufs]),
                                     _lib.ptr_array([t.data_ptr() for t in recvbufs]),
                                     count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs),
                                     _stream_handle(stream))
    _lib.check("ar_allreduce", rc)
    return recvbufs


def _check_shards(shards, count, n, what):
    for r, t in enumerate(shards):
        b, e = ar_chunk_range(r, count, n)
        if t.numel() != e - b:
            raise ValueError(f"{what}[{r}] must hold chunk {r}: {e - b} elements")


def ar_reduce_scatter_ex(sendbufs, recvbufs, op: str = "sum", algo: str = "fused", workspace=None, stream=None):
    """Reduce-scatter: recvbufs[r] receives chunk r of the reduction.

    The ring algorithm needs a workspace (ar_workspace_bytes); when none is
    given one is taken from torch's allocator on the stream of the call.
    """
    dev = _check_tensors(sendbufs, recvbufs)
    dtype = _dtype_of(list(sendbufs) + list(recvbufs))
    n = len(sendbufs)
    count = sendbufs[0].numel()
    if any(t.numel() != count for t in sendbufs):
        raise ValueError("every send buffer must hold count elements")
    _check_shards(recvbufs, count, n, "recvbufs")
    need = ar_workspace_bytes("reduce_scatter", algo, count, dtype, n)
    with _device_guard(dev):
        if need and workspace is None:
            if stream is not None and not isinstance(stream, torch.cuda.Stream):
                raise ValueError("pass a workspace when the stream is a raw handle")
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            if stream is not None:
                workspace.record_stream(stream)   # freed only after the stream's work
        rc = _lib.lib().ar_reduce_scatter_ex(_lib.ptr_array([t.data_ptr() for t in sendbufs]),
                                             _lib.ptr_array([t.data_ptr() for t in recvbufs]),
                                             count, _lib.DTYPES[dtype], _lib.OPS[op], n, _lib.ALGOS[algo],
                                             None if workspace is None else workspace.data_ptr(),
                                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                                             _stream_handle(stream))
    _lib.check("ar_reduce_scatter_ex", rc)
    return recvbufs


def ar_reduce_scatter(sendbufs, recvbufs, op: str = "sum", stream=None):
    """Reduce-scatter with the fused one-pass kernel."""
    dev = _check_tensors(sendbufs, recvbufs)
    dtype = _dtype_of(list(sendbufs) + list(recvbufs))
    n = len(sendbufs)
    count = sendbufs[0].numel()
    if any(t.numel() != count for t in sendbufs):
        raise ValueError("every send buffer must hold count elements")
    _check_shards(recvbufs, count, n, "recvbufs")
    with _device_guard(dev):
        rc = _lib.lib().ar_reduce_scatter(_lib.ptr_array([t.data_ptr() for t in sendbufs]),
                                          _lib.ptr_array([t.data_ptr() for t in recvbufs]),
                                          count, _lib.DTYPES[dtype], _lib.OPS[op], n, _stream_handle(stream))
    _lib.check("ar_reduce_scatter", rc)
    return recvbufs


def ar_all_gather_ex(sendbufs, recvbufs, algo: str = "fused", workspace=None, stream=None):
    """All-gather: every recvbufs[r] receives all shards sendbufs[*] in rank order."""
    dev = _check_tensors(sendbufs, recvbufs)
    dtype = _dtype_of(list(sendbufs) + list(recvbufs))
    n = len(sendbufs)
    count = recvbufs[0].numel()
    if any(t.numel() != count for t in recvbufs):
        raise ValueError("every receive buffer must hold count elements")
    _check_shards(sendbufs, count, n, "sendbufs")
    with _device_guard(dev):
        rc = _lib.lib().ar_all_gather_ex(_lib.ptr_array([t.data_ptr() for t in sendbufs]),
                                         _lib.ptr_array([t.data_ptr() for t in recvbufs]),
                                         count, _lib.DTYPES[dtype], n, _lib.ALGOS[algo],
                                         None if workspace is None else workspace.data_ptr(),
                                         0 if workspace is None else workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream))
    _lib.check("ar_all_gather_ex", rc)
    return recvbufs


def ar_all_gather(sendbufs, recvbufs, stream=None):
    """All-gather with the fused one-pass kernel."""
    dev = _check_tensors(sendbufs, recvbufs)
    dtype = _dtype_of(list(sendbufs) + list(recvbufs))
    n = len(sendbufs)
    count = recvbufs[0].numel()
    if any(t.numel() != count for t in recvbufs):
        raise ValueError("every receive buffer must hold count elements")
    _check_shards(sendbufs, count, n, "sendbufs")
    with _device_guard(dev):
        rc = _lib.lib().ar_all_gather(_lib.ptr_array([t.data_ptr() for t in sendbufs]),
                                      _lib.ptr_array([t.data_ptr() for t in recvbufs]),
                                      count, _lib.DTYPES[dtype], n, _stream_handle(stream))
    _lib.check("ar_all_gather", rc)
    return recvbufs
