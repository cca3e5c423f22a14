"""Python binding of libar.so with the C ABI's names, taking torch tensors.

Argument marshalling only: each function checks the tensors (same CUDA
device, contiguous, matching dtype and sizes), collects their device
addresses and the stream handle, and makes one call into the library.  All
arithmetic runs in the library's HIP kernels.  PyTorch provides the device
memory and the stream.

``sendbufs`` / ``recvbufs`` are sequences of one tensor per virtual rank.
``count`` is always the full per-rank length (see include/ar.h): for
reduce-scatter the receive tensors hold one chunk each, for all-gather the
send tensors do.  ``algo`` names an ``ar_algo_t`` in lower case ("fused",
"ring", "phases", "auto", "ring_persistent", "ring_pipelined", "staged", and the tree
orders "tree", "tree_steps", "recursive_doubling", "halving_doubling",
"halving_doubling_steps", "double_binary_tree", "double_binary_tree_steps");
``op`` one of "sum", "prod", "min", "max", "avg".  The element type follows
the tensors (float32, bfloat16, float16, int32); ``dtype="bf16acc32"`` with
bfloat16 tensors keeps the partial sums in float32.

The ``*_init`` functions return a :class:`Plan`, the persistent form of a
call: validated once, then enqueued by :meth:`Plan.start` (or
:func:`ar_plan_start`) as often as wanted, including inside a HIP graph
capture.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

_TORCH_DTYPES = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int32: "i32", torch.float16: "f16"}


# The current stream's raw handle without building a torch.cuda.Stream object
# (measured on MI355X: 0.07 us against 2.7 us per call, a large share of a
# small call's host time); the public route where torch lacks the accessor.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device_index):
    """The hipStream_t to enqueue on: `stream` when given (a torch stream must
    belong to device `device_index`, the device the buffers live on; a raw
    handle is taken as given), else that device's current stream."""
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(device_index)
        return torch.cuda.current_stream(device_index).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        if stream.device_index != device_index:
            raise ValueError(f"the stream belongs to device {stream.device_index}, "
                             f"the buffers to device {device_index}")
        return stream.cuda_stream
    return int(stream)


def _marshal(sendbufs, recvbufs, dtype=None):
    """Check the two tensor lists; return (device, dtype name, send array, recv array)."""
    n = len(sendbufs)
    if len(recvbufs) != n:
        raise ValueError("need one send and one receive buffer per rank")
    if not 1 <= n <= _lib.MAX_RANKS:
        raise ValueError(f"nranks must be in [1, {_lib.MAX_RANKS}]")
    t0 = sendbufs[0]
    if not isinstance(t0, torch.Tensor) or not t0.is_cuda:
        raise ValueError("buffers must be CUDA tensors")
    dev, dt = t0.device, t0.dtype
    index = t0.get_device()
    if dt not in _TORCH_DTYPES:
        raise TypeError(f"unsupported dtype {dt}; use float32, bfloat16, float16 or int32")
    name = _TORCH_DTYPES[dt]
    if dtype is not None and dtype != name:
        if not (dtype == "bf16acc32" and name == "bf16"):
            raise TypeError(f"dtype {dtype!r} does not fit {dt} tensors")
        name = dtype
    sp = (ctypes.c_void_p * n)()
    rp = (ctypes.c_void_p * n)()
    tensor = torch.Tensor
    for i in range(n):
        s, r = sendbufs[i], recvbufs[i]
        # one cheap test per tensor; the slow path below says what is wrong
        if not (type(s) is tensor and type(r) is tensor and s.dtype is dt and r.dtype is dt
                and s.get_device() == index and r.get_device() == index
                and s.is_contiguous() and r.is_contiguous()):
            for t in (s, r):
                if not isinstance(t, torch.Tensor) or t.device != dev:
                    raise ValueError("all buffers must be tensors on the same GPU")
                if t.dtype != dt:
                    raise TypeError("all buffers must have the same dtype")
                if not t.is_contiguous():
                    raise ValueError("buffers must be contiguous")
        sp[i] = s.data_ptr()
        rp[i] = r.data_ptr()
    return dev, name, sp, rp


class _on_device:
    """Make ``dev`` the current device for a call, switching only when it is not already."""

    __slots__ = ("index", "prev")

    def __init__(self, dev):
        self.index = dev.index if dev.index is not None else torch.cuda.current_device()
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.index:
            self.prev = cur
            torch.cuda.set_device(self.index)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)
        return False


def _ws(workspace, dev):
    """Address and size of a workspace tensor, which must be contiguous memory of the buffers' GPU."""
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev:
        raise ValueError("the workspace must be a tensor on the buffers' GPU")
    if not workspace.is_contiguous():
        raise ValueError("the workspace must be contiguous")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


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


def ar_get_last_error_detail() -> str:
    """The calling thread's text for the last failed call into the library ("" if none)."""
    return _lib.lib().ar_get_last_error_detail().decode()


def _check_counts(coll, sendbufs, recvbufs):
    n = len(sendbufs)
    if coll == "allreduce":
        count = sendbufs[0].numel()
        for t in sendbufs:
            if t.numel() != count:
                raise ValueError("every AllReduce buffer must hold count elements")
        for t in recvbufs:
            if t.numel() != count:
                raise ValueError("every AllReduce buffer must hold count elements")
        return count
    full, shards, what = (sendbufs, recvbufs, "recvbufs") if coll == "reduce_scatter" else \
        (recvbufs, sendbufs, "sendbufs")
    count = full[0].numel()
    if any(t.numel() != count for t in full):
        raise ValueError("every full-length buffer must hold count elements")
    for r, t in enumerate(shards):
        b, e = ar_chunk_range(r, count, n)
        if t.numel() != e - b:
            raise ValueError(f"{what}[{r}] must hold chunk {r}: {e - b} elements")
    return count


def _workspace(coll, algo, count, dtype, n, workspace, dev, stream):
    need = ar_workspace_bytes(coll, algo, count, dtype, n)
    if need and workspace is None:
        if stream is not None and not isinstance(stream, torch.cuda.Stream):
            raise ValueError("pass a workspace when the stream is a raw handle")
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if stream is not None:
            workspace.record_stream(stream)   # freed only after the stream's work
    return workspace


# --------------------------------------------------------------------------
# one-shot calls
# --------------------------------------------------------------------------

def ar_allreduce(sendbufs, recvbufs=None, op: str = "sum", stream=None, dtype=None):
    """AllReduce (algorithm AR_ALGO_AUTO); in place when recvbufs is None."""
    recvbufs = sendbufs if recvbufs is None else recvbufs
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("allreduce", sendbufs, recvbufs)
    with _on_device(dev):
        rc = _lib.lib().ar_allreduce(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs),
                                     _stream_handle(stream, dev.index))
    _lib.check("ar_allreduce", rc)
    return recvbufs


def ar_allreduce_ex(sendbufs, recvbufs=None, op: str = "sum", algo: str = "fused", workspace=None, stream=None,
                    dtype=None):
    """AllReduce with the algorithm chosen by the caller; in place when recvbufs is None.

    Algorithms that keep float32 partials between steps (the ring, launched
    per step or pipelined, and the staged tree algorithms, for bf16acc32)
    need a workspace; when none is given one is taken from torch's allocator
    on the stream of the call.
    """
    recvbufs = sendbufs if recvbufs is None else recvbufs
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("allreduce", sendbufs, recvbufs)
    with _on_device(dev):
        workspace = _workspace("allreduce", algo, count, dtype, len(sendbufs), workspace, dev, stream)
        wp, wb = _ws(workspace, dev)
        rc = _lib.lib().ar_allreduce_ex(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs),
                                        _lib.ALGOS[algo], wp, wb, _stream_handle(stream, dev.index))
    _lib.check("ar_allreduce_ex", rc)
    return recvbufs


def ar_reduce_scatter(sendbufs, recvbufs, op: str = "sum", stream=None, dtype=None):
    """Reduce-scatter with the fused kernel: recvbufs[r] receives chunk r of the reduction."""
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("reduce_scatter", sendbufs, recvbufs)
    with _on_device(dev):
        rc = _lib.lib().ar_reduce_scatter(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs),
                                          _stream_handle(stream, dev.index))
    _lib.check("ar_reduce_scatter", rc)
    return recvbufs


def ar_reduce_scatter_ex(sendbufs, recvbufs, op: str = "sum", algo: str = "fused", workspace=None, stream=None,
                         dtype=None):
    """Reduce-scatter with the algorithm chosen by the caller.

    The ring algorithms ("ring", "ring_pipelined") need a workspace
    (ar_workspace_bytes); when none is given one is taken from torch's
    allocator on the stream of the call.
    """
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("reduce_scatter", sendbufs, recvbufs)
    n = len(sendbufs)
    with _on_device(dev):
        workspace = _workspace("reduce_scatter", algo, count, dtype, n, workspace, dev, stream)
        wp, wb = _ws(workspace, dev)
        rc = _lib.lib().ar_reduce_scatter_ex(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], n,
                                             _lib.ALGOS[algo], wp, wb, _stream_handle(stream, dev.index))
    _lib.check("ar_reduce_scatter_ex", rc)
    return recvbufs


def ar_reduce_scatter_noalloc(sendbufs, recvbufs, op: str = "sum", algo: str = "ring", stream=None, dtype=None):
    """Reduce-scatter as :func:`ar_reduce_scatter_ex`, with the ring's workspace
    taken from the library's fixed device array: no device memory is allocated."""
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("reduce_scatter", sendbufs, recvbufs)
    with _on_device(dev):
        rc = _lib.lib().ar_reduce_scatter_noalloc(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs),
                                                  _lib.ALGOS[algo], _stream_handle(stream, dev.index))
    _lib.check("ar_reduce_scatter_noalloc", rc)
    return recvbufs


def ar_all_gather(sendbufs, recvbufs, stream=None):
    """All-gather with the fused kernel: every recvbufs[r] receives all shards in rank order."""
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs)
    count = _check_counts("all_gather", sendbufs, recvbufs)
    with _on_device(dev):
        rc = _lib.lib().ar_all_gather(sp, rp, count, _lib.DTYPES[dtype], len(sendbufs),
                                      _stream_handle(stream, dev.index))
    _lib.check("ar_all_gather", rc)
    return recvbufs


def ar_all_gather_ex(sendbufs, recvbufs, algo: str = "fused", workspace=None, stream=None):
    """All-gather with the algorithm chosen by the caller."""
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs)
    count = _check_counts("all_gather", sendbufs, recvbufs)
    wp, wb = _ws(workspace, dev)
    with _on_device(dev):
        rc = _lib.lib().ar_all_gather_ex(sp, rp, count, _lib.DTYPES[dtype], len(sendbufs), _lib.ALGOS[algo],
                                         wp, wb, _stream_handle(stream, dev.index))
    _lib.check("ar_all_gather_ex", rc)
    return recvbufs


# --------------------------------------------------------------------------
# persistent collectives
# --------------------------------------------------------------------------

class Plan:
    """A persistent collective from one of the ``*_init`` calls.

    Holds references to its tensors (and workspace) so they outlive it;
    :meth:`start` enqueues the planned kernels; the plan is freed by
    :meth:`close` or when collected.
    """

    def __init__(self, handle, device, keep):
        self._handle = handle
        self.device = device
        self._index = device.index if device.index is not None else torch.cuda.current_device()
        self._keep = keep

    @property
    def num_launches(self) -> int:
        return _lib.lib().ar_plan_num_launches(self._handle)

    @property
    def algo(self) -> str:
        """The algorithm the plan runs (the default's choice for its shape), by name."""
        code = _lib.lib().ar_plan_algo(self._handle)
        return {v: k for k, v in _lib.ALGOS.items()}.get(code, str(code))

    def start(self, stream=None):
        if self._handle is None:
            raise ValueError("plan is closed")
        _lib.check("ar_plan_start", _lib.lib().ar_plan_start(self._handle, _stream_handle(stream, self._index)))

    def limit_blocks(self, max_blocks: int):
        """Cap the workgroups of every launch (0: back to the planned grids)."""
        if self._handle is None:
            raise ValueError("plan is closed")
        _lib.check("ar_plan_limit_blocks", _lib.lib().ar_plan_limit_blocks(self._handle, int(max_blocks)))

    def close(self):
        """Free the plan and drop its references to the tensors.  Work it has
        enqueued still reads and writes them: close it after that work has
        completed, or keep the tensors alive until then."""
        if self._handle is not None:
            _lib.lib().ar_plan_free(self._handle)
            self._handle = None
            self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def _make_plan(fn_name, call, device, keep):
    handle = ctypes.c_void_p()
    with torch.cuda.device(device):
        rc = call(ctypes.byref(handle))
    _lib.check(fn_name, rc)
    return Plan(handle, device, keep)


def ar_allreduce_init(sendbufs, recvbufs=None, op: str = "sum", algo: str = "auto", workspace=None,
                      dtype=None) -> Plan:
    """Persistent AllReduce; in place when recvbufs is None."""
    recvbufs = sendbufs if recvbufs is None else recvbufs
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("allreduce", sendbufs, recvbufs)
    with _on_device(dev):
        workspace = _workspace("allreduce", algo, count, dtype, len(sendbufs), workspace, dev, None)
    wp, wb = _ws(workspace, dev)
    L = _lib.lib()
    return _make_plan("ar_allreduce_init",
                      lambda h: L.ar_allreduce_init(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], len(sendbufs),
                                                    _lib.ALGOS[algo], wp, wb, h),
                      dev, (list(sendbufs), list(recvbufs), workspace))


def ar_reduce_scatter_init(sendbufs, recvbufs, op: str = "sum", algo: str = "fused", workspace=None,
                           dtype=None) -> Plan:
    """Persistent reduce-scatter (the ring algorithm gets a workspace from torch if none is given)."""
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs, dtype)
    count = _check_counts("reduce_scatter", sendbufs, recvbufs)
    n = len(sendbufs)
    with _on_device(dev):
        workspace = _workspace("reduce_scatter", algo, count, dtype, n, workspace, dev, None)
    wp, wb = _ws(workspace, dev)
    L = _lib.lib()
    return _make_plan("ar_reduce_scatter_init",
                      lambda h: L.ar_reduce_scatter_init(sp, rp, count, _lib.DTYPES[dtype], _lib.OPS[op], n,
                                                         _lib.ALGOS[algo], wp, wb, h),
                      dev, (list(sendbufs), list(recvbufs), workspace))


def ar_all_gather_init(sendbufs, recvbufs, algo: str = "fused", workspace=None) -> Plan:
    """Persistent all-gather."""
    dev, dtype, sp, rp = _marshal(sendbufs, recvbufs)
    count = _check_counts("all_gather", sendbufs, recvbufs)
    wp, wb = _ws(workspace, dev)
    L = _lib.lib()
    return _make_plan("ar_all_gather_init",
                      lambda h: L.ar_all_gather_init(sp, rp, count, _lib.DTYPES[dtype], len(sendbufs),
                                                     _lib.ALGOS[algo], wp, wb, h),
                      dev, (list(sendbufs), list(recvbufs), workspace))


def ar_plan_start(plan: Plan, stream=None):
    """Enqueue a persistent collective's kernels (same as ``plan.start``)."""
    plan.start(stream)


def ar_plan_num_launches(plan: Plan) -> int:
    """Kernel launches one start of the plan enqueues (same as ``plan.num_launches``)."""
    return plan.num_launches


def ar_plan_algo(plan: Plan) -> str:
    """The algorithm a persistent collective runs, by name (same as ``plan.algo``)."""
    return plan.algo


def ar_plan_free(plan: Plan):
    """Release a persistent collective (same as ``plan.close``)."""
    plan.close()


def ar_plan_limit_blocks(plan: Plan, max_blocks: int):
    """Cap the workgroups of a plan's launches (same as ``plan.limit_blocks``)."""
    plan.limit_blocks(max_blocks)
