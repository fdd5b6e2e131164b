"""Same-device collective primitives for MI355X: Python binding of include/dt.h.

Every function here only marshals torch tensors into the C ABI of
libdtcoll.so (device pointers, element counts, dtype and op codes, the HIP
stream handle) and raises ``DtError`` on a non-OK status.  All data movement
runs in the library's HIP kernels; PyTorch supplies device memory and
streams.  There is no fallback path: if the library is missing, import fails.

Names follow the C ABI (``dt_allreduce`` ...).  Rank r's buffer is element r
of a list of tensors on the same GPU.  Calls are queued on ``stream``
(default: torch's current stream) and return before the GPU runs them.
With ``async_op=True`` the call follows the async mode of the c10d page
(arganzheng.life, "PyTorch communication stack", sec. 4.3-4.4): it is queued
on a side stream that first waits for the current stream, and the returned
``Work`` keeps the tensors alive until ``wait()`` makes the consumer stream
wait for the end event.
"""
from __future__ import annotations

import atexit
import ctypes
import threading
import weakref
from typing import Dict, List, Optional, Sequence

import torch

from . import _lib

_L = _lib.load()

DT_FLOAT32, DT_BFLOAT16, DT_INT32 = 0, 1, 2
DT_SUM, DT_MAX, DT_MIN, DT_AVG = 0, 1, 2, 3
DT_OK, DT_ERR_ARG, DT_ERR_UNSUPPORTED, DT_ERR_HIP, DT_ERR_TIMEOUT = 0, 1, 2, 3, 4
DT_MAX_RANKS = 16
DEFAULT_BUCKET_BYTES = 25 << 20
SCRATCH_BYTES = 256 << 20  # DT_SCRATCH_BYTES: the static staging buffer of dt_bucket_allreduce_noalloc

_DTYPES = {torch.float32: DT_FLOAT32, torch.bfloat16: DT_BFLOAT16, torch.int32: DT_INT32}
_OPS = {"sum": DT_SUM, "max": DT_MAX, "min": DT_MIN, "avg": DT_AVG}

LIBRARY_PATH = _lib.LIBRARY


class DtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} ({status})")
        self.status = status


def _check(status: int) -> None:
    if status != DT_OK:
        detail = _L.dt_last_error().decode() or _L.dt_status_string(status).decode()
        raise DtError(status, detail)


def status_string(status: int) -> str:
    return _L.dt_status_string(int(status)).decode()


def version() -> str:
    return _L.dt_version().decode()


def _ptr_array(tensors: Sequence[torch.Tensor]):
    return (ctypes.c_void_p * max(1, len(tensors)))(*[t.data_ptr() for t in tensors])


def _size_array(values: Sequence[int]):
    return (ctypes.c_size_t * max(1, len(values)))(*[int(v) for v in values])


def _dtype_code(tensors: Sequence[torch.Tensor]) -> int:
    """The tensors' common dtype code, after checking that every tensor is a
    contiguous tensor of that dtype on the current GPU (a host or
    other-device pointer must never reach a kernel)."""
    t0 = tensors[0]
    dt = t0.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    dev = torch.cuda.current_device()
    for t in tensors:
        if t.dtype != dt:
            raise TypeError("all rank tensors must share one dtype")
        if t.get_device() != dev:
            raise ValueError(f"rank tensors must live on the current GPU (cuda:{dev}), got {t.device}")
        if not t.is_contiguous():
            raise ValueError("rank tensors must be contiguous")
    return _DTYPES[dt]


def _on_gpu(tensors: Sequence[torch.Tensor], what: str) -> None:
    """Every tensor must be a contiguous tensor on the current GPU."""
    dev = torch.cuda.current_device()
    for t in tensors:
        if t.get_device() != dev or not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous tensors on the current GPU (cuda:{dev}), got {t.device}")


def _check_windows(windows: Sequence[torch.Tensor], status: torch.Tensor, p: int) -> None:
    for w in windows:
        if w.dtype != torch.int32 or w.numel() < p:
            raise ValueError("each window must be an int32 tensor of at least nranks cells")
    if status.dtype != torch.int32 or status.numel() < 1:
        raise ValueError("status must be an int32 device tensor")
    _on_gpu(list(windows) + [status], "windows and status")


def _op_code(op) -> int:
    return _OPS[op] if isinstance(op, str) else int(op)


if hasattr(torch._C, "_cuda_getCurrentRawStream") and hasattr(torch._C, "_cuda_getDevice"):
    def _current_stream_handle() -> int:
        # the raw handle without building a torch Stream object (about 2 us less per call)
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
else:  # other torch builds: the public accessor
    def _current_stream_handle() -> int:
        return torch.cuda.current_stream().cuda_stream


def _stream_handle(stream) -> int:
    if stream is None:
        return _current_stream_handle()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_side_streams: Dict[int, torch.cuda.Stream] = {}


def side_stream(device: Optional[int] = None) -> torch.cuda.Stream:
    """The library's default communication stream for a device (default priority)."""
    dev = torch.cuda.current_device() if device is None else device
    if dev not in _side_streams:
        _side_streams[dev] = torch.cuda.Stream(device=dev)
    return _side_streams[dev]


def join_streams(producers: Sequence[torch.cuda.Stream], stream=None) -> None:
    """User rule 4 of the c10d page (sec. 5): inputs computed on streams other
    than the current one must be joined into it before the collective is
    issued, because an async collective orders itself after the current
    stream only.  Makes ``stream`` (default: current) wait for everything
    queued so far on each producer stream; the host does not block."""
    target = torch.cuda.current_stream() if stream is None else stream
    for p in producers:
        if p is not None and p != target:
            target.wait_stream(p)


class Work:
    """Handle of an async collective: the start/end event pair plus the stash
    of tensors that must outlive the GPU work (released by ``wait``)."""

    def __init__(self, handle: ctypes.c_void_p, stash: List[torch.Tensor]):
        self._h = handle
        self._stash = stash
        self._lib = _L
        _live_works.add(self)

    def wait(self, stream=None) -> None:
        """Make ``stream`` (default: current) wait for the end event; the host does not block."""
        _check(self._lib.dt_work_wait(self._h, _stream_handle(stream)))
        self._stash = []

    def is_completed(self) -> bool:
        rc = self._lib.dt_work_query(self._h)
        if rc < 0:
            raise DtError(DT_ERR_HIP, _L.dt_last_error().decode())
        return rc == 1

    def _release(self) -> None:
        """Free the handle now (at exit): wait for the work first if its
        tensors are still held, so they are not released under it."""
        h = getattr(self, "_h", None)
        if h:
            if getattr(self, "_stash", None):
                torch.cuda.synchronize()
            self._lib.dt_work_free(h)
            self._h = None
            self._stash = []

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            if getattr(self, "_stash", None) and _shelf is not None:
                # dropped without wait(): shelve the tensors until the GPU is done
                _shelf.append((h, self._stash))
            else:
                self._lib.dt_work_free(h)
            self._h = None
            self._stash = []


# Works dropped without wait(): (handle, tensors).  As in the c10d page
# (sec. 4.4), a forgotten wait() leaks nothing but may not free the tensors
# while the collective can still touch them: they stay here until the work's
# end event has completed, and are released by the next collective call.
_shelf: List = []

# Every object of this module that owns HIP handles, so that _release_all
# can free them before the interpreter (and with it the HIP runtime and any
# profiler attached to it) shuts down.
_live_works: "weakref.WeakSet[Work]" = weakref.WeakSet()
_live_pipelines: "weakref.WeakSet[HSDPPipeline]" = weakref.WeakSet()


def _release_all() -> None:
    """Free every HIP event the binding still owns, deterministically, while
    the runtime is whole: live HSDP pipelines (their destroy waits for the
    work they queued), live and shelved works.  Registered with atexit at
    import; afterwards no destructor of this module calls into HIP.  The
    tensors a work or pipeline kept alive are dropped only after its handle
    has been released (the c10d page, sec. 5: a stash outlives its GPU work)."""
    for pipe in list(_live_pipelines):
        pipe.close()
    for work in list(_live_works):
        work._release()
    if _shelf:
        torch.cuda.synchronize()  # the shelved tensors may still be in use on the GPU
        for h, _stash in _shelf:
            _L.dt_work_free(h)
        _shelf.clear()


atexit.register(_release_all)


def _unshelve() -> None:
    keep = []
    for h, stash in _shelf:
        if _L.dt_work_query(h) == 0:
            keep.append((h, stash))
        else:
            _L.dt_work_free(h)
    _shelf[:] = keep


# prepare() runs a collective's validation and marshalling once and keeps the
# resulting launch instead of enqueuing it.
_preparing = threading.local()


class Prepared:
    """One collective bound to fixed buffers, counts, dtype and op (made by
    ``prepare``).  Each call enqueues it again on ``stream`` (default: the
    current stream) at the host cost of the C call alone: the pointer arrays
    and checks were done once.  The buffers stay referenced while this object
    lives; their contents may change between calls."""

    def __init__(self, fn, stash: List[torch.Tensor]):
        self._fn = fn
        self._stash = stash

    def __call__(self, stream=None) -> None:
        _check(self._fn(_stream_handle(stream)))


def prepare(collective, *args, **kwargs) -> Prepared:
    """Validate and marshal one call of ``collective`` (``dt_allreduce``,
    ``dt_reduce_scatter``, ...; same arguments, without ``async_op``) once,
    for loops that repeat the same collective on the same buffers."""
    if kwargs.get("async_op"):
        raise ValueError("prepare() binds a synchronous call; order it with streams and events")
    _preparing.active = True
    _preparing.result = None
    try:
        collective(*args, **kwargs)
        if _preparing.result is None:
            raise TypeError(f"{collective!r} does not enqueue a collective")
        fn, stash = _preparing.result
    finally:
        _preparing.active = False
        _preparing.result = None
    return Prepared(fn, stash)


def _launch(fn, stash, async_op: bool, stream, comm_stream):
    """Queue ``fn(stream_handle)`` either on ``stream`` or, for async_op, on a
    side stream ordered after the current stream."""
    if getattr(_preparing, "active", False):
        _preparing.result = (fn, list(stash))
        return None
    if _shelf:
        _unshelve()
    if not async_op:
        _check(fn(_stream_handle(stream)))
        return None
    producer = _stream_handle(stream)
    comm = _stream_handle(comm_stream if comm_stream is not None else side_stream())
    h = ctypes.c_void_p()
    _check(_L.dt_work_begin(producer, comm, ctypes.byref(h)))
    work = Work(h, list(stash))
    _check(fn(comm))
    _check(_L.dt_work_end(h, comm))
    return work


# ----------------------------------------------------------- collectives --
def dt_allreduce(send: Sequence[torch.Tensor], recv: Optional[Sequence[torch.Tensor]] = None, op="sum",
                 stream=None, async_op: bool = False, comm_stream=None):
    """AllReduce: recv[q] = fold over ranks of send[r] (in place when recv is None)."""
    recv = list(send) if recv is None else list(recv)
    n = send[0].numel()
    if any(t.numel() != n for t in list(send) + recv) or len(recv) != len(send):
        raise ValueError("every rank's send and recv must have the same number of elements")
    code = _dtype_code(list(send) + recv)
    s, r = _ptr_array(send), _ptr_array(recv)
    w = _launch(lambda st: _L.dt_allreduce(s, r, len(send), n, code, _op_code(op), st), list(send) + recv,
                async_op, stream, comm_stream)
    return w if async_op else recv


def dt_reduce_scatter(send: Sequence[torch.Tensor], recv: Sequence[torch.Tensor], op="sum", stream=None,
                      async_op: bool = False, comm_stream=None):
    """ReduceScatter: recv[r] = chunk r of the fold; send[r] holds P * recv[r].numel() elements."""
    p = len(send)
    m = recv[0].numel()
    if len(recv) != p or any(t.numel() != p * m for t in send) or any(t.numel() != m for t in recv):
        raise ValueError("send[r] must hold nranks * recvcount elements and recv[r] recvcount")
    code = _dtype_code(list(send) + list(recv))
    s, r = _ptr_array(send), _ptr_array(recv)
    w = _launch(lambda st: _L.dt_reduce_scatter(s, r, p, m, code, _op_code(op), st), list(send) + list(recv),
                async_op, stream, comm_stream)
    return w if async_op else list(recv)


def dt_all_gather(send: Sequence[torch.Tensor], recv: Sequence[torch.Tensor], stream=None,
                  async_op: bool = False, comm_stream=None):
    """AllGather (equal or uneven Shard(0)): recv[q] = concat(send[0], ..., send[P-1])."""
    p = len(send)
    counts = [t.numel() for t in send]
    total = sum(counts)
    if len(recv) != p or any(t.numel() != total for t in recv):
        raise ValueError("every recv must hold the sum of the send counts")
    code = _dtype_code(list(send) + list(recv))
    s, r = _ptr_array(send), _ptr_array(recv)
    equal = all(c == counts[0] for c in counts)
    c_arr = None if equal else _size_array(counts)
    w = _launch(lambda st: _L.dt_all_gather(s, r, p, c_arr, counts[0] if equal else 0, code, st),
                list(send) + list(recv), async_op, stream, comm_stream)
    return w if async_op else list(recv)


def dt_all_to_all(send: Sequence[torch.Tensor], recv: Sequence[torch.Tensor], splits, stream=None,
                  async_op: bool = False, comm_stream=None):
    """AllToAll with splits[i][j] elements from rank i to rank j (row-major P x P)."""
    p = len(send)
    flat = [int(v) for row in splits for v in row] if hasattr(splits[0], "__len__") else [int(v) for v in splits]
    if len(flat) != p * p:
        raise ValueError("splits must be P x P")
    for i in range(p):
        if send[i].numel() != sum(flat[i * p:(i + 1) * p]):
            raise ValueError(f"send[{i}] must hold the sum of row {i} of splits")
        if recv[i].numel() != sum(flat[j * p + i] for j in range(p)):
            raise ValueError(f"recv[{i}] must hold the sum of column {i} of splits")
    code = _dtype_code(list(send) + list(recv))
    s, r, sp = _ptr_array(send), _ptr_array(recv), _size_array(flat)
    w = _launch(lambda st: _L.dt_all_to_all(s, r, p, sp, code, st), list(send) + list(recv), async_op, stream,
                comm_stream)
    return w if async_op else list(recv)


def dt_all_gather_into_vec(send: Sequence[torch.Tensor], recv: Sequence[Sequence[torch.Tensor]], stream=None,
                           async_op: bool = False, comm_stream=None):
    """AllGatherIntoVec: recv[q][r] receives a copy of send[r] for every rank q."""
    p = len(send)
    if len(recv) != p or any(len(row) != p for row in recv):
        raise ValueError("recv must be P lists of P tensors")
    for q in range(p):
        for r in range(p):
            if recv[q][r].numel() != send[r].numel():
                raise ValueError(f"recv[{q}][{r}] must hold send[{r}].numel() elements")
    flat = [t for row in recv for t in row]
    code = _dtype_code(list(send) + flat)
    counts = [t.numel() for t in send]
    s, r, c = _ptr_array(send), _ptr_array(flat), _size_array(counts)
    w = _launch(lambda st: _L.dt_all_gather_into_vec(s, r, p, c, 0, code, st), list(send) + flat, async_op,
                stream, comm_stream)
    return w if async_op else recv


def dt_broadcast(root_send: torch.Tensor, recv: Sequence[torch.Tensor], stream=None, async_op: bool = False,
                 comm_stream=None):
    """Broadcast: every recv[q] receives a copy of root_send."""
    n = root_send.numel()
    if any(t.numel() != n for t in recv):
        raise ValueError("every recv must hold root_send.numel() elements")
    code = _dtype_code([root_send] + list(recv))
    r = _ptr_array(recv)
    w = _launch(lambda st: _L.dt_broadcast(root_send.data_ptr(), r, len(recv), n, code, st),
                [root_send] + list(recv), async_op, stream, comm_stream)
    return w if async_op else list(recv)


def dt_replicate_to_shard(send: Sequence[torch.Tensor], recv: Sequence[torch.Tensor], stream=None,
                          async_op: bool = False, comm_stream=None):
    """ReplicateToShard: recv[r] = slice r of send[r] (send[r] holds P * recv[r].numel())."""
    p = len(send)
    m = recv[0].numel()
    if len(recv) != p or any(t.numel() != p * m for t in send) or any(t.numel() != m for t in recv):
        raise ValueError("send[r] must hold nranks * recvcount elements and recv[r] recvcount")
    code = _dtype_code(list(send) + list(recv))
    s, r = _ptr_array(send), _ptr_array(recv)
    w = _launch(lambda st: _L.dt_replicate_to_shard(s, r, p, m, code, st), list(send) + list(recv), async_op,
                stream, comm_stream)
    return w if async_op else list(recv)


def dt_all_to_all_dims(send: Sequence[torch.Tensor], recv: Sequence[torch.Tensor], rows: int, cols: int,
                       src_dim: int, dst_dim: int, stream=None, async_op: bool = False, comm_stream=None):
    """AllToAll between shard dimensions of a [rows, cols] tensor: send[r] is
    rank r's block under Shard(src_dim), recv[r] its block under Shard(dst_dim)."""
    p = len(send)
    blk = {0: (rows // p) * cols, 1: rows * (cols // p)}
    if len(recv) != p or any(t.numel() != blk[src_dim] for t in send) or any(t.numel() != blk[dst_dim] for t in recv):
        raise ValueError("send/recv blocks do not match the [rows, cols] shard shapes")
    code = _dtype_code(list(send) + list(recv))
    s, r = _ptr_array(send), _ptr_array(recv)
    w = _launch(lambda st: _L.dt_all_to_all_dims(s, r, p, rows, cols, src_dim, dst_dim, code, st),
                list(send) + list(recv), async_op, stream, comm_stream)
    return w if async_op else list(recv)


def dt_bucket_allreduce(grads: Sequence[Sequence[torch.Tensor]], bucket_bytes: int = DEFAULT_BUCKET_BYTES,
                        bucket_ws: Optional[Sequence[torch.Tensor]] = None, op="sum", stream=None,
                        async_op: bool = False, comm_stream=None):
    """Fused-bucket AllReduce in place over grads[r][t] (rank r, tensor t).

    With ``bucket_ws`` (one device buffer of >= bucket_bytes per rank) each
    bucket is staged through it; without, buckets are reduced in place."""
    p, nt = len(grads), len(grads[0])
    numels = [g.numel() for g in grads[0]]
    for rank in grads:
        if len(rank) != nt or [g.numel() for g in rank] != numels:
            raise ValueError("every rank must list tensors of the same sizes")
    flat = [g for rank in grads for g in rank]
    code = _dtype_code(flat)
    if bucket_ws is not None:
        if len(bucket_ws) != p or any(w.numel() * w.element_size() < bucket_bytes for w in bucket_ws):
            raise ValueError("bucket_ws needs one buffer of at least bucket_bytes per rank")
        _on_gpu(bucket_ws, "bucket_ws")
    g_arr, n_arr = _ptr_array(flat), _size_array(numels)
    ws_arr = _ptr_array(bucket_ws) if bucket_ws is not None else None
    stash = flat + (list(bucket_ws) if bucket_ws is not None else [])
    w = _launch(lambda st: _L.dt_bucket_allreduce(g_arr, n_arr, nt, p, bucket_bytes, ws_arr, code, _op_code(op), st),
                stash, async_op, stream, comm_stream)
    return w if async_op else grads


def dt_bucket_allreduce_noalloc(grads: Sequence[Sequence[torch.Tensor]], bucket_bytes: int = DEFAULT_BUCKET_BYTES,
                                op="sum", stream=None, async_op: bool = False, comm_stream=None):
    """Staged fused-bucket AllReduce in place over grads[r][t], with the
    buckets staged in the library's static device buffer (SCRATCH_BYTES)
    instead of caller workspaces: nothing is allocated.  nranks *
    bucket_bytes must fit that buffer.  Calls that may overlap in time on one
    GPU share the buffer and must be ordered by the caller."""
    p, nt = len(grads), len(grads[0])
    numels = [g.numel() for g in grads[0]]
    for rank in grads:
        if len(rank) != nt or [g.numel() for g in rank] != numels:
            raise ValueError("every rank must list tensors of the same sizes")
    flat = [g for rank in grads for g in rank]
    code = _dtype_code(flat)
    g_arr, n_arr = _ptr_array(flat), _size_array(numels)
    w = _launch(lambda st: _L.dt_bucket_allreduce_noalloc(g_arr, n_arr, nt, p, bucket_bytes, code, _op_code(op), st),
                flat, async_op, stream, comm_stream)
    return w if async_op else grads


def dt_allreduce_coalesced(tensors: Sequence[Sequence[torch.Tensor]], op="sum", stream=None, async_op: bool = False,
                           comm_stream=None):
    """Coalesced in-place AllReduce of tensors[r][t] (rank r, tensor t): one
    launch for up to min(512, 4096 // P) tensors, no flattening."""
    p, nt = len(tensors), len(tensors[0])
    numels = [g.numel() for g in tensors[0]]
    for rank in tensors:
        if len(rank) != nt or [g.numel() for g in rank] != numels:
            raise ValueError("every rank must list tensors of the same sizes")
    flat = [g for rank in tensors for g in rank]
    code = _dtype_code(flat)
    g_arr, n_arr = _ptr_array(flat), _size_array(numels)
    w = _launch(lambda st: _L.dt_allreduce_coalesced(g_arr, n_arr, nt, p, code, _op_code(op), st), flat, async_op,
                stream, comm_stream)
    return w if async_op else tensors


def dt_bucket_plan(numels: Sequence[int], elem_size: int, bucket_bytes: int = DEFAULT_BUCKET_BYTES):
    """Host-side bucket plan: (pieces, nbuckets); each piece is a dict."""
    n_arr = _size_array(numels)
    npieces, nbuckets = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_L.dt_bucket_plan(n_arr, len(numels), elem_size, bucket_bytes, None, 0, ctypes.byref(npieces),
                             ctypes.byref(nbuckets)))
    buf = (_lib.DtPiece * max(1, npieces.value))()
    _check(_L.dt_bucket_plan(n_arr, len(numels), elem_size, bucket_bytes, buf, npieces.value,
                             ctypes.byref(npieces), ctypes.byref(nbuckets)))
    pieces = [dict(tensor=buf[i].tensor, bucket=buf[i].bucket, offset=buf[i].offset, length=buf[i].length,
                   bucket_pos=buf[i].bucket_pos) for i in range(npieces.value)]
    return pieces, nbuckets.value


# ------------------------------------------------------------------ barrier --
DT_BARRIER_PACKED, DT_BARRIER_SPREAD = 0, 1
_LAYOUTS = {"packed": DT_BARRIER_PACKED, "spread": DT_BARRIER_SPREAD}


def dt_barrier(windows: Sequence[torch.Tensor], status: torch.Tensor, first_generation: int, generations: int = 1,
               timeout_ns: int = 0, layout="packed", stream=None) -> None:
    """Signal-window barrier over int32 windows[p] (nranks cells each);
    layout "packed" (one workgroup, a wave per rank) or "spread" (a
    workgroup per rank, cooperative launch)."""
    p = len(windows)
    _check_windows(windows, status, p)
    w_arr = _ptr_array(windows)
    _check(_L.dt_barrier(w_arr, p, first_generation, generations, status.data_ptr(), timeout_ns, _LAYOUTS[layout],
                         _stream_handle(stream)))


def dt_barrier_exchange(src: Sequence[torch.Tensor], stage: Sequence[torch.Tensor], dst: Sequence[torch.Tensor],
                        windows: Sequence[torch.Tensor], status: torch.Tensor, generation: int, timeout_ns: int = 0,
                        layout="packed", stream=None) -> None:
    """Stage src[r], meet the barrier, then dst[r] = stage[(r+1) % P]."""
    p = len(src)
    nbytes = src[0].numel() * src[0].element_size()
    for group in (src, stage, dst):
        if len(group) != p or any(t.numel() * t.element_size() != nbytes for t in group):
            raise ValueError("src, stage and dst need one contiguous buffer of equal bytes per rank")
        _on_gpu(group, "src, stage and dst")
    if len(windows) != p:
        raise ValueError("one window per rank")
    _check_windows(windows, status, p)
    _check(_L.dt_barrier_exchange(_ptr_array(src), _ptr_array(stage), _ptr_array(dst), nbytes, _ptr_array(windows),
                                  p, generation, status.data_ptr(), timeout_ns, _LAYOUTS[layout],
                                  _stream_handle(stream)))


# -------------------------------------------------------------- HSDP -------
class HSDPPipeline:
    """Per-layer ReduceScatter -> fused AllReduce pipeline (dt_hsdp_*).

    The two phases may run on two streams (the page's layout: the
    AllReduce of layer L-1 never blocks the ReduceScatter of layer L) or on
    one.  With every rank on one device both phases draw on the same HBM, and
    issuing them back to back on one stream, in the same order, measured 4%
    faster (30.5 vs 31.8 ms for the 32-layer workload), so one side stream
    for both is the default; pass two streams for the split layout, or the
    stream that produces the gradients as both, for a pipeline without
    cross-stream events (its collectives then queue behind the producer's
    work, in order).

    A layer's fused buffers must not be passed again (as the next layer's)
    before ``finish()``: the previous layer's AllReduce is still pending on
    them, and the library refuses the overlap."""

    def __init__(self, replicate: int, shard: int, bucket_bytes: int = DEFAULT_BUCKET_BYTES,
                 dtype=torch.bfloat16, op="sum", rs_stream=None, ar_stream=None):
        self.replicate, self.shard = replicate, shard
        if rs_stream is None and ar_stream is None:
            rs_stream = ar_stream = torch.cuda.Stream()
        self.rs_stream = rs_stream if rs_stream is not None else torch.cuda.Stream()
        self.ar_stream = ar_stream if ar_stream is not None else torch.cuda.Stream()
        self._h = ctypes.c_void_p()
        self._stash: List[torch.Tensor] = []
        self._lib = _L
        _check(_L.dt_hsdp_create(replicate, shard, bucket_bytes, _DTYPES[dtype], _op_code(op),
                                 _stream_handle(self.rs_stream), _stream_handle(self.ar_stream),
                                 ctypes.byref(self._h)))
        _live_pipelines.add(self)

    def post_backward(self, grads: Sequence[Sequence[torch.Tensor]], fused: Sequence[torch.Tensor],
                      producer=None) -> None:
        """grads[r][t]: rank r's full gradients of one layer; fused[r]: its
        flat shard buffer (sum(numel)/shard elements)."""
        p = self.replicate * self.shard
        nt = len(grads[0])
        numels = [g.numel() for g in grads[0]]
        flat = [g for rank in grads for g in rank]
        _dtype_code(flat + list(fused))
        if len(grads) != p or len(fused) != p:
            raise ValueError("one gradient list and one fused buffer per rank")
        if any(f.numel() != sum(numels) // self.shard for f in fused):
            raise ValueError("fused[r] must hold sum(numels) / shard elements")
        self._stash.extend(flat + list(fused))
        _check(self._lib.dt_hsdp_post_backward(self._h, _ptr_array(flat), _size_array(numels), nt, _ptr_array(fused),
                                        _stream_handle(producer)))

    def finish(self, consumer=None) -> None:
        _check(self._lib.dt_hsdp_finish(self._h, _stream_handle(consumer)))
        self._stash = []

    def close(self) -> None:
        """Release the handle: the library waits for the work it queued to
        stop writing the buffers, then the buffers are let go.  A layer
        posted without finish() gets no AllReduce."""
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.dt_hsdp_destroy(h)
        self._h = None
        self._stash = []

    def __del__(self):
        self.close()


def shard_views(fused: torch.Tensor, numels: Sequence[int], shard: int) -> List[torch.Tensor]:
    """Each parameter's reduced shard as a view of a fused buffer (the page's
    get_param_grad_view): no copy."""
    out, at = [], 0
    for n in numels:
        m = n // shard
        out.append(fused[at:at + m])
        at += m
    return out


__all__ = [
    "dt_allreduce", "dt_reduce_scatter", "dt_all_gather", "dt_all_to_all", "dt_bucket_allreduce", "dt_bucket_plan",
    "dt_all_gather_into_vec", "dt_broadcast", "dt_replicate_to_shard", "dt_all_to_all_dims",
    "dt_allreduce_coalesced", "dt_bucket_allreduce_noalloc", "dt_barrier", "dt_barrier_exchange", "HSDPPipeline", "Work", "DtError", "shard_views", "side_stream",
    "status_string", "version",
]
