"""ctypes loader for libdtcoll.so (the C ABI of include/dt.h).

There is no fallback: if the library is not built, importing the package
raises, so nothing can silently run on another path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libdtcoll.so")

# Every function declared in include/dt.h.
EXPORTS = (
    "dt_allreduce", "dt_reduce_scatter", "dt_all_gather", "dt_all_to_all", "dt_bucket_allreduce",
    "dt_all_gather_into_vec", "dt_broadcast", "dt_replicate_to_shard", "dt_all_to_all_dims",
    "dt_allreduce_coalesced", "dt_bucket_allreduce_noalloc",
    "dt_barrier", "dt_barrier_exchange", "dt_bucket_plan", "dt_work_begin", "dt_work_end",
    "dt_work_wait", "dt_work_query", "dt_work_free", "dt_hsdp_create", "dt_hsdp_post_backward",
    "dt_hsdp_finish", "dt_hsdp_destroy", "dt_status_string", "dt_last_error", "dt_version",
)


class DtPiece(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("bucket", ctypes.c_int32), ("offset", ctypes.c_size_t),
                ("length", ctypes.c_size_t), ("bucket_pos", ctypes.c_size_t)]


def load(path: str = LIBRARY) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python collective_communication_primitives_amd/build.py` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, sz, i32, u64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint64
    sig = {
        "dt_allreduce": [vp, vp, i32, sz, i32, i32, vp],
        "dt_reduce_scatter": [vp, vp, i32, sz, i32, i32, vp],
        "dt_all_gather": [vp, vp, i32, vp, sz, i32, vp],
        "dt_all_to_all": [vp, vp, i32, vp, i32, vp],
        "dt_all_gather_into_vec": [vp, vp, i32, vp, sz, i32, vp],
        "dt_broadcast": [vp, vp, i32, sz, i32, vp],
        "dt_replicate_to_shard": [vp, vp, i32, sz, i32, vp],
        "dt_all_to_all_dims": [vp, vp, i32, sz, sz, i32, i32, i32, vp],
        "dt_bucket_allreduce": [vp, vp, i32, i32, sz, vp, i32, i32, vp],
        "dt_allreduce_coalesced": [vp, vp, i32, i32, i32, i32, vp],
        "dt_bucket_allreduce_noalloc": [vp, vp, i32, i32, sz, i32, i32, vp],
        "dt_barrier": [vp, i32, ctypes.c_int32, ctypes.c_int32, vp, u64, i32, vp],
        "dt_barrier_exchange": [vp, vp, vp, sz, vp, i32, ctypes.c_int32, vp, u64, i32, vp],
        "dt_bucket_plan": [vp, i32, sz, sz, vp, sz, vp, vp],
        "dt_work_begin": [vp, vp, vp],
        "dt_work_end": [vp, vp],
        "dt_work_wait": [vp, vp],
        "dt_work_query": [vp],
        "dt_work_free": [vp],
        "dt_hsdp_create": [i32, i32, sz, i32, i32, vp, vp, vp],
        "dt_hsdp_post_backward": [vp, vp, vp, i32, vp, vp],
        "dt_hsdp_finish": [vp, vp],
        "dt_hsdp_destroy": [vp],
        "dt_status_string": [i32],
        "dt_last_error": [],
        "dt_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("dt_status_string", "dt_last_error", "dt_version") else ctypes.c_int
    return lib
