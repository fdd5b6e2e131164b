"""CPU oracle for the same-device collective primitives -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and this
package never imports the library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain single-threaded loops, one function
per primitive, each citing the page passage it follows).  This module only
marshals numpy arrays through ctypes.

Element types are taken from the numpy dtype: ``float32`` -> fp32,
``uint16`` -> bf16 bit patterns, ``int32`` -> int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")
# The same source built with -fopenmp: the all-cores leg of the CPU timing.
LIBRARY_OMP = os.path.join(HERE, "liboracle_omp.so")

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra"]

FLOAT32, BFLOAT16, INT32 = 0, 1, 2
SUM, MAX, MIN, AVG = 0, 1, 2, 3
OPS = {"sum": SUM, "max": MAX, "min": MIN, "avg": AVG}


def build(source: str = SOURCE, output: str = LIBRARY, extra: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc (no GPU, no HIP)."""
    cmd = ["gcc", *GCC_FLAGS, *extra, "-o", output + ".tmp", source]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def build_omp() -> str:
    """The OpenMP build of the same source (all host cores, same bits)."""
    return build(output=LIBRARY_OMP, extra=["-fopenmp"])


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return FLOAT32
    if a.dtype == np.uint16:
        return BFLOAT16
    if a.dtype == np.int32:
        return INT32
    raise TypeError(f"oracle: unsupported element type {a.dtype}")


def _op_code(op) -> int:
    return OPS[op] if isinstance(op, str) else int(op)


def _ptrs(arrays: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * max(1, len(arrays)))()
    for i, a in enumerate(arrays):
        assert a.flags["C_CONTIGUOUS"]
        arr[i] = a.ctypes.data
    return arr


def _sizes(values: Sequence[int]):
    arr = (ctypes.c_size_t * max(1, len(values)))()
    for i, v in enumerate(values):
        arr[i] = int(v)
    return arr


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Optional[str] = None):
        if path is None:
            path = LIBRARY
            if not os.path.exists(path):
                build()
        self.path = path
        lib = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_float_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_float_to_bf16.restype = ctypes.c_uint16
        lib.oracle_float_to_bf16_array.argtypes = [vp, vp, sz]
        lib.oracle_allreduce.argtypes = [vp, vp, i32, sz, i32, i32]
        lib.oracle_reduce_scatter.argtypes = [vp, vp, i32, sz, i32, i32]
        lib.oracle_all_gather.argtypes = [vp, vp, i32, vp, sz]
        lib.oracle_all_to_all.argtypes = [vp, vp, i32, vp, sz]
        lib.oracle_bucket_allreduce.argtypes = [vp, vp, i32, i32, sz, vp, i32, i32]
        lib.oracle_hsdp_layer.argtypes = [vp, vp, vp, i32, i32, i32, sz, vp, i32, i32]
        lib.oracle_broadcast.argtypes = [vp, vp, i32, sz]
        lib.oracle_replicate_to_shard.argtypes = [vp, vp, i32, sz, sz]
        lib.oracle_all_gather_into_vec.argtypes = [vp, vp, i32, vp, sz]
        lib.oracle_all_to_all_dims.argtypes = [vp, vp, i32, sz, sz, i32, i32, sz]
        lib.oracle_barrier.argtypes = [vp, i32, i32, i32]
        lib.oracle_barrier_exchange.argtypes = [vp, vp, i32, sz]
        for name in ("oracle_allreduce", "oracle_reduce_scatter", "oracle_all_gather",
                     "oracle_all_to_all", "oracle_bucket_allreduce", "oracle_hsdp_layer",
                     "oracle_barrier", "oracle_barrier_exchange", "oracle_broadcast", "oracle_replicate_to_shard",
                     "oracle_all_gather_into_vec", "oracle_all_to_all_dims"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib

    def threads(self) -> int:
        """Threads of the parallel loops: 1 unless this is the OpenMP build."""
        return int(self.lib.oracle_threads())

    # -- conversions ------------------------------------------------------
    def float_to_bf16(self, values: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(values, dtype=np.float32)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_float_to_bf16_array(v.ctypes.data, out.ctypes.data, v.size)
        return out

    # -- reductions -------------------------------------------------------
    def allreduce(self, xs: Sequence[np.ndarray], op="sum") -> List[np.ndarray]:
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        n = xs[0].size
        assert all(x.size == n and x.dtype == xs[0].dtype for x in xs)
        ys = [np.empty_like(xs[0]) for _ in xs]
        rc = self.lib.oracle_allreduce(_ptrs(xs), _ptrs(ys), len(xs), n, _dtype_code(xs[0]), _op_code(op))
        assert rc == 0, rc
        return ys

    def reduce_scatter(self, xs: Sequence[np.ndarray], op="sum") -> List[np.ndarray]:
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        p = len(xs)
        assert xs[0].size % p == 0
        m = xs[0].size // p
        ys = [np.empty(m, dtype=xs[0].dtype) for _ in xs]
        rc = self.lib.oracle_reduce_scatter(_ptrs(xs), _ptrs(ys), p, m, _dtype_code(xs[0]), _op_code(op))
        assert rc == 0, rc
        return ys

    # -- copies -----------------------------------------------------------
    def all_gather(self, xs: Sequence[np.ndarray]) -> List[np.ndarray]:
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        counts = [x.size for x in xs]
        total = sum(counts)
        ys = [np.empty(total, dtype=xs[0].dtype) for _ in xs]
        rc = self.lib.oracle_all_gather(_ptrs(xs), _ptrs(ys), len(xs), _sizes(counts), xs[0].itemsize)
        assert rc == 0, rc
        return ys

    def all_to_all(self, xs: Sequence[np.ndarray], splits: np.ndarray) -> List[np.ndarray]:
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        p = len(xs)
        s = np.asarray(splits, dtype=np.int64).reshape(p, p)
        for i in range(p):
            assert xs[i].size == int(s[i].sum()), "row sum of splits must equal the sender's length"
        ys = [np.empty(int(s[:, j].sum()), dtype=xs[0].dtype) for j in range(p)]
        rc = self.lib.oracle_all_to_all(_ptrs(xs), _ptrs(ys), p, _sizes(s.reshape(-1).tolist()),
                                        xs[0].itemsize)
        assert rc == 0, rc
        return ys

    def broadcast(self, x_root: np.ndarray, nranks: int) -> List[np.ndarray]:
        x = np.ascontiguousarray(x_root).reshape(-1)
        ys = [np.empty_like(x) for _ in range(nranks)]
        assert self.lib.oracle_broadcast(x.ctypes.data, _ptrs(ys), nranks, x.nbytes) == 0
        return ys

    def replicate_to_shard(self, xs: Sequence[np.ndarray]) -> List[np.ndarray]:
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        p = len(xs)
        assert xs[0].size % p == 0
        m = xs[0].size // p
        ys = [np.empty(m, dtype=xs[0].dtype) for _ in xs]
        assert self.lib.oracle_replicate_to_shard(_ptrs(xs), _ptrs(ys), p, m, xs[0].itemsize) == 0
        return ys

    def all_gather_into_vec(self, xs: Sequence[np.ndarray]) -> List[List[np.ndarray]]:
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        p = len(xs)
        ys = [[np.empty_like(xs[r]) for r in range(p)] for _ in range(p)]
        flat = [t for row in ys for t in row]
        assert self.lib.oracle_all_gather_into_vec(_ptrs(xs), _ptrs(flat), p, _sizes([x.size for x in xs]),
                                                   xs[0].itemsize) == 0
        return ys

    def all_to_all_dims(self, xs: Sequence[np.ndarray], rows: int, cols: int, src_dim: int,
                        dst_dim: int) -> List[np.ndarray]:
        """xs[i]: rank i's block of the [rows, cols] tensor under Shard(src_dim);
        returns the blocks under Shard(dst_dim), flat."""
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        p = len(xs)
        n_out = (rows // p) * cols if dst_dim == 0 else rows * (cols // p)
        ys = [np.empty(n_out, dtype=xs[0].dtype) for _ in range(p)]
        rc = self.lib.oracle_all_to_all_dims(_ptrs(xs), _ptrs(ys), p, rows, cols, src_dim, dst_dim, xs[0].itemsize)
        assert rc == 0, rc
        return ys

    # -- fused gradient reductions ----------------------------------------
    def bucket_allreduce(self, grads: Sequence[Sequence[np.ndarray]], bucket_bytes: int,
                         op="sum") -> List[List[np.ndarray]]:
        """grads[r][t] -> reduced copies (inputs are not modified)."""
        p, t = len(grads), len(grads[0])
        work = [[np.ascontiguousarray(g).reshape(-1).copy() for g in rank] for rank in grads]
        numels = [g.size for g in work[0]]
        flat = [np.empty(max(1, sum(numels)), dtype=work[0][0].dtype) for _ in range(p)]
        flat_ptrs = _ptrs(flat)
        rc = self.lib.oracle_bucket_allreduce(_ptrs([g for rank in work for g in rank]), _sizes(numels), t, p,
                                              bucket_bytes, flat_ptrs, _dtype_code(work[0][0]), _op_code(op))
        assert rc == 0, rc
        return work

    def hsdp_layer(self, grads: Sequence[Sequence[np.ndarray]], replicate: int, shard: int,
                   bucket_bytes: int, op="sum") -> List[List[np.ndarray]]:
        """grads[r][t] (full gradients) -> out[r][t] (reduced dim-0 shards)."""
        p, t = len(grads), len(grads[0])
        assert p == replicate * shard
        gs = [[np.ascontiguousarray(g).reshape(-1) for g in rank] for rank in grads]
        numels = [g.size for g in gs[0]]
        dt = gs[0][0].dtype
        out = [[np.empty(n // shard, dtype=dt) for n in numels] for _ in range(p)]
        work = [np.empty(max(1, sum(numels) // shard), dtype=dt) for _ in range(p)]
        rc = self.lib.oracle_hsdp_layer(_ptrs([g for rank in gs for g in rank]),
                                        _ptrs([o for rank in out for o in rank]), _sizes(numels), t,
                                        replicate, shard, bucket_bytes, _ptrs(work), _dtype_code(gs[0][0]),
                                        _op_code(op))
        assert rc == 0, rc
        return out

    # -- barrier ----------------------------------------------------------
    def barrier(self, window: np.ndarray, first_generation: int, generations: int) -> int:
        """window: int32 [P, P], updated in place. Returns generations passed."""
        assert window.dtype == np.int32 and window.flags["C_CONTIGUOUS"]
        p = window.shape[0]
        return self.lib.oracle_barrier(window.ctypes.data, p, first_generation, generations)

    def barrier_exchange(self, xs: Sequence[np.ndarray]) -> List[np.ndarray]:
        xs = [np.ascontiguousarray(x) for x in xs]
        ys = [np.empty_like(xs[0]) for _ in xs]
        rc = self.lib.oracle_barrier_exchange(_ptrs(xs), _ptrs(ys), len(xs), xs[0].nbytes)
        assert rc == 0, rc
        return ys


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` in this directory."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


_omp = None


def get_omp() -> Oracle:
    """The OpenMP build of the same oracle (built on first use)."""
    global _omp
    if _omp is None:
        if not os.path.exists(LIBRARY_OMP):
            build_omp()
        _omp = Oracle(LIBRARY_OMP)
    return _omp
