"""The C-ABI library loads, exports every declared symbol, and its host-side
logic (validation, bucket planning) behaves as documented.  No GPU work."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dt.h")


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dt_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("dt_allreduce", "dt_reduce_scatter", "dt_all_gather", "dt_all_to_all",
                     "dt_bucket_allreduce", "dt_barrier", "dt_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(dt):
    lib = ctypes.CDLL(dt.LIBRARY_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    from collective_communication_primitives_amd import _lib
    assert sorted(_lib.EXPORTS) == declared_functions()


def test_status_strings_and_version(dt):
    assert dt.status_string(0) == "DT_OK"
    assert "TIMEOUT" in dt.status_string(4)
    assert "gfx950" in dt.version()


def _raw():
    from collective_communication_primitives_amd import _lib
    return _lib.load()


def test_validation_rejects_bad_rank_counts():
    lib = _raw()
    ptrs = (ctypes.c_void_p * 17)(*([0x1000] * 17))
    for n in (0, -1, 17):
        assert lib.dt_allreduce(ptrs, ptrs, n, 0, 0, 0, None) == 1
        assert lib.dt_reduce_scatter(ptrs, ptrs, n, 0, 0, 0, None) == 1
        assert lib.dt_all_gather(ptrs, ptrs, n, None, 0, 0, None) == 1
    assert b"nranks" in lib.dt_last_error()


def test_validation_rejects_bad_enums_nulls_and_aliases():
    lib = _raw()
    a = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    b = (ctypes.c_void_p * 2)(0x3000, 0x4000)
    assert lib.dt_allreduce(a, b, 2, 0, 7, 0, None) == 1           # dtype
    assert lib.dt_allreduce(a, b, 2, 0, 0, 9, None) == 1           # op
    assert lib.dt_allreduce(None, b, 2, 0, 0, 0, None) == 1        # NULL array
    nul = (ctypes.c_void_p * 2)(0x1000, 0)
    assert lib.dt_allreduce(nul, b, 2, 8, 0, 0, None) == 1         # NULL entry
    assert lib.dt_allreduce(nul, b, 2, 0, 0, 0, None) == 0         # ... allowed when empty
    crossed = (ctypes.c_void_p * 2)(0x2000, 0x1000)
    assert lib.dt_allreduce(a, crossed, 2, 8, 0, 0, None) == 1     # recv[0] aliases send[1]
    assert lib.dt_allreduce(a, a, 2, 0, 0, 0, None) == 0           # in place, count 0: no-op
    assert lib.dt_reduce_scatter(a, a, 2, 8, 0, 0, None) == 1      # RS may not alias
    same = (ctypes.c_void_p * 2)(0x3000, 0x3000)
    assert lib.dt_allreduce(a, same, 2, 8, 0, 0, None) == 1        # two ranks share one output
    counts = (ctypes.c_size_t * 2)(0, 4)
    nul0 = (ctypes.c_void_p * 2)(0, 0x1000)
    assert lib.dt_all_gather(nul0, (ctypes.c_void_p * 2)(0, 0x9000), 2, counts, 0, 0, None) == 1  # recv NULL
    splits = (ctypes.c_size_t * 4)(0, 0, 0, 3)
    assert lib.dt_all_to_all(nul0, (ctypes.c_void_p * 2)(0x8000, 0), 2, splits, 0, None) == 1  # recv[1] gets data
    assert lib.dt_all_to_all(a, b, 2, None, 0, None) == 1          # NULL splits
    assert lib.dt_bucket_allreduce(a, None, 1, 2, 16, None, 0, 0, None) == 1
    sizes = (ctypes.c_size_t * 1)(4)
    assert lib.dt_bucket_allreduce(a, sizes, 1, 2, 24, None, 0, 0, None) == 1  # not a multiple of 16
    assert lib.dt_barrier(None, 2, 1, 1, None, 0, 0, None) == 1
    w = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert lib.dt_barrier(w, 2, 0, 1, ctypes.c_void_p(0x5000), 0, 0, None) == 1   # generation must be >= 1
    assert lib.dt_barrier(w, 2, 1, 1, ctypes.c_void_p(0x5000), 0, 7, None) == 1   # bad layout
    assert lib.dt_barrier(w, 2, 1, 0, ctypes.c_void_p(0x5000), 0, 0, None) == 0   # zero generations: no-op


def test_all_gather_rejects_overlapping_output():
    lib = _raw()
    # send[1] points into recv[0] at a slot that is not rank 1's own
    recv = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    send = (ctypes.c_void_p * 2)(0x30000, 0x10000)
    counts = (ctypes.c_size_t * 2)(4, 4)
    assert lib.dt_all_gather(send, recv, 2, counts, 0, 0, None) == 1


def _plan(dt, numels, es, bb):
    pieces, nb = dt.dt_bucket_plan(numels, es, bb)
    return pieces, nb


@pytest.mark.parametrize("numels,es,bb", [
    ([17, 1, 40, 3, 0, 64], 2, 32),
    ([1000] * 7, 4, 4096),
    ([4096 * 4096] * 4 + [11008 * 4096] * 2 + [4096 * 11008] + [4096] * 2, 2, 25 << 20),
    ([5], 4, 4),
    ([], 2, 16),
])
def test_bucket_plan_covers_every_element_once(dt, numels, es, bb):
    pieces, nb = _plan(dt, numels, es, bb)
    per = bb // es
    total = sum(numels)
    assert nb == (total + per - 1) // per
    covered = {t: np.zeros(n, dtype=np.int32) for t, n in enumerate(numels)}
    flat_pos = np.cumsum([0] + numels)
    bucket_fill = {}
    for p in pieces:
        assert p["length"] > 0
        covered[p["tensor"]][p["offset"]:p["offset"] + p["length"]] += 1
        # the piece's place in the flat concatenation agrees with its bucket position
        g = flat_pos[p["tensor"]] + p["offset"]
        assert g == p["bucket"] * per + p["bucket_pos"]
        assert p["bucket_pos"] + p["length"] <= per
        bucket_fill[p["bucket"]] = bucket_fill.get(p["bucket"], 0) + p["length"]
    for t, c in covered.items():
        assert (c == 1).all(), t
    for b, n in bucket_fill.items():
        assert n == min(per, total - b * per)


def test_bucket_plan_rejects_tiny_buckets(dt):
    with pytest.raises(dt.DtError):
        dt.dt_bucket_plan([4], 4, 2)
