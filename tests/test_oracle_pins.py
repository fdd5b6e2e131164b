"""The CPU oracle against its pins (no GPU): the plain build, and the
OpenMP build of the same source that the CPU timing uses, which must pass
the same pins and give the plain build's bytes."""
import os

import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.fixture(scope="module")
def orc_omp():
    oracle.build_omp()
    return oracle.Oracle(oracle.LIBRARY_OMP)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_openmp_build(orc_omp, pin):
    pin(orc_omp)


def _inputs(kind, p, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "f32":
        return [rng.uniform(-1, 1, n).astype(np.float32) for _ in range(p)]
    if kind == "bf16":
        return [(rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for _ in range(p)]
    return [rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32) for _ in range(p)]


@pytest.mark.parametrize("kind", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("op", ["sum", "max", "avg"])
@pytest.mark.parametrize("p", [3, 8])
def test_openmp_build_gives_the_same_bytes(orc, orc_omp, kind, op, p):
    if (os.cpu_count() or 1) > 1:
        assert orc_omp.threads() > 1
    assert orc.threads() == 1
    n = p * 100_003
    xs = _inputs(kind, p, n, seed=p * 10 + len(op))
    for a, b in zip(orc.allreduce(xs, op), orc_omp.allreduce(xs, op)):
        assert a.tobytes() == b.tobytes()
    rs_a, rs_b = orc.reduce_scatter(xs, op), orc_omp.reduce_scatter(xs, op)
    for a, b in zip(rs_a, rs_b):
        assert a.tobytes() == b.tobytes()
    uneven = [x[: (i * 7919) % len(x)] for i, x in enumerate(xs)]
    for a, b in zip(orc.all_gather(uneven), orc_omp.all_gather(uneven)):
        assert a.tobytes() == b.tobytes()


@pytest.mark.skipif(not os.environ.get("DT_SLOW_PINS"), reason="five-minute exhaustive sweep; set DT_SLOW_PINS=1")
def test_bf16_exhaustive(orc):
    pins.pin_bf16_exhaustive(orc)
