"""GPU: the signal-window barrier against the oracle's window model, the
barrier-ordered exchange golden y[r] = x[(r+1) % P], and the bounded wait."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


def windows(p):
    return [torch.zeros(p, dtype=torch.int32, device="cuda") for _ in range(p)]


def window_matrix(ws):
    return np.stack([w.cpu().numpy() for w in ws])


@pytest.mark.parametrize("layout", ["packed", "spread"])
@pytest.mark.parametrize("p", [1, 2, 3, 8, 16])
def test_barrier_rows_after_generations(dt, p, layout):
    """After G generations every rank's row reads G except its own 0 -- the
    oracle's window model run on the same generations."""
    orc = oracle.get()
    ws = windows(p)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    note(f"barrier P={p} {layout} 1000 generations in one launch")
    dt.dt_barrier(ws, status, first_generation=1, generations=1000, layout=layout)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    model = np.zeros((p, p), np.int32)
    assert orc.barrier(model, 1, 1000) == 1000
    assert np.array_equal(window_matrix(ws), model)
    note(f"barrier P={p} {layout} 100 single-generation launches")
    for g in range(1001, 1101):
        dt.dt_barrier(ws, status, first_generation=g, generations=1, layout=layout)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    orc.barrier(model, 1001, 100)
    assert np.array_equal(window_matrix(ws), model)


def test_barrier_golden_two_ranks(dt):
    """The printed pattern: after one barrier rank r's row is 1 except its own 0."""
    ws = windows(2)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    note("barrier golden P=2")
    dt.dt_barrier(ws, status, 1, 1)
    torch.cuda.synchronize()
    assert window_matrix(ws).tolist() == [[0, 1], [1, 0]]


@pytest.mark.parametrize("layout", ["packed", "spread"])
def test_barrier_unreachable_generation_times_out(dt, layout):
    """A threshold two generations ahead can never be met: the bounded wait
    must give up, report DT_ERR_TIMEOUT in the status word, and exit."""
    p = 4
    ws = windows(p)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dt.dt_barrier(ws, status, 1, 3, layout=layout)
    torch.cuda.synchronize()
    note(f"barrier forced timeout {layout} (threshold unreachable, 20 ms budget)")
    dt.dt_barrier(ws, status, first_generation=6, generations=1, timeout_ns=20_000_000, layout=layout)
    torch.cuda.synchronize()
    assert int(status.item()) == dt.DT_ERR_TIMEOUT
    # each rank still notified once: the windows read 4 off the diagonal
    want = np.full((p, p), 4, np.int32)
    np.fill_diagonal(want, 0)
    assert np.array_equal(window_matrix(ws), want)


@pytest.mark.parametrize("layout", ["packed", "spread"])
@pytest.mark.parametrize("p,nbytes", [(2, 64), (5, 4099), (16, 1 << 20)])
def test_barrier_exchange_golden(dt, p, nbytes, layout):
    orc = oracle.get()
    n = nbytes // 4 if nbytes % 4 == 0 else nbytes
    dtype = torch.int32 if nbytes % 4 == 0 else torch.uint8
    src = [torch.randint(0, 100, (n,), dtype=torch.int64, device="cuda").to(dtype) + 0 for _ in range(p)]
    stage = [torch.zeros_like(s) for s in src]
    dst = [torch.full_like(s, 77) for s in src]
    ws = windows(p)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    note(f"barrier exchange {layout} P={p} bytes={nbytes}")
    for g in (1, 2, 3):
        dt.dt_barrier_exchange(src, stage, dst, ws, status, generation=g, layout=layout)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        want = orc.barrier_exchange([s.cpu().numpy() for s in src])
        for r in range(p):
            assert np.array_equal(dst[r].cpu().numpy(), want[r]), (g, r)
        src = [s.roll(1) for s in src]  # new data each generation
