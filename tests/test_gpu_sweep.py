"""GPU parity across the message-size sweep: fp32 AllReduce, P=16, per-rank
sizes 4 KiB .. 1 GiB in powers of 4, values U[-1,1).  Every element of rank
0's output is compared with the oracle (its OpenMP build, whose bytes equal
the single-threaded build's), slice by slice of at most 64 Mi elements (an
AllReduce is element-wise, so the oracle over a slice is the definition
over that slice), and every other rank's output is checked on the device to
be byte-identical to rank 0's."""
import pytest
import torch

import oracle
import synth
from gpu_util import compare, note, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


@pytest.mark.parametrize("nbytes", synth.SWEEP_BYTES)
def test_sweep_point(dt, nbytes):
    p, n = 16, nbytes // 4
    note(f"sweep allreduce P=16 fp32 bytes/rank={nbytes}")
    xs = synth.uniform_ranks(p, n, seed=0, device="cuda")
    ys = [torch.empty_like(x) for x in xs]
    dt.dt_allreduce(xs, ys)
    torch.cuda.synchronize()
    orc_omp = oracle.get_omp()
    step = 1 << 26
    for a in range(0, n, step):
        b = min(n, a + step)
        want = orc_omp.allreduce([to_np(x[a:b]) for x in xs], "sum")[0]
        compare(to_np(ys[0][a:b]), want, f"rank 0 elements [{a}, {b})")
    for q in range(1, p):
        assert torch.equal(ys[q].view(torch.int32), ys[0].view(torch.int32)), q
    del xs, ys
    torch.cuda.empty_cache()
