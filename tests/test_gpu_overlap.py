"""GPU: an async AllReduce on a side stream running beside a GEMM on the
compute stream (the overlap setting of the c10d page, sec. 6) produces the
oracle's result, and the GEMM's result is unchanged by the concurrency."""
import pytest
import torch

import oracle
import synth
from gpu_util import compare, note, to_np

pytestmark = pytest.mark.gpu


def test_allreduce_beside_gemm():
    import collective_communication_primitives_amd as dt
    p, n = 8, synth.BUCKET_BYTES // 4
    xs = synth.uniform_ranks(p, n, seed=4, device="cuda")
    ys = [torch.empty_like(x) for x in xs]
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    c_alone = torch.matmul(a, b)
    torch.cuda.synchronize()
    note("allreduce async on a side stream beside a GEMM")
    for _ in range(3):
        w = dt.dt_allreduce(xs, ys, async_op=True)
        c = torch.matmul(a, b)
        w.wait()
        torch.cuda.synchronize()
        assert torch.equal(c, c_alone)
        want = oracle.get().allreduce([to_np(x) for x in xs], "sum")
        for q in range(p):
            compare(to_np(ys[q]), want[q], f"rank {q}")
