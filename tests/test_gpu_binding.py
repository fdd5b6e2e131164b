"""GPU: the binding refuses tensors a kernel must never see -- host tensors,
non-contiguous views, mixed dtypes, windows off the device -- before any
pointer reaches the C ABI."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


def test_host_tensor_is_refused(dt):
    xs = [torch.ones(64, device="cuda"), torch.ones(64)]
    with pytest.raises(ValueError):
        dt.dt_allreduce(xs, [torch.empty(64, device="cuda") for _ in range(2)])
    with pytest.raises(ValueError):
        dt.dt_all_gather([torch.ones(8, device="cuda")] * 2, [torch.empty(16), torch.empty(16, device="cuda")])
    with pytest.raises(ValueError):
        dt.dt_bucket_allreduce([[torch.ones(8, device="cuda")]] * 2, bucket_bytes=64, bucket_ws=[torch.empty(64)] * 2)


def test_non_contiguous_and_mixed_dtypes_are_refused(dt):
    base = torch.ones(8, 8, device="cuda")
    with pytest.raises(ValueError):
        dt.dt_allreduce([base.t(), base.t().clone()])  # a transposed view is not contiguous
    with pytest.raises(TypeError):
        dt.dt_allreduce([torch.ones(8, device="cuda"), torch.ones(8, device="cuda", dtype=torch.int32)])


def test_barrier_windows_on_the_host_are_refused(dt):
    windows = [torch.zeros(2, dtype=torch.int32, device="cuda"), torch.zeros(2, dtype=torch.int32)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dt.dt_barrier(windows, status, 1)
    with pytest.raises(ValueError):
        dt.dt_barrier([w.cuda() for w in windows], torch.zeros(1, dtype=torch.int32), 1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_prepared_calls_follow_the_buffers(dt):
    """prepare() marshals once; every call enqueues the same collective on the
    current buffers' contents, on any stream, and matches the oracle."""
    import oracle
    import synth
    from gpu_util import compare, note, to_np
    orc = oracle.get()
    p, n = 8, 8 * 1001
    note("prepared allreduce / reduce_scatter / all_gather")
    xs = synth.uniform_ranks(p, n, seed=11, device="cuda")
    ys = [torch.empty_like(x) for x in xs]
    shards = [torch.empty(n // p, device="cuda") for _ in range(p)]
    full = [torch.empty(n, device="cuda") for _ in range(p)]
    ar = dt.prepare(dt.dt_allreduce, xs, ys, op="max")
    rs = dt.prepare(dt.dt_reduce_scatter, xs, shards)
    ag = dt.prepare(dt.dt_all_gather, shards, full)
    side = torch.cuda.Stream()
    for it in range(3):
        for x, v in zip(xs, synth.uniform_ranks(p, n, seed=20 + it, device="cuda")):
            x.copy_(v)                          # new contents, same buffers
        ar()
        side.wait_stream(torch.cuda.current_stream())
        rs(stream=side)
        ag(stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        host = [to_np(x) for x in xs]
        want_ar = orc.allreduce(host, "max")
        want_rs = orc.reduce_scatter(host, "sum")
        cat = np.concatenate(want_rs)
        for q in range(p):
            compare(to_np(ys[q]), want_ar[q], f"pass {it} AR rank {q}")
            compare(to_np(shards[q]), want_rs[q], f"pass {it} RS rank {q}")
            compare(to_np(full[q]), cat, f"pass {it} AG rank {q}")
    with pytest.raises(ValueError):
        dt.prepare(dt.dt_allreduce, xs, ys, async_op=True)


def test_overlapping_views_are_refused(dt):
    """Outputs that partly overlap another output or an input would race
    between workgroups: the library refuses them before any launch, and
    leaves the buffers untouched."""
    base = torch.zeros(6 * 1024, device="cuda")
    xs = [base[0:1024], base[1024:2048]]
    with pytest.raises(dt.DtError):
        dt.dt_allreduce(xs, [base[2048:3072], base[2560:3584]])       # recv[1] inside recv[0]
    with pytest.raises(dt.DtError):
        dt.dt_allreduce(xs, [base[512:1536], base[4096:5120]])        # recv[0] over send[0] and send[1]
    with pytest.raises(dt.DtError):
        dt.dt_reduce_scatter([base[0:2048], base[2048:4096]], [base[4096:5120], base[3072:4096]])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(base).item()) == 0
    # exact in place stays allowed
    ys = dt.dt_allreduce([base[0:1024] + 1, base[1024:2048] + 2])
    torch.cuda.synchronize()
    assert torch.all(ys[0] == 3).item() and torch.all(ys[1] == 3).item()


def test_exit_releases_handles_before_teardown():
    """At interpreter exit the binding frees every HIP handle it still owns
    (a pipeline with a layer posted but never finished, a work still held, a
    work dropped without wait()) from an atexit hook, while the runtime is
    whole, instead of from destructors during teardown.  The child process
    must report the handles released and exit cleanly."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = r'''
import torch
import collective_communication_primitives_amd as dt
p = 4
grads = [[torch.randn(64, 32, device="cuda").to(torch.bfloat16)] for _ in range(p)]
fused = [torch.empty(64 * 32 // 2, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
pipe = dt.HSDPPipeline(2, 2, bucket_bytes=1024)
pipe.post_backward(grads, fused)                  # never finished
xs = [torch.randn(1 << 16, device="cuda") for _ in range(p)]
held = dt.dt_allreduce(xs, [torch.empty_like(x) for x in xs], async_op=True)  # never waited
dt.dt_allreduce([x.clone() for x in xs], async_op=True)                        # dropped: shelved
print("posted", flush=True)
dt._release_all()
assert pipe._h is None and held._h is None and not dt._shelf
print("released", flush=True)
'''
    res = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=120, cwd=root)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "posted" in res.stdout and "released" in res.stdout
