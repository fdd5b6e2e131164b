"""GPU: the collectives captured in a HIP graph replay correctly.  The inputs
are rewritten eagerly between replays, with synchronizations in between, and
every replay is checked against the oracle on that replay's inputs."""
import numpy as np
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


def test_graph_replays_allreduce_rs_ag(dt):
    orc = oracle.get()
    p, n = 8, 8 * 4099
    xs = [torch.empty(n, device="cuda") for _ in range(p)]
    ys = [torch.empty(n, device="cuda") for _ in range(p)]
    shards = [torch.empty(n // p, device="cuda") for _ in range(p)]
    full = [torch.empty(n, device="cuda") for _ in range(p)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dt.dt_allreduce(xs, ys)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    note("graph capture of allreduce + reduce_scatter + all_gather")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dt.dt_allreduce(xs, ys)
        dt.dt_reduce_scatter(xs, shards)
        dt.dt_all_gather(shards, full)
    for replay in range(4):
        note(f"graph replay {replay}")
        vals = synth.uniform_ranks(p, n, seed=50 + replay, device="cuda")
        for x, v in zip(xs, vals):
            x.copy_(v)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        host = [to_np(x) for x in xs]
        want = orc.allreduce(host, "sum")
        want_rs = orc.reduce_scatter(host, "sum")
        for q in range(p):
            compare(to_np(ys[q]), want[q], f"replay {replay} AR rank {q}")
            compare(to_np(shards[q]), want_rs[q], f"replay {replay} RS rank {q}")
            compare(to_np(full[q]), np.concatenate(want_rs), f"replay {replay} AG rank {q}")


def test_graph_replays_two_shot_allreduce(dt):
    """An AllReduce in the two-shot window (P=16, 32 MiB fp32 per rank: a
    ReduceScatter into each output's own chunk, then an in-place AllGather)
    captured in a graph; every replay checked against the oracle (rank 0 in
    full, the other ranks bit-equal to rank 0)."""
    orc = oracle.get()
    p, n = 16, 8 << 20
    xs = [torch.empty(n, device="cuda") for _ in range(p)]
    ys = [torch.empty(n, device="cuda") for _ in range(p)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dt.dt_allreduce(xs, ys)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    note("graph capture of a two-shot allreduce P=16 32 MiB fp32")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dt.dt_allreduce(xs, ys)
    for replay in range(3):
        note(f"two-shot graph replay {replay}")
        vals = synth.uniform_ranks(p, n, seed=70 + replay, device="cuda")
        for x, v in zip(xs, vals):
            x.copy_(v)
        for y in ys:
            y.fill_(float("nan"))  # eager work between replays; stale outputs cannot pass
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = orc.allreduce([to_np(x) for x in xs], "sum")[0]
        compare(to_np(ys[0]), want, f"replay {replay} rank 0")
        for q in range(1, p):
            assert torch.equal(ys[q], ys[0]), f"replay {replay} rank {q} differs from rank 0"


def test_graph_replays_large_argument_tables(dt):
    """Launches whose kernel arguments exceed 4 KiB, captured in one graph:
    the coalesced AllReduce of 600 tensors at P=2 (a piece table of about
    43 KiB per launch), the in-place bucket AllReduce of the same tensors
    and an AllToAll over a full 16 x 16 split matrix (a 7.3 KiB block
    table).  The inputs are rewritten eagerly between replays, and every
    replay is checked against the oracle on that replay's inputs."""
    orc = oracle.get()
    rng = np.random.default_rng(5)
    p2, nt = 2, 600
    sizes = [int(x) for x in rng.integers(1, 3000, nt)]
    coal = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(p2)]
    buck = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(p2)]
    p16 = 16
    split = rng.integers(0, 600, (p16, p16)) + 1
    a_in = [torch.empty(int(split[i].sum()), dtype=torch.int32, device="cuda") for i in range(p16)]
    a_out = [torch.empty(int(split[:, j].sum()), dtype=torch.int32, device="cuda") for j in range(p16)]

    def work():
        dt.dt_allreduce_coalesced(coal, op="max")
        dt.dt_bucket_allreduce(buck, bucket_bytes=64 << 10)
        dt.dt_all_to_all(a_in, a_out, split.tolist())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # the launch path warmed outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    note("graph capture of coalesced / bucket / all-to-all launches")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for replay in range(3):
        note(f"graph replay {replay} (large argument tables)")
        for r in range(p2):
            for t, n in enumerate(sizes):
                v = synth.normal_ranks(1, (n,), seed=1000 * replay + 10 * r + t % 10, device="cuda",
                                       dtype=torch.bfloat16)[0]
                coal[r][t].copy_(v)
                buck[r][t].copy_(v)
        for i in range(p16):
            a_in[i].copy_(torch.randint(-2**31, 2**31 - 1, (a_in[i].numel(),), dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        host_c = [[to_np(t) for t in rank] for rank in coal]
        host_a = [to_np(x) for x in a_in]
        g.replay()
        torch.cuda.synchronize()
        want_max = [[orc.allreduce([host_c[r][t] for r in range(p2)], "max")[0] for t in range(nt)]]
        want_sum = orc.bucket_allreduce(host_c, 64 << 10, "sum")
        for r in range(p2):
            for t in range(nt):
                compare(to_np(coal[r][t]), want_max[0][t], f"replay {replay} coalesced rank {r} tensor {t}")
                compare(to_np(buck[r][t]), want_sum[r][t], f"replay {replay} bucket rank {r} tensor {t}")
        want_a = orc.all_to_all(host_a, split)
        for j in range(p16):
            compare(to_np(a_out[j]), want_a[j], f"replay {replay} all_to_all rank {j}")


def test_graph_replays_offsets_of_their_own(dt):
    """Buffers at offsets of their own captured in a graph: the line-grid
    AllReduce (P=8 bf16, 32 MiB + 6 bytes per rank, inputs 2 bytes off,
    outputs at 2(3q+1) bytes: the staged line-grid ReduceScatter and the
    fan-out to destinations at offsets of their own), the line-grid
    ReduceScatter with inputs 8 bytes off and outputs aligned, and the
    odd-count AllGather (the
    line-grid fan-out with its windowed piece ends); every replay checked
    against the oracle on that replay's inputs."""
    orc = oracle.get()
    p, n = 8, (16 << 20) + 3
    m = n // p
    xb = [torch.empty(n + 64, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    yb = [torch.empty(n + 64, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    rb = [torch.empty(m + 64, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    xs = [b[1:1 + n] for b in xb]
    ys = [b[3 * q + 1:3 * q + 1 + n] for q, b in enumerate(yb)]
    xs8 = [b[4:4 + p * m] for b in xb]
    rs = [b[:m] for b in rb]
    counts = [1001 + 2 * k for k in range(p)]
    ag_in = [torch.empty(c, dtype=torch.bfloat16, device="cuda") for c in counts]
    ag_out = [torch.empty(sum(counts), dtype=torch.bfloat16, device="cuda") for _ in range(p)]

    def work():
        dt.dt_allreduce(xs, ys)
        dt.dt_reduce_scatter(xs8, rs)
        dt.dt_all_gather(ag_in, ag_out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    note("graph capture of line-grid allreduce, line-grid reduce_scatter, odd-count all_gather")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for replay in range(3):
        note(f"offsets graph replay {replay}")
        vals = synth.normal_ranks(p, (n + 64,), seed=90 + replay, device="cuda", dtype=torch.bfloat16)
        for b, v in zip(xb, vals):
            b.copy_(v)  # eager work between replays
        small = synth.normal_ranks(p, (max(counts),), seed=95 + replay, device="cuda", dtype=torch.bfloat16)
        for t, v in zip(ag_in, small):
            t.copy_(v[:t.numel()])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = orc.allreduce([to_np(x) for x in xs], "sum")[0]
        view = lambda t: t.view(torch.int16)
        compare(to_np(ys[0]), want, f"replay {replay} AR rank 0")
        for q in range(1, p):
            assert torch.equal(view(ys[q]), view(ys[0])), f"replay {replay} AR rank {q}"
        want_rs = orc.reduce_scatter([to_np(x) for x in xs8], "sum")
        for r in range(p):
            compare(to_np(rs[r]), want_rs[r], f"replay {replay} RS rank {r}")
        cat = np.concatenate([to_np(t) for t in ag_in])
        for q in range(p):
            assert np.array_equal(to_np(ag_out[q]), cat), f"replay {replay} AG rank {q}"
