"""GPU parity beyond 32-bit byte offsets: rank buffers, ReduceScatter chunks,
AllGather pieces and AllToAll blocks that start or end past 4 GiB.  HBM holds
288 GB, so ranks of several GiB are an ordinary size; every offset in the
kernels and tables must be 64-bit.  Outputs are checked on sampled positions
(the first and last elements, the elements around each 4 GiB boundary, and
random ones), each recomputed by the oracle from the device inputs; copies
are compared exactly on the same positions."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, note, to_np

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_positions(n: int, esize: int, seed: int) -> torch.Tensor:
    """First/last elements, the elements around every 4 GiB byte boundary,
    and 4096 random positions, sorted and unique, as a device index."""
    picks = [np.arange(min(n, 64)), np.arange(max(0, n - 64), n)]
    for b in range(1, (n * esize) // (4 * GIB) + 1):
        at = b * 4 * GIB // esize
        picks.append(np.arange(max(0, at - 32), min(n, at + 32)))
    picks.append(np.random.default_rng(seed).integers(0, n, 4096))
    return torch.from_numpy(np.unique(np.concatenate(picks))).cuda()


def test_allreduce_ranks_beyond_4gib(dt):
    """P=2 fp32, 5 GiB + 12 bytes per rank: vector body past 4 GiB and a
    ragged element tail at the very end."""
    orc = oracle.get()
    n = 5 * GIB // 4 + 3
    note(f"large allreduce P=2 fp32 n={n}")
    xs = [torch.rand(n, device="cuda") * 2 - 1 for _ in range(2)]
    ys = [torch.empty_like(x) for x in xs]
    dt.dt_allreduce(xs, ys)
    torch.cuda.synchronize()
    idx = sample_positions(n, 4, seed=1)
    want = orc.allreduce([to_np(x[idx]) for x in xs], "sum")
    for q in range(2):
        compare(to_np(ys[q][idx]), want[q], f"rank {q}")
    assert torch.equal(ys[0].view(torch.int32), ys[1].view(torch.int32))


def test_reduce_scatter_chunk_beyond_4gib(dt):
    """P=2 bf16, 3 Gi + 8 elements per output chunk: chunk 1 of every input
    starts 6 GiB in, and each output spans 6 GiB."""
    orc = oracle.get()
    m = 3 * GIB + 8
    note(f"large reduce_scatter P=2 bf16 m={m}")
    xs = [torch.randn(2 * m, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ys = [torch.empty(m, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    dt.dt_reduce_scatter(xs, ys)
    torch.cuda.synchronize()
    idx = sample_positions(m, 2, seed=2)
    # rank q's input restricted to the sampled positions of both chunks
    mini = [np.concatenate([to_np(x[idx]), to_np(x[m + idx])]) for x in xs]
    want = orc.reduce_scatter(mini, "sum")
    for r in range(2):
        compare(to_np(ys[r][idx]), want[r], f"rank {r}")


def test_uneven_all_gather_pieces_beyond_4gib(dt):
    """P=2 bf16, pieces of 2.5 Gi + 5 and 3 elements: rank 1's piece lands
    past 5 GiB in every output."""
    c0, c1 = 5 * GIB // 2 + 5, 3
    note(f"large all_gather P=2 bf16 counts=({c0}, {c1})")
    xs = [torch.randn(c0, dtype=torch.bfloat16, device="cuda"),
          torch.randn(c1, dtype=torch.bfloat16, device="cuda")]
    ys = [torch.empty(c0 + c1, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    dt.dt_all_gather(xs, ys)
    torch.cuda.synchronize()
    idx = sample_positions(c0, 2, seed=3)
    for q in range(2):
        assert torch.equal(ys[q][idx].view(torch.int16), xs[0][idx].view(torch.int16)), q
        assert torch.equal(ys[q][c0:].view(torch.int16), xs[1].view(torch.int16)), q
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


def test_all_to_all_blocks_beyond_4gib(dt):
    """P=2 fp32, split matrix [[1.1 Gi, 5], [7, 1.1 Gi + 1]] elements: the
    5-element block starts 4.4 GiB into rank 0's input and the 7-element
    block 4.4 GiB into rank 0's output."""
    big = int(1.1 * GIB)
    s = np.array([[big, 5], [7, big + 1]])
    note(f"large all_to_all P=2 fp32 splits={s.tolist()}")
    xs = [torch.rand(int(s[i].sum()), device="cuda") for i in range(2)]
    ys = [torch.empty(int(s[:, j].sum()), device="cuda") for j in range(2)]
    dt.dt_all_to_all(xs, ys, s.tolist())
    torch.cuda.synchronize()
    # small blocks in full
    assert torch.equal(ys[1][:5], xs[0][big:big + 5])          # 0 -> 1 lands first in rank 1's output
    assert torch.equal(ys[0][big:big + 7], xs[1][:7])          # 1 -> 0 lands after 0 -> 0
    # big blocks on sampled positions
    i0 = sample_positions(big, 4, seed=4)
    assert torch.equal(ys[0][i0], xs[0][i0])                   # 0 -> 0
    i1 = sample_positions(big + 1, 4, seed=5)
    assert torch.equal(ys[1][5 + i1], xs[1][7 + i1])           # 1 -> 1


def test_bucket_and_coalesced_tensor_beyond_4gib(dt):
    """P=2 bf16, a 4.4 GiB gradient between two small ones, 25 MiB buckets
    (pieces starting past 4 GiB inside the tensor), then the coalesced form
    on a copy: both equal the oracle's AllReduce on sampled positions."""
    orc = oracle.get()
    big = int(2.2 * GIB)
    sizes = [17, big, 5]
    note(f"large bucket allreduce P=2 bf16 sizes={sizes}")
    grads = [[torch.randn(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(2)]
    idx = sample_positions(big, 2, seed=6)
    host_big = [to_np(g[1][idx]) for g in grads]
    host_small = [[to_np(g[t]) for g in grads] for t in (0, 2)]
    coal = [[g.clone() for g in rank] for rank in grads]
    dt.dt_bucket_allreduce(grads, bucket_bytes=25 << 20)
    dt.dt_allreduce_coalesced(coal)
    torch.cuda.synchronize()
    want_big = orc.allreduce(host_big, "sum")
    want_small = [orc.allreduce(h, "sum") for h in host_small]
    for out, what in ((grads, "bucket"), (coal, "coalesced")):
        for r in range(2):
            compare(to_np(out[r][1][idx]), want_big[r], f"{what} rank {r} big tensor")
            compare(to_np(out[r][0]), want_small[0][r], f"{what} rank {r} tensor 0")
            compare(to_np(out[r][2]), want_small[1][r], f"{what} rank {r} tensor 2")
        assert torch.equal(out[0][1].view(torch.int16), out[1][1].view(torch.int16)), what


def test_all_to_all_dims_blocks_beyond_4gib(dt):
    """P=2 bf16 [65536, 73728] (4.5 GiB per rank block): sampled elements of
    the Shard(1) blocks sit where the placement puts them, and Shard(0) ->
    Shard(1) -> Shard(0) returns every byte."""
    p, rows, cols = 2, 65536, 73728
    rp, cp = rows // p, cols // p
    note(f"large all_to_all_dims P=2 bf16 [{rows}, {cols}]")
    xs = [torch.randn(rp * cols, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    mid = [torch.empty(rows * cp, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    dt.dt_all_to_all_dims(xs, mid, rows, cols, 0, 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    a = torch.from_numpy(np.concatenate([rng.integers(0, rows, 4096), [0, rows - 1, rp - 1, rp]])).cuda()
    b = torch.from_numpy(np.concatenate([rng.integers(0, cols, 4096), [0, cols - 1, cp - 1, cp]])).cuda()
    # element (a, b) of the full tensor: rank a // rp holds it under Shard(0)
    # at (a % rp, b); rank b // cp holds it under Shard(1) at (a, b % cp)
    for i in range(p):
        for j in range(p):
            sel = ((a // rp) == i) & ((b // cp) == j)
            aa, bb = a[sel], b[sel]
            got = mid[j][aa * cp + (bb - j * cp)]
            want = xs[i][(aa - i * rp) * cols + bb]
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (i, j)
    back = [torch.empty_like(x) for x in xs]
    dt.dt_all_to_all_dims(mid, back, rows, cols, 1, 0)
    torch.cuda.synchronize()
    for r in range(p):
        assert torch.equal(back[r].view(torch.int16), xs[r].view(torch.int16)), r
