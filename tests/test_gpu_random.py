"""GPU: seeded random parity sweep over every primitive.  Each case draws
the rank count, sizes, element offsets (alignment), dtype and op from a
fixed seed, runs the C ABI, and compares every output with the oracle;
canary bands around each output catch stray writes."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, compare, note, to_np

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}
CASES = 40


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _data(rng, dtype, n):
    if dtype == "i32":
        return torch.from_numpy(rng.integers(-(2 ** 31), 2 ** 31, n, dtype=np.int64).astype(np.int32)).cuda()
    v = torch.from_numpy((rng.standard_normal(n) * np.exp(rng.uniform(-4, 4, n))).astype(np.float32)).cuda()
    return v if dtype == "f32" else v.to(torch.bfloat16)


def _inputs(rng, dtype, p, n):
    """Rank buffers at random element offsets inside guarded allocations."""
    out = []
    for _ in range(p):
        g = Guarded(n, DTYPES[dtype], offset_elems=int(rng.integers(0, 5)))
        if n:
            g.t.copy_(_data(rng, dtype, n))
        out.append(g)
    return out


def _outputs(rng, dtype, sizes):
    return [Guarded(n, DTYPES[dtype], offset_elems=int(rng.integers(0, 5))).poison() for n in sizes]


@pytest.mark.parametrize("case", range(CASES))
def test_random_reductions(dt, orc, case):
    rng = np.random.default_rng(1000 + case)
    dtype = ["f32", "bf16", "i32"][case % 3]
    op = ["sum", "max", "min", "avg"][int(rng.integers(0, 4))]
    p = int(rng.integers(1, 17))
    m = int(rng.choice([0, 1, int(rng.integers(2, 300)), int(rng.integers(300, 40000))]))
    note(f"random reductions case={case} {dtype} {op} P={p} m={m}")
    xs = _inputs(rng, dtype, p, p * m)
    host = [to_np(x.t) for x in xs]
    ar = _outputs(rng, dtype, [p * m] * p)
    dt.dt_allreduce([x.t for x in xs], [y.t for y in ar], op=op)
    rs = _outputs(rng, dtype, [m] * p)
    dt.dt_reduce_scatter([x.t for x in xs], [y.t for y in rs], op=op)
    torch.cuda.synchronize()
    want_ar = orc.allreduce(host, op) if p * m else [np.empty(0, host[0].dtype)] * p
    want_rs = orc.reduce_scatter(host, op) if p * m else [np.empty(0, host[0].dtype)] * p
    for q in range(p):
        ar[q].check()
        rs[q].check()
        compare(to_np(ar[q].t), want_ar[q], f"AR rank {q}")
        compare(to_np(rs[q].t), want_rs[q], f"RS rank {q}")


@pytest.mark.parametrize("case", range(CASES))
def test_random_copies(dt, orc, case):
    rng = np.random.default_rng(5000 + case)
    dtype = ["f32", "bf16", "i32"][case % 3]
    p = int(rng.integers(1, 17))
    counts = [int(rng.choice([0, int(rng.integers(1, 64)), int(rng.integers(64, 9000))])) for _ in range(p)]
    note(f"random copies case={case} {dtype} P={p} counts={counts}")
    xs = []
    for c in counts:
        g = Guarded(c, DTYPES[dtype], offset_elems=int(rng.integers(0, 5)))
        if c:
            g.t.copy_(_data(rng, dtype, c))
        xs.append(g)
    host = [to_np(x.t) for x in xs]
    total = sum(counts)
    ag = _outputs(rng, dtype, [total] * p)
    dt.dt_all_gather([x.t for x in xs], [y.t for y in ag])
    s = rng.integers(0, int(rng.choice([1, 8, 700])) + 1, (p, p))
    a2a_in = []
    for i in range(p):
        g = Guarded(int(s[i].sum()), DTYPES[dtype], offset_elems=int(rng.integers(0, 5)))
        if s[i].sum():
            g.t.copy_(_data(rng, dtype, int(s[i].sum())))
        a2a_in.append(g)
    a2a_host = [to_np(x.t) for x in a2a_in]
    a2a = _outputs(rng, dtype, [int(s[:, j].sum()) for j in range(p)])
    dt.dt_all_to_all([x.t for x in a2a_in], [y.t for y in a2a], s.tolist())
    torch.cuda.synchronize()
    if total:
        want = orc.all_gather(host)
        for q in range(p):
            ag[q].check()
            np.testing.assert_array_equal(to_np(ag[q].t).view(np.uint8), want[q].view(np.uint8))
    want = orc.all_to_all(a2a_host, s)
    for j in range(p):
        a2a[j].check()
        np.testing.assert_array_equal(to_np(a2a[j].t).view(np.uint8), want[j].view(np.uint8))


@pytest.mark.parametrize("case", range(CASES // 2))
def test_random_buckets(dt, orc, case):
    rng = np.random.default_rng(9000 + case)
    dtype = ["f32", "bf16", "i32"][case % 3]
    op = ["sum", "max", "min", "avg"][int(rng.integers(0, 4))]
    p = int(rng.integers(1, 17))
    nt = int(rng.integers(1, 80))
    sizes = [int(rng.choice([0, int(rng.integers(1, 40)), int(rng.integers(40, 3000))])) for _ in range(nt)]
    bucket = 16 * int(rng.integers(1, 400))
    use_ws = bool(rng.integers(0, 2))
    note(f"random buckets case={case} {dtype} {op} P={p} tensors={nt} bucket={bucket} ws={use_ws}")
    grads = [[(_data(rng, dtype, n) if n else torch.empty(0, dtype=DTYPES[dtype], device="cuda")) for n in sizes]
             for _ in range(p)]
    host = [[to_np(g) for g in rank] for rank in grads]
    ws = [torch.empty(bucket, dtype=torch.uint8, device="cuda") for _ in range(p)] if use_ws else None
    coal = [[g.clone() for g in rank] for rank in grads]  # the coalesced form on the same data
    dt.dt_bucket_allreduce(grads, bucket_bytes=bucket, bucket_ws=ws, op=op)
    dt.dt_allreduce_coalesced(coal, op=op)
    torch.cuda.synchronize()
    want = orc.bucket_allreduce(host, bucket, op)
    for r in range(p):
        for t in range(nt):
            compare(to_np(grads[r][t]), want[r][t], f"bucket rank {r} tensor {t}")
            compare(to_np(coal[r][t]), want[r][t], f"coalesced rank {r} tensor {t}")


def _carved(p, n, dtype, off_bytes):
    """p views of n elements cut from one allocation, each off_bytes past a
    4 KiB boundary, the allocation filled with a canary byte: every buffer
    shares its offset, which selects the deeper peels of the folds."""
    es = torch.tensor([], dtype=dtype).element_size()
    stride = -(-(n * es + off_bytes + 4096) // 4096) * 4096
    big = torch.empty(p * stride + 8192, dtype=torch.uint8, device="cuda")
    big.fill_(0xA5)
    lead = (-big.data_ptr()) % 4096
    views = [big[lead + q * stride + off_bytes:lead + q * stride + off_bytes + n * es].view(dtype) for q in range(p)]
    return views, big


def _outside_unchanged(views, big, before):
    base = big.data_ptr()
    spans = sorted((v.data_ptr() - base, v.data_ptr() - base + v.numel() * v.element_size()) for v in views)
    at = 0
    for lo, hi in spans + [(big.numel(), big.numel())]:
        assert torch.equal(big[at:lo], before[at:lo]), f"bytes [{at}, {lo}) outside the outputs changed"
        at = hi


@pytest.mark.parametrize("case", range(24))
def test_random_shared_offsets(dt, orc, case):
    """Every buffer at one random offset past a 4 KiB boundary (any multiple
    of the element size below 4 KiB), random rank count, dtype, op and size,
    a quarter of the cases large enough for the two-shot form: AllReduce
    and ReduceScatter against the oracle, nothing written outside."""
    rng = np.random.default_rng(9000 + case)
    dtype = ["f32", "bf16", "i32"][case % 3]
    es = 2 if dtype == "bf16" else 4
    op = ["sum", "max", "min", "avg"][int(rng.integers(0, 4))]
    if case % 4 == 3:
        p = int(rng.choice([8, 12, 16]))
        m = (24 << 20) // es // p + int(rng.integers(0, 4096))  # 24 MiB per rank and more: two-shot
    else:
        p = int(rng.integers(1, 17))
        m = int(rng.choice([1, int(rng.integers(2, 3000)), int(rng.integers(3000, 200000))]))
    off = int(rng.integers(0, 4096 // es)) * es
    note(f"random shared offsets case={case} {dtype} {op} P={p} m={m} off={off}")
    xs, _ = _carved(p, p * m, DTYPES[dtype], off)
    for x in xs:
        x.copy_(_data(rng, dtype, p * m))
    host = [to_np(x) for x in xs]
    ar, arbig = _carved(p, p * m, DTYPES[dtype], off)
    rs, rsbig = _carved(p, m, DTYPES[dtype], off)
    ar_before, rs_before = arbig.clone(), rsbig.clone()
    dt.dt_allreduce(xs, ar, op=op)
    dt.dt_reduce_scatter(xs, rs, op=op)
    torch.cuda.synchronize()
    want_ar = orc.allreduce(host, op)[0]
    want_rs = orc.reduce_scatter(host, op)
    for q in range(p):
        compare(to_np(ar[q]), want_ar, f"AR rank {q}")
        compare(to_np(rs[q]), want_rs[q], f"RS rank {q}")
    _outside_unchanged(ar, arbig, ar_before)
    _outside_unchanged(rs, rsbig, rs_before)


@pytest.mark.parametrize("case", range(8))
def test_random_large_offsets(dt, orc, case):
    """AllReduce and ReduceScatter past the line-grid two-shot threshold
    (P * S of 256-512 MiB) over buffers at offsets of their own: even cases
    put every input at one offset, odd cases draw every offset; all take the
    staged line-grid ReduceScatter."""
    rng = np.random.default_rng(9000 + case)
    dtype = ["f32", "bf16", "i32"][case % 3]
    op = ["sum", "max", "min", "avg"][int(rng.integers(0, 4))]
    p = int(rng.integers(2, 17))
    es = 2 if dtype == "bf16" else 4
    per_rank = int(rng.integers(256, 512)) * (1 << 20) // p
    n = per_rank // es // p * p + int(rng.integers(0, 1000)) * p
    shared = int(rng.integers(0, 64))
    send_offs = [shared if case % 2 == 0 else int(rng.integers(0, 64)) for _ in range(p)]
    note(f"random large offsets case={case} {dtype} {op} P={p} n={n} send offsets {send_offs[:4]}")
    xs = []
    for off in send_offs:
        g = Guarded(n, DTYPES[dtype], offset_elems=off)
        g.t.copy_(_data(rng, dtype, n))
        xs.append(g)
    host = [to_np(x.t) for x in xs]
    ar = [Guarded(n, DTYPES[dtype], offset_elems=int(rng.integers(0, 64))).poison() for _ in range(p)]
    dt.dt_allreduce([x.t for x in xs], [y.t for y in ar], op=op)
    torch.cuda.synchronize()
    want = orc.allreduce(host, op)[0]
    for q in range(p):
        ar[q].check()
        compare(to_np(ar[q].t), want, f"AR rank {q}")
    del ar
    rs = [Guarded(n // p, DTYPES[dtype], offset_elems=int(rng.integers(0, 64))).poison() for _ in range(p)]
    dt.dt_reduce_scatter([x.t for x in xs], [y.t for y in rs], op=op)
    torch.cuda.synchronize()
    want_rs = orc.reduce_scatter(host, op)
    for r in range(p):
        rs[r].check()
        compare(to_np(rs[r].t), want_rs[r], f"RS rank {r}")
