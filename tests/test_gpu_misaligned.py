"""GPU: buffers that are not 16-byte aligned.

When every buffer of an AllReduce or ReduceScatter is off alignment by the
same amount, the library folds the elements up to the next 16-byte boundary
on the element path and the aligned rest with the vector kernels.  The copy
engines (fan-out, AllToAll, segment copy) run unaligned pieces over their
destination's aligned 16-byte grid, building each vector from aligned loads
of the source.  Every case is compared with the oracle element by element
(bit for bit: copies and fixed-order folds), and guard bands around every
output prove that nothing is written outside it."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, compare, note, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dt():
    import collective_communication_primitives_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _views(src, offset):
    """Copies of src placed `offset` elements past a 16-byte aligned start."""
    out = []
    for x in src:
        g = Guarded(x.numel(), x.dtype, offset_elems=offset)
        g.t.copy_(x.reshape(-1))
        out.append(g)
    return out


@pytest.mark.parametrize("p,dtype,n,off,op", [
    (8, torch.bfloat16, 8192 * 8192, 1, "sum"),     # the RS -> AG workload's shape, 2 bytes off: two-shot body
    (8, torch.bfloat16, 8192 * 8192 + 5, 3, "max"), # ragged too
    (16, torch.float32, (16 << 20) + 3, 1, "sum"),  # 64 MiB + 12 B, 4 bytes off
    (4, torch.float32, 1 << 20, 2, "avg"),          # the small AllReduce, 8 bytes off
    (3, torch.bfloat16, 1000, 7, "min"),            # shorter than a vector after the head
])
def test_allreduce_shared_misalignment(dt, orc, p, dtype, n, off, op):
    note(f"misaligned allreduce P={p} {dtype} n={n} off={off} {op}")
    src = (synth.normal_ranks(p, (n,), seed=p + off, device="cuda", dtype=dtype) if dtype == torch.bfloat16
           else synth.uniform_ranks(p, n, seed=p + off, device="cuda"))
    xs = _views(src, off)
    ys = [Guarded(n, dtype, offset_elems=off).poison() for _ in range(p)]
    dt.dt_allreduce([g.t for g in xs], [g.t for g in ys], op=op)
    torch.cuda.synchronize()
    want = orc.allreduce([to_np(x) for x in src], op)[0]
    compare(to_np(ys[0].t), want, "rank 0")
    view = (lambda t: t.view(torch.int16)) if dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    for q in range(p):
        ys[q].check()
        assert torch.equal(view(ys[q].t), view(ys[0].t)), f"rank {q} differs from rank 0"


@pytest.mark.parametrize("p,dtype,m,off", [
    (8, torch.bfloat16, 8192 * 1024, 1),   # chunks of whole vectors, 2 bytes off: head, body, tail per chunk
    (8, torch.float32, 4096 + 8, 3),       # 12 bytes off
    (5, torch.bfloat16, 4099, 2),          # chunk bytes not a multiple of 16: element path
])
def test_reduce_scatter_shared_misalignment(dt, orc, p, dtype, m, off):
    note(f"misaligned reduce_scatter P={p} {dtype} m={m} off={off}")
    src = (synth.normal_ranks(p, (p * m,), seed=3 * p, device="cuda", dtype=dtype) if dtype == torch.bfloat16
           else synth.uniform_ranks(p, p * m, seed=3 * p, device="cuda"))
    xs = _views(src, off)
    ys = [Guarded(m, dtype, offset_elems=off).poison() for _ in range(p)]
    dt.dt_reduce_scatter([g.t for g in xs], [g.t for g in ys])
    torch.cuda.synchronize()
    want = orc.reduce_scatter([to_np(x) for x in src], "sum")
    for r in range(p):
        ys[r].check()
        compare(to_np(ys[r].t), want[r], f"rank {r}")


def test_uneven_all_gather_odd_bf16_counts(dt, orc):
    """The uneven AllGather workload's row counts, in bf16, each count odd:
    every piece after the first lands at an odd element offset, so its
    destinations are 2 bytes off alignment (the shifted fan-out)."""
    p = 8
    rows = synth.uneven_row_counts(seed=0)
    counts = [int(r) * 4096 + 2 * k + 1 for k, r in enumerate(rows)]
    note(f"uneven bf16 all_gather odd counts total={sum(counts)}")
    xs = [synth.normal_ranks(1, (c,), seed=50 + k, device="cuda", dtype=torch.bfloat16)[0] for k, c in enumerate(counts)]
    total = sum(counts)
    ys = [Guarded(total, torch.bfloat16).poison() for _ in range(p)]
    dt.dt_all_gather(xs, [g.t for g in ys])
    torch.cuda.synchronize()
    want = np.concatenate([to_np(x) for x in xs])
    for q in range(p):
        ys[q].check()
        assert np.array_equal(to_np(ys[q].t), want), f"output {q}"


@pytest.mark.parametrize("p,dtype,counts,recv_off,src_off,in_place", [
    # equal 16 MiB bf16 shards, output q 2(3q+1) bytes off: every destination on a line grid of its own
    (8, torch.bfloat16, [8 << 20] * 8, "3r+1", "0", False),
    # uneven fp32 pieces, sources off alignment too, pieces shorter than a vector and than a line
    (5, torch.float32, [1, 7, 33, 100003, 0], "r", "2r+1", False),
    (3, torch.int32, [4096 * 3 + 5, 1, 65537], "3r", "1", False),
    # in place: each rank's piece already in its own slot, the slots at offsets of their own
    (4, torch.bfloat16, [300001, 299999, 300003, 300000], "2r+1", "0", True),
    # 384 MiB of sources: the windowed fan-out with its read passes
    (8, torch.bfloat16, [24 << 20] * 8, "r", "0", False),
    # from 9 ranks on two workgroups share a tile, each staging the source for its half of the destinations
    (16, torch.bfloat16, [(1 << 18) + k for k in range(16)], "3r+1", "0", False),
    (12, torch.float32, [100000 + 7 * k for k in range(12)], "r", "3r", False),
    (2, torch.int32, [1 << 20, 5], "1", "2r+1", False),
])
def test_all_gather_outputs_offsets_of_their_own(dt, orc, p, dtype, counts, recv_off, src_off, in_place):
    """AllGather whose outputs sit at offsets of their own, so no piece's
    destinations share a line offset: each destination takes the piece over
    its own line grid, every vector shifted out of the source lines staged
    in LDS."""
    note(f"all_gather outputs at offsets of their own P={p} {dtype} counts={counts[:3]}.. recv {recv_off} "
         f"src {src_off} in_place={in_place}")
    total = sum(counts)
    src = []
    for k, c in enumerate(counts):
        if dtype == torch.bfloat16:
            src.append(synth.normal_ranks(1, (c,), seed=90 + k, device="cuda", dtype=dtype)[0])
        elif dtype == torch.int32:
            src.append(synth.int_ranks(1, c, seed=90 + k, device="cuda")[0])
        else:
            src.append(synth.uniform_ranks(1, c, seed=90 + k, device="cuda")[0])
    ys = [Guarded(total, dtype, offset_elems=o).poison() for o in _offsets(recv_off, p)]
    starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    if in_place:
        for k in range(p):
            ys[k].t[starts[k]:starts[k + 1]].copy_(src[k])
        xs = [ys[k].t[starts[k]:starts[k + 1]] for k in range(p)]
    else:
        xs = [g.t for g in _placed(src, _offsets(src_off, p))]
    dt.dt_all_gather(xs, [g.t for g in ys])
    torch.cuda.synchronize()
    want = orc.all_gather([to_np(x) for x in src])
    for q in range(p):
        ys[q].check()
        assert np.array_equal(to_np(ys[q].t), want[q]), f"output {q}"


@pytest.mark.parametrize("dtype,off_send,off_recv", [(torch.bfloat16, 0, 3), (torch.float32, 1, 2), (torch.int32, 3, 0)])
def test_all_to_all_odd_splits(dt, orc, dtype, off_send, off_recv):
    """A split matrix of odd element counts: blocks start at every offset
    inside their source and destination (shifted 1:1 copies)."""
    p = 6
    rng = np.random.default_rng(11)
    s = rng.integers(0, 40000, (p, p)) * 2 + 1
    s[1, 2] = 0
    note(f"all_to_all odd splits {dtype} offsets {off_send}/{off_recv}")
    xs = []
    for i in range(p):
        n = int(s[i].sum())
        t = torch.arange(n, dtype=torch.int32, device="cuda").to(dtype) if dtype != torch.bfloat16 else \
            synth.normal_ranks(1, (n,), seed=70 + i, device="cuda", dtype=dtype)[0]
        g = Guarded(n, dtype, offset_elems=off_send)
        g.t.copy_(t)
        xs.append(g)
    ys = [Guarded(int(s[:, j].sum()), dtype, offset_elems=off_recv).poison() for j in range(p)]
    dt.dt_all_to_all([g.t for g in xs], [g.t for g in ys], s.tolist())
    torch.cuda.synchronize()
    want = orc.all_to_all([to_np(g.t) for g in xs], s)
    for j in range(p):
        ys[j].check()
        assert np.array_equal(to_np(ys[j].t), want[j]), f"rank {j}"


def test_broadcast_and_gather_into_vec_misaligned(dt, orc):
    p, n = 8, (3 << 20) + 7
    root = synth.normal_ranks(1, (n,), seed=90, device="cuda", dtype=torch.bfloat16)[0]
    src = Guarded(n, torch.bfloat16, offset_elems=5)
    src.t.copy_(root)
    outs = [Guarded(n, torch.bfloat16, offset_elems=3).poison() for _ in range(p)]
    note("misaligned broadcast")
    dt.dt_broadcast(src.t, [g.t for g in outs])
    counts = [1000 + 17 * r for r in range(p)]
    pieces = [Guarded(c, torch.bfloat16, offset_elems=r % 8) for r, c in enumerate(counts)]
    for r, g in enumerate(pieces):
        g.t.copy_(synth.normal_ranks(1, (counts[r],), seed=95 + r, device="cuda", dtype=torch.bfloat16)[0])
    vec = [[Guarded(counts[r], torch.bfloat16, offset_elems=1).poison() for r in range(p)] for _ in range(p)]
    note("misaligned all_gather_into_vec")
    dt.dt_all_gather_into_vec([g.t for g in pieces], [[g.t for g in row] for row in vec])
    torch.cuda.synchronize()
    want = to_np(root)
    for q in range(p):
        outs[q].check()
        assert np.array_equal(to_np(outs[q].t), want), f"broadcast {q}"
        for r in range(p):
            vec[q][r].check()
            assert np.array_equal(to_np(vec[q][r].t), to_np(pieces[r].t)), f"vec {q} {r}"


def test_replicate_to_shard_misaligned(dt, orc):
    p, m = 8, (1 << 18) + 3
    src = synth.normal_ranks(p, (p * m,), seed=7, device="cuda", dtype=torch.bfloat16)
    xs = _views(src, 1)
    ys = [Guarded(m, torch.bfloat16, offset_elems=6).poison() for _ in range(p)]
    note("misaligned replicate_to_shard")
    dt.dt_replicate_to_shard([g.t for g in xs], [g.t for g in ys])
    torch.cuda.synchronize()
    want = orc.replicate_to_shard([to_np(x) for x in src])
    for r in range(p):
        ys[r].check()
        assert np.array_equal(to_np(ys[r].t), want[r]), f"rank {r}"


def _carved(p, n, dtype, off_bytes):
    """p views of n elements in one allocation, each off_bytes past a 1 KiB
    (in fact 4 KiB) boundary: every buffer shares its offset modulo 4 KiB,
    which selects the deeper peels.  Returns (views, the whole allocation)."""
    es = torch.tensor([], dtype=dtype).element_size()
    stride = -(-(n * es + off_bytes + 4096) // 4096) * 4096  # bytes between view starts, a 4 KiB multiple
    big = torch.empty(p * stride + 8192, dtype=torch.uint8, device="cuda")
    big.fill_(0xA5)
    lead = (-big.data_ptr()) % 4096
    views = [big[lead + q * stride + off_bytes:lead + q * stride + off_bytes + n * es].view(dtype) for q in range(p)]
    return views, big


@pytest.mark.parametrize("p,dtype,n,off,in_place", [
    (8, torch.bfloat16, 64 << 20, 512, False),      # line-aligned, half a tile in: the 1 KiB peel before the two-shot
    (16, torch.float32, 96 << 20, 256, True),       # the same before 64 MiB windows, in place
    (8, torch.bfloat16, (64 << 20) + 5, 2, False),  # 2 bytes off, shared within 4 KiB: the 4 KiB peel, a ragged end
    (4, torch.float32, 4 << 20, 512, False),        # one-shot size: no peel for line-aligned buffers
])
def test_allreduce_shared_offset_peels(dt, p, dtype, n, off, in_place):
    note(f"allreduce carved views P={p} {dtype} n={n} off={off} in_place={in_place}")
    xs, xbig = _carved(p, n, dtype, off)
    src = (synth.normal_ranks(p, (n,), seed=11 + p, device="cuda", dtype=dtype) if dtype == torch.bfloat16
           else synth.uniform_ranks(p, n, seed=11 + p, device="cuda"))
    for x, s in zip(xs, src):
        x.copy_(s)
    if in_place:
        ys, ybig = xs, xbig
    else:
        ys, ybig = _carved(p, n, dtype, off)
    outside = ybig.clone()
    dt.dt_allreduce(xs, ys)
    torch.cuda.synchronize()
    orc_omp = oracle.get_omp()
    step = 1 << 26
    for a in range(0, n, step):
        b = min(n, a + step)
        want = orc_omp.allreduce([to_np(s[a:b]) for s in src], "sum")[0]
        compare(to_np(ys[0][a:b]), want, f"rank 0 elements [{a}, {b})")
    view = (lambda t: t.view(torch.int16)) if dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    for q in range(1, p):
        assert torch.equal(view(ys[q]), view(ys[0])), f"rank {q} differs from rank 0"
    # nothing outside the outputs was written: every gap between them unchanged
    base = ybig.data_ptr()
    spans = sorted((y.data_ptr() - base, y.data_ptr() - base + y.numel() * y.element_size()) for y in ys)
    at = 0
    for lo, hi in spans + [(ybig.numel(), ybig.numel())]:
        assert torch.equal(ybig[at:lo], outside[at:lo]), f"bytes [{at}, {lo}) outside the outputs changed"
        at = hi


@pytest.mark.parametrize("p,dtype,m,off", [
    (8, torch.bfloat16, 8 << 20, 2),        # 2 bytes past a 4 KiB boundary in every buffer: the 4 KiB peel
    (4, torch.float32, (1 << 20) + 256, 516),  # 516 bytes, chunks 4 MiB + 1 KiB apart: the 1 KiB peel, a ragged end
])
def test_reduce_scatter_shared_offset_peels(dt, p, dtype, m, off):
    """ReduceScatter on views that all sit at one offset past a 4 KiB boundary
    (inputs and outputs carved from single allocations): the head and the
    ragged end of every chunk go out in one element launch, the body on the
    vector kernel.  Compared with the oracle element by element; the bytes
    around the outputs stay untouched."""
    note(f"reduce_scatter carved views P={p} {dtype} m={m} off={off}")
    xs, _ = _carved(p, p * m, dtype, off)
    src = (synth.normal_ranks(p, (p * m,), seed=21 + p, device="cuda", dtype=dtype) if dtype == torch.bfloat16
           else synth.uniform_ranks(p, p * m, seed=21 + p, device="cuda"))
    for x, s in zip(xs, src):
        x.copy_(s)
    ys, ybig = _carved(p, m, dtype, off)
    outside = ybig.clone()
    dt.dt_reduce_scatter(xs, ys)
    torch.cuda.synchronize()
    want = oracle.get_omp().reduce_scatter([to_np(s) for s in src], "sum")
    for r in range(p):
        compare(to_np(ys[r]), want[r], f"rank {r}")
    base = ybig.data_ptr()
    spans = sorted((y.data_ptr() - base, y.data_ptr() - base + y.numel() * y.element_size()) for y in ys)
    at = 0
    for lo, hi in spans + [(ybig.numel(), ybig.numel())]:
        assert torch.equal(ybig[at:lo], outside[at:lo]), f"bytes [{at}, {lo}) outside the outputs changed"
        at = hi


# per-rank element offsets (mod 64) by rule name
_RULES = {"0": lambda r: 0, "1": lambda r: 1, "2": lambda r: 2, "4": lambda r: 4, "8": lambda r: 8, "r": lambda r: r,
          "2r+1": lambda r: 2 * r + 1, "3r+1": lambda r: 3 * r + 1, "3r": lambda r: 3 * r, "5r": lambda r: 5 * r,
          "8r": lambda r: 8 * r}


def _offsets(rule, p):
    return [_RULES[rule](r) % 64 for r in range(p)]


def _placed(src, offsets):
    """Guarded copies of src, copy r placed offsets[r] elements past a 16-byte
    aligned start."""
    out = []
    for x, off in zip(src, offsets):
        g = Guarded(x.numel(), x.dtype, offset_elems=off)
        g.t.copy_(x.reshape(-1))
        out.append(g)
    return out


@pytest.mark.parametrize("p,dtype,n,send_off,recv_off,op,in_place", [
    # the RS -> AG workload's size; inputs at offsets of their own, outputs aligned:
    # the line-grid ReduceScatter, then the fan-out on its aligned path
    (8, torch.bfloat16, 8192 * 8192, "r", "0", "sum", False),
    # inputs 2 bytes off, outputs aligned: the line-grid ReduceScatter, then the aligned fan-out
    (8, torch.bfloat16, 8192 * 8192, "1", "0", "sum", False),
    # vector-aligned inputs 16 bytes off their lines, past P * S = 256 MiB: the line grid, not the vector two-shot
    (8, torch.bfloat16, 1 << 24, "8", "0", "sum", False),
    (16, torch.float32, (1 << 22) + 4, "4", "0", "max", False),
    # outputs at offsets of their own too: the fan-out's byte path
    (8, torch.bfloat16, (1 << 24) + 5, "r", "3r+1", "sum", False),
    # outputs 4 bytes off, inputs aligned; ragged
    (16, torch.float32, (16 << 20) + 3, "0", "1", "sum", False),
    # outputs 16 bytes past a line, inputs 2 bytes off
    (4, torch.bfloat16, 1 << 25, "1", "8", "max", False),
    (3, torch.bfloat16, (1 << 26) + 1, "2r+1", "r", "min", False),
    (5, torch.int32, (1 << 24) + 1, "r", "2", "max", False),
    (6, torch.float32, 1 << 24, "r", "r", "avg", True),    # in place, every rank at its own offset
    # P * S = 160 MiB at P = 6-12: the line-grid two-shot form
    (8, torch.bfloat16, (10 << 20) + 3, "r", "0", "sum", False),
    (6, torch.float32, 7 << 20, "0", "1", "max", False),
    # below the line-grid threshold (P * S = 160 MiB at P = 6-12, else 256 MiB): the element kernel
    (8, torch.bfloat16, (1 << 23) + 3, "r", "0", "sum", False),
    (16, torch.float32, 3 << 20, "0", "1", "sum", False),
    # vector-aligned outputs 16 bytes into their lines at one-shot sizes: the element kernel
    (8, torch.bfloat16, (1 << 20) + 8, "0", "8", "sum", False),
    (16, torch.float32, 1 << 18, "0", "4", "max", False),
    (4, torch.float32, (1 << 22) + 4, "r", "4", "avg", False),
    (4, torch.bfloat16, 300001, "r", "0", "sum", False),
    (4, torch.float32, 1000, "r", "0", "sum", False),
])
def test_allreduce_offsets_of_their_own(dt, orc, p, dtype, n, send_off, recv_off, op, in_place):
    """Buffers at offsets that differ between ranks or between inputs and
    outputs, so no peel aligns them all: the line-grid two-shot form (or the
    element kernel below its threshold)."""
    note(f"allreduce offsets of their own P={p} {dtype} n={n} send {send_off} recv {recv_off} {op} in_place={in_place}")
    src = (synth.normal_ranks(p, (n,), seed=7 * p, device="cuda", dtype=dtype) if dtype == torch.bfloat16
           else synth.int_ranks(p, n, seed=7 * p, device="cuda") if dtype == torch.int32
           else synth.uniform_ranks(p, n, seed=7 * p, device="cuda"))
    xs = _placed(src, _offsets(send_off, p))
    ys = xs if in_place else [Guarded(n, dtype, offset_elems=o).poison() for o in _offsets(recv_off, p)]
    dt.dt_allreduce([g.t for g in xs], [g.t for g in ys], op=op)
    torch.cuda.synchronize()
    want = orc.allreduce([to_np(x) for x in src], op)[0]
    view = (lambda t: t.view(torch.int16)) if dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    compare(to_np(ys[0].t), want, "rank 0")
    for q in range(p):
        ys[q].check()
        assert torch.equal(view(ys[q].t), view(ys[0].t)), f"rank {q} differs from rank 0"


@pytest.mark.parametrize("p,dtype,m,send_off,recv_off,op", [
    (8, torch.bfloat16, 8192 * 1024, "r", "2r+1", "sum"),   # the RS -> AG workload's size
    (8, torch.bfloat16, 8192 * 1024, "1", "0", "sum"),      # inputs 2 bytes off, outputs aligned
    (8, torch.bfloat16, 1 << 20, "8", "0", "sum"),          # inputs 16 bytes off their lines: the grid, not the vector kernel
    (4, torch.float32, 1000, "0", "0", "sum"),               # aligned, chunks of 4000 bytes: inputs off lines from chunk 1
    (4, torch.float32, (1 << 20) + 32, "2", "0", "max"),    # inputs 8 bytes off; chunks end inside a tile
    (8, torch.float32, 4096 + 8, "0", "1", "sum"),           # outputs 4 bytes off only
    (8, torch.bfloat16, 65536, "0", "8r", "sum"),            # outputs 16 bytes apart past their lines
    (16, torch.bfloat16, 1000, "r", "5r", "max"),            # chunks shorter than a tile
    (7, torch.int32, 12345, "3r", "r", "min"),
    (2, torch.bfloat16, 3, "1", "0", "avg"),                 # shorter than one vector
    (1, torch.float32, 777, "1", "2", "sum"),                # one rank: a copy
    # chunks of many tiles, so the staged interior tiles run at these rank counts
    (16, torch.float32, (1 << 18) + 5, "r", "3r+1", "sum"),
    (1, torch.bfloat16, (1 << 20) + 3, "1", "2", "max"),
    (3, torch.int32, 100003, "3r", "5r", "min"),
    (12, torch.bfloat16, (1 << 19) + 7, "2r+1", "0", "avg"),
])
def test_reduce_scatter_offsets_of_their_own(dt, orc, p, dtype, m, send_off, recv_off, op):
    """ReduceScatter over buffers whose offsets differ: the line-grid kernel
    (each chunk tiled over its output's lines, every input shifted into
    place)."""
    note(f"reduce_scatter offsets of their own P={p} {dtype} m={m} send {send_off} recv {recv_off} {op}")
    src = (synth.normal_ranks(p, (p * m,), seed=5 * p, device="cuda", dtype=dtype) if dtype == torch.bfloat16
           else synth.int_ranks(p, p * m, seed=5 * p, device="cuda") if dtype == torch.int32
           else synth.uniform_ranks(p, p * m, seed=5 * p, device="cuda"))
    xs = _placed(src, _offsets(send_off, p))
    ys = [Guarded(m, dtype, offset_elems=o).poison() for o in _offsets(recv_off, p)]
    dt.dt_reduce_scatter([g.t for g in xs], [g.t for g in ys], op=op)
    torch.cuda.synchronize()
    want = orc.reduce_scatter([to_np(x) for x in src], op)
    for r in range(p):
        ys[r].check()
        compare(to_np(ys[r].t), want[r], f"rank {r}")
