"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes an oracle object and raises AssertionError when the
oracle disagrees with a fact fixed by the pages or by mathematics:
brute force against Python integers on tiny inputs, closed forms, library
special cases (numpy float32 arithmetic, torch's bf16 conversion,
np.concatenate / np.split), Higham's error bound for recursive summation,
and the patterns the barrier page prints.

The same functions run against deliberately broken copies of the oracle in
``test_oracle_mutants.py``: every planted mistake must trip at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

P_SET = (1, 2, 3, 4, 8, 16)
N_SET = (0, 1, 3, 7, 16, 33)


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16) if a.dtype == np.uint16 else a


def _torch_bf16(values: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _is_nan_bf16(h: np.ndarray) -> np.ndarray:
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)


def _bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------- bf16 --
def pin_bf16_rounding_hand_values(orc):
    """Round-to-nearest-even worked by hand on the binary32 bit patterns."""
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0x3F808000: 0x3F80,  # 1 + 2^-8: exact tie, even neighbour is 1.0
        0x3F818000: 0x3F82,  # 1 + 3*2^-8: tie, rounds up to the even 1+2^-6
        0x3F808001: 0x3F81,  # just above the tie: up
        0x3F807FFF: 0x3F80,  # just below the tie: down
        0x7F7FFFFF: 0x7F80,  # largest finite fp32 overflows to +inf
        0xFF7FFFFF: 0xFF80,  # ... and to -inf
        0x00000001: 0x0000,  # smallest denormal rounds to +0
        0x00008000: 0x0000,  # tie between 0 and the smallest bf16 denormal: even = 0
        0x00018000: 0x0002,  # tie between denormals 1 and 2: even = 2
        0x80000000: 0x8000,  # -0 keeps its sign
        0x7F800000: 0x7F80,  # +inf
    }
    src = np.array(list(cases.keys()), dtype=np.uint32).view(np.float32)
    got = orc.float_to_bf16(src)
    want = np.array(list(cases.values()), dtype=np.uint16)
    assert np.array_equal(got, want), (got, want)
    nan = np.array([0x7FC00000, 0xFF800001, 0x7F800001, 0x7FFFFFFF], dtype=np.uint32).view(np.float32)
    hn = orc.float_to_bf16(nan)
    assert _is_nan_bf16(hn).all(), hn
    assert ((hn >> 15) == np.array([0, 1, 0, 0])).all(), "NaN sign must be kept"


def pin_bf16_rounding_vs_torch(orc, lows=None):
    """Every upper half with the interesting lower halves, against torch's RNE."""
    if lows is None:
        rng = np.random.default_rng(7)
        lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32),
                               rng.integers(0, 1 << 16, 4).astype(np.uint32)])
    highs = np.arange(1 << 16, dtype=np.uint32)
    pats = ((highs[:, None] << 16) | lows[None, :]).reshape(-1)
    vals = pats.view(np.float32)
    got = orc.float_to_bf16(vals)
    ref = _torch_bf16(vals)
    nan_in = np.isnan(vals)
    assert np.array_equal(got[~nan_in], ref[~nan_in])
    assert _is_nan_bf16(got[nan_in]).all()


def pin_bf16_exhaustive(orc, chunk_bits=26):
    """All 2^32 binary32 patterns against torch's RNE (NaN compared by class)."""
    step = 1 << chunk_bits
    for start in range(0, 1 << 32, step):
        pats = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        vals = pats.view(np.float32)
        got = orc.float_to_bf16(vals)
        ref = _torch_bf16(vals)
        nan_in = np.isnan(vals)
        assert np.array_equal(got[~nan_in], ref[~nan_in]), hex(start)
        assert _is_nan_bf16(got[nan_in]).all(), hex(start)


# -------------------------------------------------------------- reductions --
def _int_valued_f32(rng, p, n, bound=1 << 20):
    return [rng.integers(-bound, bound + 1, n).astype(np.float32) for _ in range(p)]


def pin_allreduce_bruteforce(orc):
    """Integer-valued fp32 (every partial sum exact) and int32 against Python ints."""
    rng = np.random.default_rng(11)
    for p in P_SET:
        for n in N_SET:
            xs = _int_valued_f32(rng, p, n)
            ints = [[int(v) for v in x] for x in xs]
            want_sum = [sum(col) for col in zip(*ints)] if n else []
            want_max = [max(col) for col in zip(*ints)] if n else []
            want_min = [min(col) for col in zip(*ints)] if n else []
            for op, want in (("sum", want_sum), ("max", want_max), ("min", want_min)):
                ys = orc.allreduce(xs, op)
                assert len(ys) == p
                for y in ys:
                    assert [int(v) for v in y] == want, (p, n, op)
            xi = [rng.integers(-(2 ** 31), 2 ** 31, n, dtype=np.int64).astype(np.int32) for _ in range(p)]
            for op in ("sum", "max", "min"):
                ys = orc.allreduce(xi, op)
                for e in range(n):
                    col = [int(x[e]) for x in xi]
                    if op == "sum":
                        w = (sum(col) + 2 ** 31) % 2 ** 32 - 2 ** 31  # two's-complement wrap
                    else:
                        w = max(col) if op == "max" else min(col)
                    for y in ys:
                        assert int(y[e]) == w, (p, n, op, e)


def pin_allreduce_numpy_fold(orc):
    """The fp32 sum is numpy's float32 left fold, bit for bit (IEEE add, no FMA)."""
    rng = np.random.default_rng(12)
    for p in (2, 3, 5, 8, 16):
        xs = [(rng.random(997, dtype=np.float32) * 2 - 1).astype(np.float32) for _ in range(p)]
        acc = xs[0].copy()
        for x in xs[1:]:
            acc = (acc + x).astype(np.float32)
        for y in orc.allreduce(xs, "sum"):
            assert np.array_equal(_bits(y), _bits(acc)), p
        # order matters: reversing the ranks generally changes the bits, and
        # the oracle must follow rank order, not any other
        rev = orc.allreduce(xs[::-1], "sum")[0]
        acc_rev = xs[-1].copy()
        for x in xs[-2::-1]:
            acc_rev = (acc_rev + x).astype(np.float32)
        assert np.array_equal(_bits(rev), _bits(acc_rev))
        # max/min with no NaN equal numpy's reductions
        assert np.array_equal(orc.allreduce(xs, "max")[0], np.maximum.reduce(xs))
        assert np.array_equal(orc.allreduce(xs, "min")[0], np.minimum.reduce(xs))
        xi = [rng.integers(-(2 ** 31), 2 ** 31, 513, dtype=np.int64).astype(np.int32) for _ in range(p)]
        assert np.array_equal(orc.allreduce(xi, "max")[0], np.maximum.reduce(xi))
        assert np.array_equal(orc.allreduce(xi, "min")[0], np.minimum.reduce(xi))


def pin_higham_bound(orc):
    """Recursive fp32 summation error within gamma_{P-1} * sum|x_r| of the exact sum."""
    rng = np.random.default_rng(13)
    u = 2.0 ** -24
    for p in (2, 4, 8, 16):
        xs = [(rng.standard_normal(4001) * np.exp(rng.uniform(-8, 8, 4001))).astype(np.float32) for _ in range(p)]
        y = orc.allreduce(xs, "sum")[0].astype(np.float64)
        k = p - 1
        gamma = k * u / (1 - k * u)
        for e in range(0, 4001, 7):
            col = [float(x[e]) for x in xs]
            exact = math.fsum(col)
            assert abs(y[e] - exact) <= gamma * sum(abs(c) for c in col) * (1 + 1e-12), (p, e)


def pin_bf16_sum_one_rounding(orc):
    """bf16: widen exactly, fold in fp32, round once (torch RNE); and 2^-8 of the exact sum."""
    rng = np.random.default_rng(14)
    for p in (2, 4, 8):
        h = [_torch_bf16(rng.standard_normal(2048).astype(np.float32)) for _ in range(p)]
        wide = [_bf16_to_f32(x) for x in h]
        acc = wide[0].copy()
        for w in wide[1:]:
            acc = (acc + w).astype(np.float32)
        want = _torch_bf16(acc)
        for y in orc.allreduce(h, "sum"):
            assert np.array_equal(y, want), p
        got = _bf16_to_f32(orc.allreduce(h, "sum")[0]).astype(np.float64)
        exact = np.sum(np.stack([w.astype(np.float64) for w in wide]), axis=0)
        k = p - 1
        gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
        bound = 2.0 ** -8 * np.abs(acc.astype(np.float64)) + gamma * np.sum(
            np.abs(np.stack(wide).astype(np.float64)), axis=0)
        assert (np.abs(got - exact) <= bound).all()
        # bf16 max/min select an input: exact
        assert np.array_equal(_bf16_to_f32(orc.allreduce(h, "max")[0]), np.maximum.reduce(wide))


def pin_float_max_min_specials(orc):
    """NaN propagates; ties between +0 and -0 keep the earlier rank (the reading taken)."""
    nan = np.float32("nan")
    xs = [np.array([1.0, nan, 0.0, -0.0, 2.0], np.float32),
          np.array([nan, 3.0, -0.0, 0.0, 2.0], np.float32),
          np.array([5.0, 1.0, -0.0, 0.0, -1.0], np.float32)]
    for op in ("max", "min"):
        y = orc.allreduce(xs, op)[0]
        assert np.isnan(y[0]) and np.isnan(y[1]), (op, y)
        assert _bits(y[2:3])[0] == 0x00000000, (op, y)     # rank 0 held +0
        assert _bits(y[3:4])[0] == 0x80000000, (op, y)     # rank 0 held -0
    assert orc.allreduce(xs, "max")[0][4] == 2.0 and orc.allreduce(xs, "min")[0][4] == -1.0


def pin_allreduce_closed_forms(orc):
    """x_r = r+1 -> sum P(P+1)/2, max P, min 1;  x_r[e] = e*P + r -> P*e*P + P(P-1)/2."""
    for p in (1, 2, 5, 16):
        n = 37
        xs = [np.full(n, r + 1, np.float32) for r in range(p)]
        assert (orc.allreduce(xs, "sum")[0] == p * (p + 1) // 2).all()
        assert (orc.allreduce(xs, "max")[0] == p).all()
        assert (orc.allreduce(xs, "min")[0] == 1).all()
        xi = [(np.arange(n) * p + r).astype(np.int32) for r in range(p)]
        want = p * np.arange(n) * p + p * (p - 1) // 2
        assert np.array_equal(orc.allreduce(xi, "sum")[0], want.astype(np.int32))


def pin_denormals_kept(orc):
    """Subnormal fp32 inputs add exactly (no flush to zero)."""
    tiny = np.array([1], np.uint32).view(np.float32)  # 2^-149
    xs = [np.repeat(tiny, 5) for _ in range(3)]
    y = orc.allreduce(xs, "sum")[0]
    assert (_bits(y) == 3).all(), _bits(y)


def pin_reduce_scatter(orc):
    """RS_r == chunk r of AR, closed form on integer data, and P=1 is the identity."""
    rng = np.random.default_rng(15)
    for p in (1, 2, 3, 4, 8):
        for m in (0, 1, 5, 64):
            for dt in ("f32", "bf16", "i32"):
                if dt == "f32":
                    xs = [(rng.random(p * m, dtype=np.float32) * 2 - 1) for _ in range(p)]
                elif dt == "bf16":
                    xs = [_torch_bf16(rng.standard_normal(p * m).astype(np.float32)) for _ in range(p)]
                else:
                    xs = [rng.integers(-1000, 1001, p * m).astype(np.int32) for _ in range(p)]
                for op in ("sum", "max", "min"):
                    rs = orc.reduce_scatter(xs, op)
                    ar = orc.allreduce(xs, op)[0]
                    for r in range(p):
                        assert np.array_equal(_bits(rs[r]), _bits(ar[r * m:(r + 1) * m])), (p, m, dt, op, r)
        xi = [(np.arange(p * 9) * p + r).astype(np.int32) for r in range(p)]
        rs = orc.reduce_scatter(xi, "sum")
        for r in range(p):
            e = np.arange(r * 9, (r + 1) * 9)
            assert np.array_equal(rs[r], (p * e * p + p * (p - 1) // 2).astype(np.int32)), (p, r)
    x1 = [rng.random(10, dtype=np.float32)]
    assert np.array_equal(orc.reduce_scatter(x1, "sum")[0], x1[0])


# ------------------------------------------------------------------ copies --
def pin_all_gather(orc):
    """AG equals np.concatenate in rank order on every rank; AG(RS(x)) == AR(x)."""
    rng = np.random.default_rng(16)
    for p in (1, 2, 3, 8):
        counts = rng.integers(0, 9, p)
        xs = [rng.random(int(c), dtype=np.float32) for c in counts]
        want = np.concatenate(xs) if p else None
        for y in orc.all_gather(xs):
            assert np.array_equal(y, want)
        hs = [rng.integers(0, 1 << 16, int(c)).astype(np.uint16) for c in counts]
        for y in orc.all_gather(hs):
            assert np.array_equal(y, np.concatenate(hs))
        for dt in ("f32", "bf16"):
            m = 13
            if dt == "f32":
                xa = [(rng.random(p * m, dtype=np.float32) * 2 - 1) for _ in range(p)]
            else:
                xa = [_torch_bf16(rng.standard_normal(p * m).astype(np.float32)) for _ in range(p)]
            ag = orc.all_gather(orc.reduce_scatter(xa, "sum"))
            ar = orc.allreduce(xa, "sum")
            for q in range(p):
                assert np.array_equal(_bits(ag[q]), _bits(ar[q])), (p, dt, q)


def _a2a_by_split(xs, s):
    """Block permutation written with np.split / np.concatenate."""
    p = len(xs)
    blocks = [np.split(xs[i], np.cumsum(s[i])[:-1]) for i in range(p)]
    return [np.concatenate([blocks[i][j] for i in range(p)]) for j in range(p)]


def pin_all_to_all(orc):
    """A2A equals the np.split block permutation; A2A(A2A(x,S),S^T) == x;
    S = diag(n) is the identity; S = n * ones is a block transpose."""
    rng = np.random.default_rng(17)
    for p in (1, 2, 3, 5, 8):
        s = rng.integers(0, 6, (p, p))
        xs = [rng.random(int(s[i].sum()), dtype=np.float32) for i in range(p)]
        ys = orc.all_to_all(xs, s)
        for got, want in zip(ys, _a2a_by_split(xs, s)):
            assert np.array_equal(got, want), p
        back = orc.all_to_all(ys, s.T)
        for a, b in zip(back, xs):
            assert np.array_equal(a, b), p
        d = np.diag(rng.integers(0, 5, p))
        xd = [rng.random(int(d[i].sum()), dtype=np.float32) for i in range(p)]
        for a, b in zip(orc.all_to_all(xd, d), xd):
            assert np.array_equal(a, b)
        n = 3
        xt = [np.arange(p * n, dtype=np.int32) + 1000 * i for i in range(p)]
        yt = orc.all_to_all(xt, np.full((p, p), n))
        for j in range(p):
            want = np.concatenate([xt[i][j * n:(j + 1) * n] for i in range(p)])
            assert np.array_equal(yt[j], want)


# ------------------------------------------------------------ bucket / HSDP --
def pin_bucket_allreduce(orc):
    """Bucketed result == per-tensor AR, whatever the bucket size; closed form."""
    rng = np.random.default_rng(18)
    for p in (1, 2, 4):
        sizes = [17, 1, 40, 3, 0, 64]
        grads = [[_torch_bf16(rng.standard_normal(n).astype(np.float32)) for n in sizes] for _ in range(p)]
        want = [orc.allreduce([grads[r][t] for r in range(p)], "sum")[0] for t in range(len(sizes))]
        for bb in (2, 64, 4096, 25 << 20):
            out = orc.bucket_allreduce(grads, bb, "sum")
            for r in range(p):
                for t in range(len(sizes)):
                    assert np.array_equal(out[r][t], want[t]), (p, bb, r, t)
        gf = [[np.full(n, r + 1, np.float32) for n in sizes] for r in range(p)]
        out = orc.bucket_allreduce(gf, 8, "sum")
        for r in range(p):
            for t in range(len(sizes)):
                assert (out[r][t] == p * (p + 1) // 2).all()


def pin_hsdp_layer(orc):
    """Degenerate meshes reduce to RS (replicate=1) and AR (shard=1); the general
    mesh equals RS inside shard groups then AR across replicate groups, and an
    integer closed form holds."""
    rng = np.random.default_rng(19)
    sizes = [8, 16, 4, 24]
    for rep, sh, dt in ((1, 4, "bf16"), (4, 1, "bf16"), (2, 4, "bf16"), (2, 2, "bf16"), (3, 2, "bf16"),
                        (3, 2, "f32"), (4, 2, "f32")):
        p = rep * sh
        if dt == "bf16":
            grads = [[_torch_bf16(rng.standard_normal(n).astype(np.float32)) for n in sizes] for _ in range(p)]
        else:  # fp32 makes the fold order visible in the bits
            grads = [[(rng.random(n, dtype=np.float32) * 2 - 1) for n in sizes] for _ in range(p)]
        out = orc.hsdp_layer(grads, rep, sh, 6, "sum")
        for t, n in enumerate(sizes):
            m = n // sh
            rs_all = {}
            for i in range(rep):
                members = [grads[i * sh + j][t] for j in range(sh)]
                rs = orc.reduce_scatter(members, "sum")
                for j in range(sh):
                    rs_all[(i, j)] = rs[j]
            for j in range(sh):
                ar = orc.allreduce([rs_all[(i, j)] for i in range(rep)], "sum")
                for i in range(rep):
                    assert np.array_equal(_bits(out[i * sh + j][t]), _bits(ar[i])), (rep, sh, dt, t, i, j)
                    assert out[i * sh + j][t].size == m
        gi = [[np.full(n, r + 1, np.float32) for n in sizes] for r in range(p)]
        oi = orc.hsdp_layer(gi, rep, sh, 4, "sum")
        for r in range(p):
            for t in range(len(sizes)):
                assert (oi[r][t] == p * (p + 1) // 2).all(), (rep, sh, r, t)


# ----------------------------------------------------------------- barrier --
def load_golden_rows(path):
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":")
            p, g, r = (int(v) for v in key.split())
            rows[(p, g, r)] = [int(v) for v in vals.split()]
    return rows


def pin_barrier(orc):
    """Rows after G generations read G everywhere but the rank's own 0 (the
    printed pattern at G=1), every generation's waits pass, and a window left
    with one missing notify fails the wait."""
    golden = load_golden_rows(os.path.join(GOLDEN, "barrier_rows.txt"))
    for (p, g, r), row in golden.items():
        w = np.zeros((p, p), np.int32)
        assert orc.barrier(w, 1, g) == g
        assert list(w[r]) == row, (p, g, r, list(w[r]))
    for p in (1, 2, 3, 16):
        w = np.zeros((p, p), np.int32)
        assert orc.barrier(w, 1, 1000) == 1000
        want = np.full((p, p), 1000, np.int32)
        np.fill_diagonal(want, 0)
        assert np.array_equal(w, want)
    # a threshold that is not raised can be met by stale counts: the rising
    # threshold makes an unreached generation fail
    w = np.zeros((4, 4), np.int32)
    orc.barrier(w, 1, 1)
    assert orc.barrier(w.copy(), 3, 1) == 0


def pin_barrier_exchange(orc):
    """The printed golden of the barrier page: y[r] = x[(r+1) % N]."""
    for p in (1, 2, 5, 16):
        xs = [np.full(8, 100 + r, np.int32) for r in range(p)]
        ys = orc.barrier_exchange(xs)
        for r in range(p):
            assert (ys[r] == 100 + (r + 1) % p).all()


# ------------------------------------------------ placement-matrix extras --
def pin_avg(orc):
    """AVG = rank-order sum, then one division by P in the accumulation type:
    numpy float32 fold / float32(P); int32 truncation toward zero of the
    wrapped sum; bf16 = torch RNE of the fp32 mean; RS(avg) = chunk of AR(avg)."""
    rng = np.random.default_rng(21)
    for p in (1, 2, 3, 5, 8, 16):
        xs = [(rng.random(301, dtype=np.float32) * 2 - 1) for _ in range(p)]
        acc = xs[0].copy()
        for x in xs[1:]:
            acc = (acc + x).astype(np.float32)
        want = (acc / np.float32(p)).astype(np.float32)
        for y in orc.allreduce(xs, "avg"):
            assert np.array_equal(_bits(y), _bits(want)), p
        xi = [rng.integers(-(2 ** 31), 2 ** 31, 97, dtype=np.int64).astype(np.int32) for _ in range(p)]
        got = orc.allreduce(xi, "avg")[0]
        for e in range(97):
            s_ = (sum(int(x[e]) for x in xi) + 2 ** 31) % 2 ** 32 - 2 ** 31
            q = abs(s_) // p
            assert int(got[e]) == (-q if s_ < 0 else q), (p, e)
        h = [_torch_bf16(rng.standard_normal(200).astype(np.float32)) for _ in range(p)]
        wide = [_bf16_to_f32(x) for x in h]
        acc = wide[0].copy()
        for w in wide[1:]:
            acc = (acc + w).astype(np.float32)
        assert np.array_equal(orc.allreduce(h, "avg")[0], _torch_bf16((acc / np.float32(p)).astype(np.float32)))
        xr = [(rng.random(p * 11, dtype=np.float32) * 2 - 1) for _ in range(p)]
        rs = orc.reduce_scatter(xr, "avg")
        ar = orc.allreduce(xr, "avg")[0]
        for r in range(p):
            assert np.array_equal(_bits(rs[r]), _bits(ar[r * 11:(r + 1) * 11]))
        ones = [np.full(9, r + 1, np.float32) for r in range(p)]
        assert (orc.allreduce(ones, "avg")[0] == np.float32((p + 1) / 2)).all()


def pin_broadcast(orc):
    rng = np.random.default_rng(22)
    for p in (1, 2, 7, 16):
        x = rng.random(33, dtype=np.float32)
        for y in orc.broadcast(x, p):
            assert np.array_equal(y, x)
        assert len(orc.broadcast(x, p)) == p


def pin_replicate_to_shard(orc):
    """R -> S keeps slice r on rank r (np.split); after an AllReduce it equals
    the ReduceScatter of the same inputs, bit for bit (P->R->S == P->S)."""
    rng = np.random.default_rng(23)
    for p in (1, 2, 3, 8):
        xs = [rng.random(p * 6, dtype=np.float32) for _ in range(p)]
        ys = orc.replicate_to_shard(xs)
        for r in range(p):
            assert np.array_equal(ys[r], np.split(xs[r], p)[r])
        hb = [_torch_bf16(rng.standard_normal(p * 10).astype(np.float32)) for _ in range(p)]
        ar = orc.allreduce(hb, "sum")
        rs = orc.reduce_scatter(hb, "sum")
        for a, b in zip(orc.replicate_to_shard(ar), rs):
            assert np.array_equal(a, b)


def pin_all_gather_into_vec(orc):
    """Rank q's vector entry r is rank r's piece; concatenated, it is the AllGather."""
    rng = np.random.default_rng(24)
    for p in (1, 2, 3, 5):
        xs = [rng.integers(0, 1000, int(rng.integers(0, 7))).astype(np.int32) for _ in range(p)]
        vec = orc.all_gather_into_vec(xs)
        ag = orc.all_gather(xs)
        for q in range(p):
            for r in range(p):
                assert np.array_equal(vec[q][r], xs[r])
            assert np.array_equal(np.concatenate(vec[q]) if p else vec[q], ag[q])


def _shard_blocks(g, p, dim):
    return [np.ascontiguousarray(b).reshape(-1) for b in np.split(g, p, axis=dim)]


def pin_all_to_all_dims(orc):
    """Shard(i) -> Shard(j) equals np.split of the reassembled tensor along j;
    0 -> 1 -> 0 returns every block; i -> i is the identity."""
    rng = np.random.default_rng(25)
    for p, rows, cols in ((1, 3, 5), (2, 4, 6), (3, 6, 9), (4, 8, 4), (8, 16, 24)):
        g = rng.integers(0, 1 << 30, (rows, cols)).astype(np.int32)
        for src in (0, 1):
            xs = _shard_blocks(g, p, src)
            for dst in (0, 1):
                ys = orc.all_to_all_dims(xs, rows, cols, src, dst)
                for got, want in zip(ys, _shard_blocks(g, p, dst)):
                    assert np.array_equal(got, want), (p, src, dst)
        x0 = _shard_blocks(g, p, 0)
        back = orc.all_to_all_dims(orc.all_to_all_dims(x0, rows, cols, 0, 1), rows, cols, 1, 0)
        for a, b in zip(back, x0):
            assert np.array_equal(a, b)


ALL_PINS = [
    pin_bf16_rounding_hand_values,
    pin_bf16_rounding_vs_torch,
    pin_allreduce_bruteforce,
    pin_allreduce_numpy_fold,
    pin_higham_bound,
    pin_bf16_sum_one_rounding,
    pin_float_max_min_specials,
    pin_allreduce_closed_forms,
    pin_denormals_kept,
    pin_reduce_scatter,
    pin_all_gather,
    pin_all_to_all,
    pin_bucket_allreduce,
    pin_hsdp_layer,
    pin_barrier,
    pin_barrier_exchange,
    pin_avg,
    pin_broadcast,
    pin_replicate_to_shard,
    pin_all_gather_into_vec,
    pin_all_to_all_dims,
]
