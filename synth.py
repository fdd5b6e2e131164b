"""Seeded synthetic inputs for the same-device collective workloads.

This module holds only random-number draws and shapes; none of the
primitives' arithmetic.  Both the HIP-path tests and the CPU oracle read the
same tensors produced here (the oracle always receives the bytes that were
actually placed on the device, so the generators need not agree across
devices).

Workloads (sizes per rank; P logical ranks share one GPU):
  allreduce_small   P=4, fp32 1,048,576 elements U[-1,1) with seed s+rank,
                    plus int32 values uniform in [-1000, 1000].
  rs_ag_bf16        P=8, bf16 [8192, 8192] drawn N(0,1), sum; int32 of the same
                    shape over the full int32 range for the max op.
  uneven_a2a        P=8, fp32 rows of width 4096; AllGather row counts
                    uniform in [1, 16384]; AllToAll split matrix uniform in
                    [0, 4096] rows per (source, destination) pair.
  bucket_grads      P=8, 32 layers x {[4096,4096] x4, [11008,4096] x2,
                    [4096,11008] x1, [4096] x2} bf16 drawn N(0, 1e-3).
  barrier_sweep     P=16, 1000 barrier generations; fp32 AllReduce at
                    per-rank sizes 4 KiB .. 1 GiB in powers of 4.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np
import torch

MiB = 1 << 20

LAYER_SHAPES: Tuple[Tuple[int, ...], ...] = (
    (4096, 4096), (4096, 4096), (4096, 4096), (4096, 4096),
    (11008, 4096), (11008, 4096),
    (4096, 11008),
    (4096,), (4096,),
)
NUM_LAYERS = 32
BUCKET_BYTES = 25 * MiB
SWEEP_BYTES = tuple(4 ** k for k in range(6, 16))  # 4 KiB .. 1 GiB per rank
ROW_WIDTH = 4096


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def uniform_ranks(nranks: int, numel: int, seed: int = 0, device="cpu",
                  dtype=torch.float32) -> List[torch.Tensor]:
    """Rank r: U[-1, 1) drawn from seed + r."""
    out = []
    for r in range(nranks):
        t = torch.rand(numel, generator=_gen(device, seed + r), device=device, dtype=torch.float32)
        out.append((t * 2 - 1).to(dtype))
    return out


def normal_ranks(nranks: int, shape: Sequence[int], seed: int = 0, device="cpu",
                 dtype=torch.bfloat16, std: float = 1.0) -> List[torch.Tensor]:
    """Rank r: N(0, std^2) drawn from seed + r, stored in ``dtype``."""
    out = []
    for r in range(nranks):
        t = torch.randn(*shape, generator=_gen(device, seed + r), device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out.append(t.to(dtype))
    return out


def int_ranks(nranks: int, numel: int, seed: int = 0, device="cpu", low: int = -1000,
              high: int = 1000) -> List[torch.Tensor]:
    """Rank r: int32 uniform in [low, high] (inclusive) drawn from seed + r."""
    return [torch.randint(low, high + 1, (numel,), generator=_gen(device, seed + r), device=device,
                          dtype=torch.int64).to(torch.int32) for r in range(nranks)]


def full_range_int_ranks(nranks: int, numel: int, seed: int = 0, device="cpu") -> List[torch.Tensor]:
    """Rank r: int32 uniform over the whole int32 range, drawn from seed + r."""
    return [torch.randint(-(2 ** 31), 2 ** 31, (numel,), generator=_gen(device, seed + r), device=device,
                          dtype=torch.int64).to(torch.int32) for r in range(nranks)]


def uneven_row_counts(seed: int = 0, nranks: int = 8, low: int = 1, high: int = 16384) -> np.ndarray:
    """Per-rank Shard(0) row counts, uniform in [low, high]."""
    return np.random.default_rng(seed).integers(low, high + 1, nranks)


def split_matrix(seed: int = 0, nranks: int = 8, high: int = 4096) -> np.ndarray:
    """AllToAll split matrix S[i][j] = rows sent from rank i to rank j, uniform in [0, high]."""
    return np.random.default_rng(seed + 1).integers(0, high + 1, (nranks, nranks))


def uniform_rows(row_counts: Sequence[int], width: int = ROW_WIDTH, seed: int = 0,
                 device="cpu") -> List[torch.Tensor]:
    """Rank r: row_counts[r] rows of ``width`` fp32 values U[-1, 1), seed + r."""
    out = []
    for r, c in enumerate(row_counts):
        t = torch.rand(int(c) * width, generator=_gen(device, seed + r), device=device, dtype=torch.float32)
        out.append(t * 2 - 1)
    return out


def layer_grads(nranks: int, layer: int, seed: int = 0, device="cpu", std: float = 1e-3,
                shapes=LAYER_SHAPES, dtype=torch.bfloat16) -> List[List[torch.Tensor]]:
    """grads[r][t] of one synthetic transformer layer, N(0, std^2) in bf16.

    Seeds are distinct per (seed, layer, rank, tensor)."""
    out = []
    for r in range(nranks):
        row = []
        for t, shape in enumerate(shapes):
            s = ((seed * 1000 + layer) * 64 + r) * 16 + t
            x = torch.randn(*shape, generator=_gen(device, s), device=device, dtype=torch.float32)
            x.mul_(std)
            row.append(x.to(dtype))
        out.append(row)
    return out


def layer_numel(shapes=LAYER_SHAPES) -> int:
    return sum(int(np.prod(s)) for s in shapes)
