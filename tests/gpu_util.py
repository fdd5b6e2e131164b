"""Helpers for the GPU parity tests: device <-> numpy views and guarded buffers."""
from __future__ import annotations

import sys

import numpy as np
import torch

POISON_F32 = 0x7FBADBAD  # a signalling-NaN bit pattern no kernel result can equal
GUARD = 4096              # bytes of canary before and after every guarded buffer


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says which."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 comes back as uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    return t.cpu().numpy().reshape(-1)


def bits(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def assert_same_bits(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    g, w = bits(np.asarray(got)), bits(np.asarray(want))
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: got {g[bad[:5]]} want {w[bad[:5]]}"


def assert_bf16_within(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    """The bf16 bar: |g - o| <= 2^-8 |o| element-wise (NaN matches NaN), then
    bit equality, which the fixed fold order and one rounding make exact."""
    g = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    o = (want.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan_g, nan_o = np.isnan(g), np.isnan(o)
    assert np.array_equal(nan_g, nan_o), what
    ok = ~nan_o
    differ = ok & (g != o)  # equal values (infinities included) pass outright
    err = np.abs(g[differ] - o[differ])
    assert (err <= 2.0 ** -8 * np.abs(o[differ])).all(), f"{what}: relative error beyond 2^-8"
    assert_same_bits(got[ok], want[ok], what + " (bits)")


def compare(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    """Bit equality; where the oracle's result is a NaN only NaN-ness is
    compared, because IEEE 754 leaves the payload of a NaN produced by an
    addition to the implementation (x86 and the GPU may pick differently)."""
    if got.shape == want.shape and got.dtype == want.dtype and np.array_equal(got.view(np.uint8), want.view(np.uint8)):
        return  # identical bits pass every bar below; large arrays take only this test
    if want.dtype == np.uint16:
        assert_bf16_within(got, want, what)
    elif want.dtype == np.float32:
        nan_w, nan_g = np.isnan(want), np.isnan(got)
        assert np.array_equal(nan_w, nan_g), f"{what}: NaN positions differ"
        assert_same_bits(got[~nan_w], want[~nan_w], what)
    else:
        assert_same_bits(got, want, what)


class Guarded:
    """A device buffer of `numel` elements with poisoned canary bands on both
    sides; `check()` proves nothing was written outside the buffer."""

    def __init__(self, numel: int, dtype: torch.dtype, device="cuda", offset_elems: int = 0):
        es = torch.tensor([], dtype=dtype).element_size()
        g = GUARD // es
        self.raw = torch.empty(g + offset_elems + numel + g, dtype=dtype, device=device)
        self.raw.view(torch.uint8).fill_(0xA5)
        self.g, self.off, self.numel = g, offset_elems, numel
        self.t = self.raw[g + offset_elems:g + offset_elems + numel]

    def poison(self) -> "Guarded":
        self.t.view(torch.uint8).fill_(0xFF)
        return self

    def check(self) -> None:
        head = self.raw[:self.g + self.off].view(torch.uint8)
        tail = self.raw[self.g + self.off + self.numel:].view(torch.uint8)
        assert bool((head == 0xA5).all()), "write before the buffer"
        assert bool((tail == 0xA5).all()), "write after the buffer"
