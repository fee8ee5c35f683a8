"""Parity gates between the GPU path and the fp64 oracle.

Gates (on bf16 O against the unrounded fp64 oracle O, and fp32 LSE):
  * max |O_gpu - O_ref| <= 8e-3, with one exception: where |O_ref| >= 4 the
    bf16 spacing is 2^-5 (half of it, 1.5625e-2, already exceeds 8e-3), so
    there the GPU value must be one of the two bf16 neighbours of O_ref
    (a faithful rounding);
  * mean |O_gpu - O_ref| <= 1e-3;
  * max |LSE_gpu - LSE_ref| <= 1e-3 where finite;
  * rows that see no key: O exactly +0, LSE = -inf, on both sides.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

MAX_ABS = 8e-3
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _bf16_neighbours(x: np.ndarray):
    """The bf16 values just below and just above each element of x (fp64,
    |x| >= 4 where used): bf16 keeps 8 significant bits, so the spacing in
    the binade [2^e, 2^(e+1)) is 2^(e-7)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-300)))
    ulp = np.exp2(e - 7)
    lo = np.floor(x / ulp) * ulp
    return lo, lo + ulp


@dataclass
class ParityReport:
    max_abs: float
    mean_abs: float
    lse_max_abs: float
    n_elements: int
    n_over_gate: int
    n_faithful_exceptions: int

    def __str__(self):
        return (f"max_abs={self.max_abs:.3e} mean_abs={self.mean_abs:.3e} "
                f"lse_max_abs={self.lse_max_abs:.3e} n={self.n_elements} "
                f"over_gate={self.n_over_gate} faithful_exceptions={self.n_faithful_exceptions}")


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray
            ) -> ParityReport:
    """o_*: [..., D] fp64; lse_*: [...] fp64.  Raises AssertionError on a gate."""
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    masked = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), masked), "rows with no visible key differ"
    if masked.any():
        zo = o_gpu[masked]
        assert np.all(zo == 0.0) and not np.any(np.signbit(zo)), "fully masked rows must be +0"
    live = ~masked
    if not live.any():
        return ParityReport(0.0, 0.0, 0.0, 0, 0, 0)
    og, orf = o_gpu[live], o_ref[live]
    assert np.all(np.isfinite(og)), "non-finite output"
    err = np.abs(og - orf)
    over = err > MAX_ABS
    n_exc = 0
    if over.any():
        big = np.abs(orf) >= 4.0
        lo, hi = _bf16_neighbours(orf)
        faithful = (og == lo) | (og == hi)
        bad = over & ~(big & faithful)
        n_exc = int((over & big & faithful).sum())
        if bad.any():
            idx = np.argwhere(bad)[0]
            raise AssertionError(
                f"max-abs gate: {int(bad.sum())} elements over {MAX_ABS}; first at {tuple(idx)}: "
                f"gpu={og[tuple(idx)]!r} ref={orf[tuple(idx)]!r} err={err[tuple(idx)]:.3e}")
    mean_abs = float(err.mean())
    assert mean_abs <= MEAN_ABS, f"mean-abs gate: {mean_abs:.3e}"
    lg, lr = lse_gpu[live], lse_ref[live]
    lse_err = float(np.max(np.abs(lg - lr)))
    assert lse_err <= LSE_ABS, f"LSE gate: {lse_err:.3e}"
    return ParityReport(float(err.max()), mean_abs, lse_err, int(err.size), int(over.sum()), n_exc)


def default_scale(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))
