"""Comparison helpers for the GPU-vs-oracle parity tests (test infrastructure).

Margin rule for top-k index sets: with the oracle's fp64 scores x, let x_(k)
and x_(k+1) be the k-th and (k+1)-th largest. The case is unambiguous when
x_(k) - x_(k+1) > tol, with tol = tau * max(|x_(k)|, |x_(k+1)|) + abs_tol
(tau = 1e-4 is far above the fp32 score error of the GPU path). Unambiguous:
the GPU's ascending list must equal the oracle's exactly. Ambiguous: the GPU
list must be ascending and unique, have k entries, contain every index whose
score is above x_(k) + tol and none whose score is below x_(k+1) - tol.
"""
from __future__ import annotations

import numpy as np
import torch

TAU = 1e-4


def to_np(t) -> np.ndarray:
    """Exact host copy of a tensor (bf16 is widened to float32, which is exact)."""
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def check_topk(x, got, k, tau=TAU, abs_tol=0.0, want=None) -> bool:
    """Assert the margin rule; returns True when the case was unambiguous."""
    x = np.asarray(x, dtype=np.float64)
    got = np.asarray(got, dtype=np.int64)
    n = x.shape[0]
    k = min(int(k), n)
    assert got.shape[0] == k, (got.shape, k)
    assert np.all(np.diff(got) > 0), "indices must be ascending and unique"
    assert got.size == 0 or (got[0] >= 0 and got[-1] < n)
    if k == 0 or k == n:
        assert got.tolist() == list(range(k))
        return True
    order = np.lexsort((np.arange(n), -x))
    xk, xk1 = x[order[k - 1]], x[order[k]]
    tol = tau * max(abs(xk), abs(xk1)) + abs_tol
    if want is None:
        want = np.sort(order[:k])
    if xk - xk1 > tol:
        assert got.tolist() == np.asarray(want).tolist(), "unambiguous top-k differs from the oracle"
        return True
    gs = set(got.tolist())
    must = np.nonzero(x > xk + tol)[0]
    never = np.nonzero(x < xk1 - tol)[0]
    assert set(must.tolist()) <= gs, "a clearly-in index is missing"
    assert not (set(never.tolist()) & gs), "a clearly-out index was selected"
    return False


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def check_lse(got, want, atol=2e-3):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    inf_w = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), inf_w), "empty-row pattern differs"
    if (~inf_w).any():
        assert np.max(np.abs(got[~inf_w] - want[~inf_w])) <= atol
