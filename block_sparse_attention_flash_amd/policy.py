"""Threshold policy lambda = a / L and its one-pass calibration (host side).

BLASST blog, section on the lambda = a/L policy and the calibration algorithm
(Algorithm 2): the threshold that keeps a given block sparsity falls inversely
with the context length L, lambda = a / L, and the constant comes from one
forward pass over calibration sequences.  For every sequence i (length L_i)
and candidate threshold lambda_j the measured sparsity s_ij gives a point
(lambda_j * L_i, s_ij); an exponential model a = alpha * exp(beta * s) is fitted
to the points, and at run time the threshold for a target sparsity S is
lambda = alpha * exp(beta * S) / L.

One pass suffices because a block's skip test compares a lambda-independent
margin D with ln(lambda) (the margin entry points of the library emit D); the
sparsity at any lambda is then the fraction of decisions with D < ln(lambda).
Everything here is host arithmetic on those margins: it is not on the hot path.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

__all__ = ["sparsity_at", "margin_histogram", "calibration_points", "fit_exponential", "lambda_for"]


def _as_numpy(margins) -> np.ndarray:
    if hasattr(margins, "detach"):  # a torch tensor, on the GPU or not
        margins = margins.detach().float().cpu().numpy()
    return np.asarray(margins, dtype=np.float64)


def sparsity_at(margins, lambdas: Iterable[float]) -> np.ndarray:
    """Block sparsity at each lambda: the fraction of decisions (non-NaN margins,
    NaN marks a block the causal mask never visits) with margin < ln(lambda).
    lambda = 0 never skips."""
    m = _as_numpy(margins).ravel()
    m = m[~np.isnan(m)]
    out = []
    for lam in lambdas:
        if not (0.0 <= lam < 1.0):
            raise ValueError("lambda must lie in [0, 1)")
        if lam == 0.0 or m.size == 0:
            out.append(0.0)
        else:
            out.append(float(np.count_nonzero(m < math.log(lam))) / m.size)
    return np.asarray(out)


def margin_histogram(margins, edges: Sequence[float]) -> np.ndarray:
    """Counts of decisions (non-NaN margins) per bin: [-inf, e0), [e0, e1), ...,
    [e_last, +inf) -- len(edges) + 1 bins.  With ln(lambda) on an edge, the
    counts below it over the total are the block sparsity at that lambda."""
    m = _as_numpy(margins).ravel()
    m = m[~np.isnan(m)]
    e = np.asarray(edges, dtype=np.float64)
    if e.ndim != 1 or e.size == 0 or np.any(np.diff(e) <= 0):
        raise ValueError("edges must be a non-empty increasing sequence")
    return np.bincount(np.searchsorted(e, m, side="right"), minlength=e.size + 1)


def calibration_points(margins_by_sequence: Sequence, lengths: Sequence[int],
                       lambdas: Sequence[float]) -> Tuple[np.ndarray, np.ndarray]:
    """The calibration data of Algorithm 2: for every sequence and candidate
    lambda, (a = lambda * L, measured sparsity s)."""
    if len(margins_by_sequence) != len(lengths):
        raise ValueError("one length per margin array")
    a, s = [], []
    for mg, L in zip(margins_by_sequence, lengths):
        sp = sparsity_at(mg, lambdas)
        for lam, sv in zip(lambdas, sp):
            a.append(lam * L)
            s.append(sv)
    return np.asarray(a), np.asarray(s)


def fit_exponential(a: np.ndarray, s: np.ndarray) -> Tuple[float, float]:
    """Least-squares fit of ln a = ln alpha + beta * s over the points with
    0 < s < 1 (a point at 0% or 100% sparsity only bounds the curve).
    Returns (alpha, beta)."""
    a = np.asarray(a, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    keep = (s > 0.0) & (s < 1.0) & (a > 0.0)
    if np.count_nonzero(keep) < 2 or np.ptp(s[keep]) == 0.0:
        raise ValueError("need at least two points with distinct sparsities strictly between 0 and 1")
    beta, ln_alpha = np.polyfit(s[keep], np.log(a[keep]), 1)
    return float(math.exp(ln_alpha)), float(beta)


def lambda_for(target_sparsity: float, length: int, alpha: float, beta: float) -> float:
    """Run-time threshold for a target block sparsity at context length L:
    lambda = alpha * exp(beta * S) / L (clipped below 1)."""
    if not (0.0 <= target_sparsity <= 1.0) or length <= 0:
        raise ValueError("target sparsity in [0, 1] and a positive length")
    return min(alpha * math.exp(beta * target_sparsity) / length, math.nextafter(1.0, 0.0))


def lambda_at_sparsity(margins, target_sparsity: float) -> float:
    """The inverse of sparsity_at on one set of margins: a lambda at which the
    fraction of decisions skipped is the target rounded up to a whole decision
    (k = ceil(target * n) decisions, more where the k-th smallest margin is
    tied).  ln(lambda) lies above the k-th smallest margin and at most at the
    next one.  Used to time a kernel at a stated sparsity; clipped below 1
    (decisions with margin 0, the blocks that set the running max, are never
    skipped) and above 0 (lambda = 0 never skips)."""
    if not (0.0 <= target_sparsity <= 1.0):
        raise ValueError("target sparsity in [0, 1]")
    m = _as_numpy(margins).ravel()
    m = np.sort(m[~np.isnan(m)])
    k = int(math.ceil(target_sparsity * m.size))
    if k == 0:
        return 0.0
    lo = float(m[k - 1])
    hi = float(m[k]) if k < m.size else 0.0
    if hi > lo:
        ln_lam = 0.5 * (lo + hi) if math.isfinite(lo) else hi - 1.0
    else:
        ln_lam = math.nextafter(lo, math.inf) if math.isfinite(lo) else -700.0
    lam = math.exp(ln_lam) if ln_lam < 0.0 else 1.0
    return min(max(lam, math.ulp(0.0)), math.nextafter(1.0, 0.0))
