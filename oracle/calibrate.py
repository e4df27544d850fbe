"""Sequential temperature scaling of the confidence head (oracle, float64).

DSpark digest, "Verification scheduling (system side)": neural confidences
are over-confident while the scheduler needs their absolute size (it sums
survivals into an expected accepted length), so each position gets a
temperature. Following the chain rule, the running prefix product
prod_{i<=k} c_i is calibrated left to right: at position k a one-dimensional
grid search picks the temperature that minimises the expected calibration
error of that product, with the temperatures of positions < k already fixed.
A positive temperature keeps each position's ranking of the scores.

Readings (the digest gives the procedure, not its details):
  * c_k = sigmoid(z_k * beta_k) with beta_k the inverse temperature (the
    confidence head's inv_temp), z_k the head's logit;
  * the grid is a caller-supplied list of inverse temperatures; the first
    minimiser wins ties;
  * labels y_k in [0, 1] per sample and position: hard (the prefix of length k
    was accepted) or soft (the analytic probability prod_{i<=k} c*_i); a mask
    marks the (sample, position) pairs that have a label;
  * ECE with n_bins equal-width bins on [0, 1] (p clamped, the top edge in the
    last bin): sum over bins of |sum of a_k - sum of y_k| / number of pairs,
    the same binning as the observability accumulator.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def ece_of(p: np.ndarray, y: np.ndarray, n_bins: int) -> float:
    """Expected calibration error of probabilities p against labels y (1-D)."""
    p = np.asarray(p, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if p.size == 0:
        return float("nan")
    pc = np.clip(np.nan_to_num(p, nan=0.0), 0.0, 1.0)
    b = np.minimum(np.floor(pc * n_bins).astype(np.int64), n_bins - 1)
    tot = 0.0
    for i in range(n_bins):
        m = b == i
        tot += abs(pc[m].sum() - y[m].sum())
    return tot / p.size


def sts_fit(z: np.ndarray, y: np.ndarray, mask: np.ndarray, betas: Sequence[float],
            n_bins: int, fixed: Optional[Sequence[float]] = None) -> Dict[str, np.ndarray]:
    """z, y, mask [N, gamma]. Returns inv_temp [gamma], the ECE curve
    ece[gamma, n_grid] and the ECE of the products at beta = 1 (ece_before).

    fixed: optional inverse temperatures to use for the positions before each
    k instead of the fitted ones (a teacher-forced check of one position)."""
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    N, gamma = z.shape
    betas = [float(b) for b in betas]
    inv_temp = np.zeros(gamma)
    curve = np.zeros((gamma, len(betas)))
    before = np.zeros(gamma)
    a_prev = np.ones(N)
    a_plain = np.ones(N)
    for k in range(gamma):
        m = mask[:, k]
        for j, beta in enumerate(betas):
            a = a_prev * _sigmoid(z[:, k] * beta)
            curve[k, j] = ece_of(a[m], y[m, k], n_bins)
        a_plain = a_plain * _sigmoid(z[:, k])
        before[k] = ece_of(a_plain[m], y[m, k], n_bins)
        j_best = int(np.argmin(curve[k]))      # first minimiser
        inv_temp[k] = betas[j_best]
        beta_used = inv_temp[k] if fixed is None else float(fixed[k])
        a_prev = a_prev * _sigmoid(z[:, k] * beta_used)
    return {"inv_temp": inv_temp, "ece": curve, "ece_before": before,
            "ece_after": curve[np.arange(gamma), [betas.index(b) for b in inv_temp]]}


def apply(z: np.ndarray, inv_temp: Sequence[float]) -> Dict[str, np.ndarray]:
    """Calibrated confidences and their running products."""
    c = _sigmoid(np.asarray(z, dtype=np.float64) * np.asarray(inv_temp, dtype=np.float64))
    return {"conf": c, "surv": np.cumprod(c, axis=1)}
