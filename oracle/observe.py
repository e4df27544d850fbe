"""Observability outputs of the chain (oracle).

SGLang DSpark blog, "Observability": compact verification only checks the
scheduler's window, so the acceptance a full-block verification would have
reached (the ceiling) goes unseen; a cap-accept run commits what compact
commits while exposing that ceiling, and the engine also reports each
request's confidence and calibration metrics such as ECE. Its section "Per-
request differentiation on mixed traffic" reports the windows and the
utilisation against the ceiling per workload class.

DSpark digest, "Verification scheduling (system side)": the confidence head is
trained against the analytic per-slot acceptance rate
c*_k = 1 - 1/2 || p_d,k - p_t,k ||_1 (one minus the total-variation distance
between the slot's draft and target distributions), and sequential temperature
scaling calibrates the running products prod_{i<=k} c_i per position by their
expected calibration error.

Readings:
  * A verified slot k of request r (k <= Lv_r = cu[r+1] - cu[r] - 1) has draft
    distribution softmax(U[r, k] + W1[x_{k-1}] W2) and target distribution
    softmax(target_packed[cu[r] + k - 1]); c* of an unverified slot is NaN.
  * Per step and request the accumulator counts: the commit A_r + 1, the
    accepted drafts A_r, the ceiling C_r (leading accepts over every verified
    slot, the verify's ceiling output), the scheduler window L_r and the
    verified slots Lv_r; histograms of L_r, A_r and C_r over 0..gamma.
  * Calibration pairs, per position k:
      conditional -- (c_k, slot k accepted) for k <= min(C_r + 1, Lv_r): the
                     slots whose whole prefix was accepted, which is the event
                     c_k is defined on;
      prefix      -- (a_k, C_r >= k) for k <= Lv_r: the running product against
                     the acceptance of the whole prefix up to k.
    A pair lands in bin floor(p * n_bins) (p clamped to [0, 1], the top edge in
    the last bin, NaN in bin 0) and adds 1 to the bin's count, floor(p * 2^32)
    to its probability sum and the outcome to its hit count -- integers, so the
    totals do not depend on the order of accumulation.
  * ECE = sum over bins of |sum p - hits| / total count; utilisation =
    accepted / ceiling, and committed utilisation = (accepted + steps) /
    (ceiling + steps) per request.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

from .markov import widen, markov_logits

P_SCALE = 1 << 32
KIND_CONDITIONAL, KIND_PREFIX = 0, 1


def _softmax(z: np.ndarray) -> np.ndarray:
    m = z.max()
    w = np.exp(z - m)
    return w / w.sum()


def analytic_acceptance(target_packed, cu_seqlens: Sequence[int], anchor: Sequence[int],
                        tokens: np.ndarray, U: np.ndarray, W1: np.ndarray, W2: np.ndarray,
                        requests: Optional[Sequence[int]] = None) -> np.ndarray:
    """c*[r, k-1] = 1 - 1/2 ||p_d - p_t||_1 for every verified slot (float64);
    NaN elsewhere. `requests`: optional subset (others stay NaN)."""
    tokens = np.asarray(tokens)
    R, gamma = tokens.shape
    out = np.full((R, gamma), np.nan)
    todo = range(R) if requests is None else requests
    for r in todo:
        Lv = int(cu_seqlens[r + 1]) - int(cu_seqlens[r]) - 1
        for k in range(1, min(Lv, gamma) + 1):
            x_prev = int(anchor[r]) if k == 1 else int(tokens[r, k - 2])
            pd = _softmax(markov_logits(U[r, k - 1], W1, W2, x_prev))
            pt = _softmax(widen(target_packed[int(cu_seqlens[r]) + k - 1]))
            out[r, k - 1] = 1.0 - 0.5 * np.abs(pd - pt).sum()
    return out


def new_stats(R: int, gamma: int, n_bins: int) -> Dict[str, np.ndarray]:
    """Zeroed accumulator (Python ints in object arrays: no overflow)."""
    z = lambda *shape: np.zeros(shape, dtype=object)
    return {"steps": 0, "req_steps": 0, "committed": 0, "accepted": 0, "ceiling": 0,
            "window": 0, "verified": 0,
            "hist_window": z(gamma + 1), "hist_accept": z(gamma + 1), "hist_ceiling": z(gamma + 1),
            "req_accepted": z(R), "req_ceiling": z(R), "req_window": z(R),
            "bins": z(2, gamma, n_bins, 3)}


def _bin(p: float, n_bins: int) -> int:
    if math.isnan(p):
        return 0
    p = min(max(p, 0.0), 1.0)
    return min(int(math.floor(p * n_bins)), n_bins - 1)


def _pscaled(p: float) -> int:
    if math.isnan(p):
        return 0
    p = min(max(p, 0.0), 1.0)
    return int(math.floor(p * P_SCALE))


def observe(stats: Dict[str, object], *, conf: np.ndarray, surv: np.ndarray,
            win_len: Sequence[int], accept_len: Sequence[int], ceiling_len: Sequence[int],
            cu_seqlens: Sequence[int]) -> Dict[str, object]:
    """Add one step to the accumulator (in place; also returned)."""
    conf = np.asarray(conf, dtype=np.float32)
    surv = np.asarray(surv, dtype=np.float32)
    R, gamma = conf.shape
    n_bins = stats["bins"].shape[2]
    stats["steps"] += 1
    stats["req_steps"] += R
    for r in range(R):
        A = min(max(int(accept_len[r]), 0), gamma)
        C = min(max(int(ceiling_len[r]), 0), gamma)
        L = min(max(int(win_len[r]), 0), gamma)
        Lv = min(max(int(cu_seqlens[r + 1]) - int(cu_seqlens[r]) - 1, 0), gamma)
        stats["committed"] += A + 1
        stats["accepted"] += A
        stats["ceiling"] += C
        stats["window"] += L
        stats["verified"] += Lv
        stats["hist_window"][L] += 1
        stats["hist_accept"][A] += 1
        stats["hist_ceiling"][C] += 1
        stats["req_accepted"][r] += A
        stats["req_ceiling"][r] += C
        stats["req_window"][r] += L
        for k in range(1, gamma + 1):
            if k <= min(C + 1, Lv):
                p = float(conf[r, k - 1])
                cell = stats["bins"][KIND_CONDITIONAL, k - 1, _bin(p, n_bins)]
                cell[0] += 1
                cell[1] += _pscaled(p)
                cell[2] += int(k <= C)
            if k <= Lv:
                p = float(surv[r, k - 1])
                cell = stats["bins"][KIND_PREFIX, k - 1, _bin(p, n_bins)]
                cell[0] += 1
                cell[1] += _pscaled(p)
                cell[2] += int(C >= k)
    return stats


def ece(bins: np.ndarray) -> float:
    """Expected calibration error of bins [..., n_bins, 3] (count, sum of
    p * 2^32, hits), pooled over the leading axes."""
    b = np.asarray(bins, dtype=object).reshape(-1, np.asarray(bins).shape[-2], 3)
    count = b[..., 0].sum(axis=0)
    psum = b[..., 1].sum(axis=0)
    hits = b[..., 2].sum(axis=0)
    n = int(count.sum())
    if n == 0:
        return float("nan")
    return float(sum(abs(float(psum[i]) / P_SCALE - int(hits[i])) for i in range(len(count))) / n)


def utilisation(stats: Dict[str, object]) -> Dict[str, object]:
    """Accepted / ceiling, overall and per request (NaN where the ceiling is 0)."""
    def ratio(a, c):
        return float(a) / float(c) if c else float("nan")
    steps = stats["steps"]
    return {"accepted_over_ceiling": ratio(stats["accepted"], stats["ceiling"]),
            "committed_over_ceiling": ratio(stats["committed"], stats["ceiling"] + stats["req_steps"]),
            "per_request": [ratio(a, c) for a, c in zip(stats["req_accepted"], stats["req_ceiling"])],
            "per_request_committed": [ratio(a + steps, c + steps) for a, c in
                                      zip(stats["req_accepted"], stats["req_ceiling"])]}
