"""Cost table and global top-B prefix scheduler (oracle, exact integers).

Sources:
  * DSpark digest, "Verification scheduling (system side)": the hardware-aware
    prefix scheduler maximises global throughput Theta = tau * SPS, where SPS is
    the engine's steps-per-second capacity curve profiled once into a cost
    table; since the prefix survival a_{r,j} does not grow with j, slots are
    admitted greedily in descending survival with an O(1) table update, and
    admission stops the first time throughput drops (non-anticipating, hence
    lossless).
  * DSpark digest, "Infra (online production @ DeepSeek-V4)": in production
    the cut length is predicted from confidences of two steps earlier; that
    causal barrier lets the search drop the early stop and search the jagged
    SPS curve globally, while the current step's candidates are still ranked by
    the latest cumulative confidence.
  * vLLM adaptive verification page, "DSpark confidence-scheduling mechanism":
    global top-B over all requests' draft slots; each request's selection is a
    contiguous prefix because survival decreases with the slot; the objective
    is expected tokens (one per request plus the survivals of the B best
    slots) against step cost.
  * SGLang DSpark blog, "Cost-table profiling": step time is additive,
    T = bias + alpha(bs) + theta(M) with M = bs + K, K the extra verify tokens.
  * vLLM adaptive verification page, "Technical implementation & CUDA graphs":
    profiled cost curves are forced monotone; graph padding makes the cost a
    staircase (a 121-token batch costs the 128-token graph).

Readings (where the pages leave a step open):
  * tau = R + sum of the selected survivals (one token per request plus the
    expected accepted drafts); SPS is read at the verify-forward size
    M = R + K.
  * Fixed point: a_q = floor(clamp(a, 0, 1) * 2**20), NaN -> 0, then made
    non-increasing along each request's slots by a running minimum (a no-op for
    products of c <= 1); tau_K = R * 2**20 + sum of the K largest a_q;
    Theta_K = tau_K * sps_milli[R + K] as an exact integer.
  * Keys are ordered by (a_q descending, request ascending, slot ascending).
  * K ranges over 0..min(B, R*gamma, M_max - R).
  * ARGMAX: the smallest K maximising Theta over the budget array.
    GREEDY: admit while Theta strictly increases, stop at the first
    non-increase. FIXED: K is given (clamped to the range).
  * The selected set is always the K best keys of the current survival array;
    L_r counts request r's selected slots (a prefix, by the ordering).
  * Cost table: raw step time T(M) -> running maximum over M (monotone) ->
    optional staircase T_eff(M) = T_mono(min(tier(M), M_max)), tier(M) the
    smallest captured tier >= M, infeasible (0) above the top tier ->
    sps_milli(M) = floor(1000 / T_eff + 0.5).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

SCHED_ARGMAX = 0
SCHED_GREEDY = 1
SCHED_FIXED = 2

QBITS = 20
QONE = 1 << QBITS
U32_MAX = (1 << 32) - 1


def cost_table_prepare(raw_T: Sequence[float], tiers: Sequence[int], staircase: bool) -> List[int]:
    """raw_T[M], M = 0..M_max, step time in seconds -> sps_milli[M] (ints)."""
    raw = [float(t) for t in raw_T]
    M_max = len(raw) - 1
    mono: List[float] = []
    run = -math.inf
    for t in raw:
        if t > run:
            run = t
        mono.append(run)
    out: List[int] = []
    for M in range(M_max + 1):
        if staircase:
            cands = [t for t in tiers if t >= M]
            if not cands:
                out.append(0)
                continue
            T = mono[min(min(cands), M_max)]
        else:
            T = mono[M]
        if not (T > 0.0) or math.isinf(T):
            out.append(0)
            continue
        v = math.floor(1000.0 / T + 0.5)
        out.append(int(min(max(v, 0), U32_MAX)))
    return out


def quantize_survival(a: float) -> int:
    """floor(clamp(a, 0, 1) * 2**20), NaN -> 0 (exact: a is a float32 value)."""
    a = float(a)
    if math.isnan(a):
        return 0
    a = min(max(a, 0.0), 1.0)
    return int(math.floor(a * QONE))


def _quantized_prefix(surv: np.ndarray) -> List[List[int]]:
    R, gamma = surv.shape
    out = []
    for r in range(R):
        row, run = [], QONE
        for j in range(gamma):
            q = quantize_survival(surv[r, j])
            run = min(run, q)
            row.append(run)
        out.append(row)
    return out


def schedule_topb(surv: np.ndarray, sps_milli: Sequence[int], B_cap: int, mode: int,
                  K_fixed: int = 0, surv_budget: Optional[np.ndarray] = None) -> Dict[str, object]:
    """surv [R, gamma] float32 survivals; sps_milli [M_max + 1].

    Returns win_len [R] (ints), K, and the Theta curve for inspection."""
    surv = np.asarray(surv, dtype=np.float32)
    R, gamma = surv.shape
    M_max = len(sps_milli) - 1
    aq = _quantized_prefix(surv)
    keys = sorted(((r, j) for r in range(R) for j in range(gamma)),
                  key=lambda rj: (-aq[rj[0]][rj[1]], rj[0], rj[1]))
    K_cap = max(0, min(int(B_cap), R * gamma, M_max - R))

    theta: List[int] = []
    if mode == SCHED_FIXED:
        K = min(max(int(K_fixed), 0), K_cap)
    else:
        bq = aq if surv_budget is None else _quantized_prefix(np.asarray(surv_budget, dtype=np.float32))
        vals = sorted((bq[r][j] for r in range(R) for j in range(gamma)), reverse=True)
        tau = R * QONE
        for Kc in range(K_cap + 1):
            if Kc:
                tau += vals[Kc - 1]
            theta.append(tau * int(sps_milli[R + Kc]))
        if mode == SCHED_ARGMAX:
            best = max(theta)
            K = theta.index(best)
        elif mode == SCHED_GREEDY:
            K = 0
            while K < K_cap and theta[K + 1] > theta[K]:
                K += 1
        else:
            raise ValueError(f"unknown scheduler mode {mode}")
    win = [0] * R
    for (r, j) in keys[:K]:
        win[r] += 1
    return {"win_len": win, "K": K, "theta": theta, "K_cap": K_cap}
