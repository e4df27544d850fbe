"""Pins of the oracle's cost table and global top-B prefix scheduler.

* brute force over every per-request prefix vector on tiny batches, with
  throughput computed from scratch as exact rationals;
* greedy == argmax on a linear SPS table (marginal gain is non-increasing);
* a staircase table where greedy's early stop is strictly worse than the
  unconstrained search (the reason production drops the early stop);
* hand-built cost tables (monotone enforcement, staircase tiers).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle.schedule import (cost_table_prepare, quantize_survival, schedule_topb,
                             SCHED_ARGMAX, SCHED_GREEDY, SCHED_FIXED)


def _monotone_surv(rng, R, gamma):
    c = rng.uniform(0.05, 1.0, (R, gamma)).astype(np.float32)
    a = np.ones(R, dtype=np.float32)
    out = np.empty((R, gamma), dtype=np.float32)
    for j in range(gamma):
        a = (a * c[:, j]).astype(np.float32)
        out[:, j] = a
    return out


def _brute(surv, sps, B_cap):
    """Best throughput over all prefix vectors, from first principles:
    expected tokens = R + sum of the kept survivals (each quantised to 2^-20
    and made non-increasing per request), speed = sps[R + total drafts]."""
    R, gamma = surv.shape
    M_max = len(sps) - 1
    q = []
    for r in range(R):
        row, run = [], 1 << 20
        for j in range(gamma):
            v = surv[r, j]
            v = 0.0 if np.isnan(v) else min(max(float(v), 0.0), 1.0)
            run = min(run, int(np.floor(v * (1 << 20))))
            row.append(run)
        q.append(row)
    best, best_vecs = None, []
    for L in itertools.product(range(gamma + 1), repeat=R):
        K = sum(L)
        if K > B_cap or R + K > M_max:
            continue
        tau = Fraction(R) + sum(Fraction(q[r][j], 1 << 20) for r in range(R) for j in range(L[r]))
        th = tau * sps[R + K]
        if best is None or th > best:
            best, best_vecs = th, [L]
        elif th == best:
            best_vecs.append(L)
    return best, best_vecs


@pytest.mark.parametrize("seed", range(12))
def test_argmax_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    surv = _monotone_surv(rng, R, gamma)
    M_max = R * (gamma + 1)
    # random positive decreasing-ish table with plateaus (staircase flavour)
    sps = sorted((int(x) for x in rng.integers(1000, 400000, M_max + 1)), reverse=True)
    sps = [sps[min(M_max, (m // 2) * 2)] for m in range(M_max + 1)]
    B_cap = int(rng.integers(0, R * gamma + 1))
    out = schedule_topb(surv, sps, B_cap, SCHED_ARGMAX)
    best, vecs = _brute(surv, sps, B_cap)
    K = out["K"]
    assert out["theta"][K] == best * (1 << 20)
    assert tuple(out["win_len"]) in vecs
    assert sum(out["win_len"]) == K
    # smallest K among maximisers
    assert K == min(sum(v) for v in vecs)


def test_greedy_equals_argmax_on_linear_sps():
    rng = np.random.default_rng(7)
    for _ in range(40):
        R, gamma = int(rng.integers(1, 9)), int(rng.integers(1, 8))
        surv = _monotone_surv(rng, R, gamma)
        M_max = R * (gamma + 1)
        s0, s1 = 1_000_000, 20_000
        sps = [max(s0 - s1 * m, 1) for m in range(M_max + 1)]
        B = R * gamma
        g = schedule_topb(surv, sps, B, SCHED_GREEDY)
        a = schedule_topb(surv, sps, B, SCHED_ARGMAX)
        assert g["theta"][g["K"]] == a["theta"][a["K"]]
        assert g["K"] == a["K"] and g["win_len"] == a["win_len"]


def test_greedy_stops_early_on_a_staircase():
    # Two requests, survivals high; SPS drops sharply at M = 3 then stays flat
    # to M = 6: greedy stops at the drop, the global search admits everything.
    surv = np.array([[0.95, 0.9], [0.94, 0.89]], dtype=np.float32)
    sps = [100, 100, 100, 100, 60, 60, 60]          # M = 0..6
    g = schedule_topb(surv, sps, 4, SCHED_GREEDY)
    a = schedule_topb(surv, sps, 4, SCHED_ARGMAX)
    assert g["K"] == 1 and a["K"] == 4
    assert a["theta"][4] > g["theta"][1]


def test_fixed_budget_and_prefix_closure():
    rng = np.random.default_rng(3)
    surv = _monotone_surv(rng, 5, 6)
    sps = [1] * 36
    for K in (0, 1, 7, 30, 99, -4):
        out = schedule_topb(surv, sps, 30, SCHED_FIXED, K_fixed=K)
        assert out["K"] == min(max(K, 0), 30)
        assert sum(out["win_len"]) == out["K"]
    # the K best keys: every kept slot beats every dropped slot
    out = schedule_topb(surv, sps, 30, SCHED_FIXED, K_fixed=13)
    kept = [surv[r, j] for r in range(5) for j in range(out["win_len"][r])]
    dropped = [surv[r, j] for r in range(5) for j in range(out["win_len"][r], 6)]
    assert min(kept) >= max(dropped)


def test_budget_cap_and_table_domain():
    rng = np.random.default_rng(4)
    surv = _monotone_surv(rng, 4, 5)
    sps = [10 ** 6] * 10 + [0] * 15                   # M_max = 24
    out = schedule_topb(surv, sps, 100, SCHED_ARGMAX)
    assert out["K_cap"] == min(100, 20, 24 - 4)
    assert out["K"] <= 6                              # M = 4 + K must stay < 10


def test_budget_array_drives_k_but_not_selection():
    surv = np.array([[0.9, 0.8, 0.1], [0.7, 0.6, 0.5]], dtype=np.float32)
    budget = np.array([[0.5, 0.4, 0.05], [0.45, 0.3, 0.05]], dtype=np.float32)
    sps = [100, 100, 100, 90, 80, 70, 60, 50, 40]
    cur = schedule_topb(surv, sps, 6, SCHED_ARGMAX)
    stale = schedule_topb(surv, sps, 6, SCHED_ARGMAX, surv_budget=budget)
    assert (stale["K"], cur["K"]) == (2, 3)
    # selection = the stale K best of the *current* survivals
    fixed = schedule_topb(surv, sps, 6, SCHED_FIXED, K_fixed=stale["K"])
    assert stale["win_len"] == fixed["win_len"]


def test_quantisation_edges():
    assert quantize_survival(float("nan")) == 0
    assert quantize_survival(-0.5) == 0
    assert quantize_survival(1.0) == 1 << 20
    assert quantize_survival(2.0) == 1 << 20
    assert quantize_survival(0.5) == 1 << 19
    assert quantize_survival(np.float32(0.1)) == int(np.floor(float(np.float32(0.1)) * 2 ** 20))


def test_nan_and_nonmonotone_input_stays_prefix():
    surv = np.array([[0.3, float("nan"), 0.9], [0.5, 0.6, 0.7]], dtype=np.float32)
    out = schedule_topb(surv, [1] * 9, 6, SCHED_FIXED, K_fixed=4)
    # request 0: 0.3 then NaN -> 0, then 0.9 capped by the running minimum 0
    # request 1: 0.5, then 0.6 and 0.7 capped at 0.5
    assert out["win_len"] == [1, 3]


def test_cost_table_monotone_and_staircase():
    raw = [1.0, 0.9, 1.2, 1.1, 1.5, 1.4, 1.6, 1.55, 2.0]     # M = 0..8, noisy
    flat = cost_table_prepare(raw, [4, 8], staircase=False)
    assert flat == [1000, 1000, 833, 833, 667, 667, 625, 625, 500]
    st = cost_table_prepare(raw, [4, 8], staircase=True)
    # tier(M) = 4 for M <= 4 (T_mono(4) = 1.5), 8 for 5..8 (T_mono(8) = 2.0)
    assert st == [667] * 5 + [500] * 4
    st2 = cost_table_prepare(raw, [2, 5], staircase=True)
    assert st2[6:] == [0, 0, 0]                       # above the top tier


def test_cost_table_linear_sps_roundtrip():
    M = np.arange(33)
    sps = 1_000_000 - 20_000 * M
    raw = 1000.0 / sps
    assert cost_table_prepare(raw, [8, 16, 32], staircase=False) == sps.tolist()
