"""Pins of the oracle's observability outputs (SGLang DSpark blog,
"Observability"; DSpark digest, "Verification scheduling (system side)").

* c* = 1 - 1/2 ||p_d - p_t||_1: a hand-computed three-entry case, the
  identical-distribution and disjoint-support limits, NaN on unverified
  slots, and the empirical slot-1 acceptance rate of the oracle's own
  rejection sampler within a binomial band (an independent estimate of the
  same probability).
* Accumulator: a hand-tallied two-request step; static verification, where
  the window is the block, reaches utilisation 1; cap-accept never commits
  more than its ceiling.
* ECE: per-bin means equal scikit-learn's calibration_curve on the same
  pairs; closed forms (constant 0.5 against all hits: 0.5; outcomes drawn
  as Bernoulli(p): near 0).
"""
import numpy as np
import pytest
from scipy import special
from sklearn.calibration import calibration_curve

import oracle
import synth
from oracle.observe import (analytic_acceptance, new_stats, observe, ece, utilisation,
                            P_SCALE, KIND_CONDITIONAL, KIND_PREFIX)


def _logp(p):
    return np.log(np.asarray(p, dtype=np.float64))


def _one_slot(pd, pt):
    """R = 1, gamma = 1 inputs whose draft and target rows are exactly the
    distributions pd and pt (W1 = W2 = 0)."""
    V = len(pd)
    U = _logp(pd)[None, None, :]
    target = np.stack([_logp(pt), _logp(pt)])          # rows: slot 1, bonus
    W1 = np.zeros((V, 2))
    W2 = np.zeros((2, V))
    return target, [0, 2], [0], np.zeros((1, 1), dtype=np.int64), U, W1, W2


def test_hand_case():
    args = _one_slot([0.5, 0.3, 0.2], [0.2, 0.3, 0.5])
    c = analytic_acceptance(*args)
    assert c.shape == (1, 1)
    assert c[0, 0] == pytest.approx(0.7, abs=1e-12)    # 0.2 + 0.3 + 0.2


def test_limits():
    p = special.softmax(np.random.default_rng(0).normal(0, 2, 50))
    assert analytic_acceptance(*_one_slot(p, p))[0, 0] == pytest.approx(1.0, abs=1e-12)
    a = np.r_[np.full(25, 1 / 25), np.full(25, 1e-300)]
    b = a[::-1].copy()
    assert analytic_acceptance(*_one_slot(a, b))[0, 0] == pytest.approx(0.0, abs=1e-12)


def test_unverified_slots_are_nan():
    spec = synth.small_spec("obs", R=5, gamma=4, V=300, r=8, d=16, dtype="f32", seed=4)
    inp = synth.generate(spec)
    d = oracle.markov_draft(inp["U"], inp["W1"], inp["W2"], inp["anchor"], 1, 0, inp["req_ids"])
    win = [0, 4, 2, 1, 3]
    pk = oracle.pack_ragged(inp["anchor"], d["tokens"], win, [spec.R * 5], spec.R * 5)
    rows = np.concatenate([inp["target"][r, :pk["cu_seqlens"][r + 1] - pk["cu_seqlens"][r]]
                           for r in range(spec.R)])
    c = analytic_acceptance(rows, pk["cu_seqlens"], inp["anchor"], d["tokens"], inp["U"],
                            inp["W1"], inp["W2"])
    for r in range(spec.R):
        assert np.all(np.isfinite(c[r, :win[r]])) and np.all(np.isnan(c[r, win[r]:]))
        assert np.all((c[r, :win[r]] > 0) & (c[r, :win[r]] < 1))


@pytest.mark.slow
def test_matches_empirical_acceptance():
    # N requests share one block; the fraction that accept slot 1 estimates c*
    N, V = 12000, 16
    rng = np.random.default_rng(3)
    T = rng.normal(0, 1.5, (2, V))
    U1 = T[:1] + rng.normal(0, 1.0, (1, V))
    W1 = rng.normal(0, 0.3, (V, 4))
    W2 = rng.normal(0, 0.3, (4, V))
    U = np.broadcast_to(U1, (N, 1, V))
    target = np.broadcast_to(T, (N, 2, V))
    anchor = np.full(N, 2)
    d = oracle.markov_draft(U, W1, W2, anchor, 1, 0, np.arange(N))
    cu = np.arange(N + 1) * 2
    rows = target.reshape(N * 2, V)
    v = oracle.verify(rows, cu, anchor, d["tokens"], d["p_draft"], U, W1, W2, None,
                      oracle.VERIFY_STATIC, 1, 0, np.arange(N))
    c = analytic_acceptance(rows, cu, anchor, d["tokens"], U, W1, W2, requests=[0])[0, 0]
    rate = (v["accept_len"] >= 1).mean()
    sigma = np.sqrt(c * (1 - c) / N)
    assert abs(rate - c) < 4 * sigma, (rate, c)


# ---------------------------------------------------------------------------
# accumulator
# ---------------------------------------------------------------------------

def test_hand_tallied_step():
    gamma, n_bins = 3, 4
    conf = np.array([[0.9, 0.6, 0.3], [0.2, 0.8, 0.55]], dtype=np.float32)
    surv = np.array([[0.9, 0.54, 0.162], [0.2, 0.16, 0.088]], dtype=np.float32)
    # request 0: window 3, all verified, ceiling 1 (slot 2 rejected), A = 1
    # request 1: window 1, compact (1 verified slot), ceiling 0, A = 0
    s = observe(new_stats(2, gamma, n_bins), conf=conf, surv=surv, win_len=[3, 1],
                accept_len=[1, 0], ceiling_len=[1, 0], cu_seqlens=[0, 4, 6])
    assert (s["steps"], s["req_steps"], s["committed"], s["accepted"], s["ceiling"],
            s["window"], s["verified"]) == (1, 2, 3, 1, 1, 4, 4)
    assert s["hist_window"].tolist() == [0, 1, 0, 1]
    assert s["hist_accept"].tolist() == [1, 1, 0, 0]
    assert s["hist_ceiling"].tolist() == [1, 1, 0, 0]
    assert s["req_accepted"].tolist() == [1, 0] and s["req_window"].tolist() == [3, 1]
    b = s["bins"]
    # conditional pairs: r0 slot 1 (0.9, hit) bin 3; r0 slot 2 (0.6, miss) bin 2;
    # r1 slot 1 (0.2, miss) bin 0. r0 slot 3 is past the first rejection.
    assert b[KIND_CONDITIONAL, 0, 3].tolist() == [1, int(np.floor(np.float32(0.9) * 2.0 ** 32)), 1]
    assert b[KIND_CONDITIONAL, 1, 2].tolist() == [1, int(np.floor(np.float32(0.6) * 2.0 ** 32)), 0]
    assert b[KIND_CONDITIONAL, 0, 0].tolist() == [1, int(np.floor(np.float32(0.2) * 2.0 ** 32)), 0]
    assert b[KIND_CONDITIONAL, 2].sum() == 0
    assert b[KIND_CONDITIONAL, :, :, 0].sum() == 3
    # prefix pairs: every verified slot; hit while k <= ceiling
    assert b[KIND_PREFIX, :, :, 0].sum() == 4
    assert b[KIND_PREFIX, 0, 3].tolist()[2] == 1        # r0 k=1 (0.9), ceiling 1 >= 1
    assert b[KIND_PREFIX, 1, 2].tolist()[2] == 0        # r0 k=2 (0.54)
    assert b[KIND_PREFIX, 2, 0].tolist()[2] == 0        # r0 k=3 (0.162)
    assert b[KIND_PREFIX, 0, 0].tolist()[0] == 1        # r1 k=1 (0.2)


def _run_chain(vmode, seed, spec, inp):
    res = oracle.chain(inp, tiers=spec.tiers, staircase=spec.staircase, B_cap=spec.budgets[0],
                       verify_mode=vmode, seed=seed)
    return res


@pytest.mark.parametrize("vmode", [oracle.VERIFY_STATIC, oracle.VERIFY_CAP_ACCEPT])
def test_utilisation_bounds(vmode):
    spec = synth.small_spec("obs", R=6, gamma=4, V=300, r=8, d=16, dtype="f32", seed=5)
    inp = synth.generate(spec)
    st = new_stats(spec.R, spec.gamma, 8)
    for seed in range(6):
        res = _run_chain(vmode, seed, spec, inp)
        v = res["verify"]
        observe(st, conf=res["conf"]["conf"], surv=res["conf"]["surv"],
                win_len=res["sched"]["win_len"], accept_len=v["accept_len"],
                ceiling_len=v["ceiling"], cu_seqlens=res["pack"]["cu_seqlens"])
    u = utilisation(st)
    assert st["accepted"] <= st["ceiling"]
    if vmode == oracle.VERIFY_STATIC:
        assert u["accepted_over_ceiling"] == 1.0
        assert st["verified"] == 6 * spec.R * spec.gamma
    assert int(st["hist_accept"].sum()) == 6 * spec.R


def test_ece_matches_scikit_learn_bins():
    rng = np.random.default_rng(11)
    n, n_bins = 20000, 10
    p = rng.uniform(0.001, 0.999, n).astype(np.float32)
    y = (rng.uniform(size=n) < np.clip(p * 1.2 - 0.1, 0, 1)).astype(int)   # miscalibrated
    bins = np.zeros((n_bins, 3), dtype=object)
    for pi, yi in zip(p, y):
        i = min(int(np.floor(float(pi) * n_bins)), n_bins - 1)
        bins[i] += [1, int(np.floor(float(pi) * P_SCALE)), int(yi)]
    prob_true, prob_pred = calibration_curve(y, p.astype(np.float64), n_bins=n_bins,
                                             strategy="uniform")
    cnt = bins[:, 0].astype(float)
    keep = cnt > 0
    ours_true = (bins[keep, 2].astype(float) / cnt[keep])
    ours_pred = (bins[keep, 1].astype(float) / P_SCALE / cnt[keep])
    np.testing.assert_allclose(ours_true, prob_true, atol=1e-12)
    np.testing.assert_allclose(ours_pred, prob_pred, atol=1e-7)
    ref = float(np.sum(cnt[keep] / n * np.abs(prob_true - prob_pred)))
    assert ece(bins) == pytest.approx(ref, abs=1e-7)


def test_ece_closed_forms():
    n_bins = 8
    b = np.zeros((n_bins, 3), dtype=object)
    b[4] = [100, 100 * (P_SCALE // 2), 100]     # p = 0.5, every outcome a hit
    assert ece(b) == pytest.approx(0.5, abs=1e-12)
    rng = np.random.default_rng(2)
    p = rng.uniform(size=200000)
    y = rng.uniform(size=p.size) < p
    b = np.zeros((n_bins, 3), dtype=object)
    idx = np.minimum((p * n_bins).astype(int), n_bins - 1)
    for i in range(n_bins):
        m = idx == i
        b[i] = [int(m.sum()), int(np.floor(p[m] * P_SCALE).sum()), int(y[m].sum())]
    assert ece(b) < 0.01
