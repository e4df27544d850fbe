"""Pins of the oracle's sequential temperature scaling (DSpark digest,
"Verification scheduling (system side)").

* Recovery: with soft labels that are exactly the prefix products of a
  planted per-position inverse temperature, the ECE at the planted values is 0
  and the fit returns them; with hard labels drawn as Bernoulli of those
  products, the fit lands within one grid step.
* The ECE it minimises equals scikit-learn's calibration_curve ECE on the same
  pairs (the library pin of the binning), and the observability
  accumulator's ECE on the same bins.
* A positive temperature keeps each position's ranking.
* The confidence oracle's logit output reproduces its confidences under any
  inverse temperature.
"""
import numpy as np
import pytest
from sklearn.calibration import calibration_curve

import oracle
import synth
from oracle.calibrate import sts_fit, ece_of, apply
from oracle.observe import P_SCALE

BETAS = [round(0.25 * 1.1 ** i, 6) for i in range(30)]      # 0.25 .. 3.97


def _planted(N=6000, gamma=5, seed=0):
    rng = np.random.default_rng(seed)
    z = rng.normal(1.0, 2.0, (N, gamma))
    beta = np.array([BETAS[i] for i in (3, 10, 14, 7, 20)][:gamma])
    prod = apply(z, beta)["surv"]
    return z, beta, prod, rng


def test_soft_labels_recover_the_planted_temperatures():
    z, beta, prod, _ = _planted()
    fit = sts_fit(z, prod, np.ones_like(z, dtype=bool), BETAS, 16)
    np.testing.assert_allclose(fit["inv_temp"], beta)
    assert np.all(fit["ece_after"] < 1e-12)
    assert np.all(fit["ece_before"] > fit["ece_after"])


@pytest.mark.slow
def test_hard_labels_land_within_one_grid_step():
    z, beta, prod, rng = _planted(N=200000, seed=1)
    y = (rng.uniform(size=prod.shape) < prod).astype(float)
    fit = sts_fit(z, y, np.ones_like(z, dtype=bool), BETAS, 16)
    for k in range(z.shape[1]):
        i_fit, i_true = BETAS.index(fit["inv_temp"][k]), BETAS.index(beta[k])
        assert abs(i_fit - i_true) <= 1, (k, fit["inv_temp"][k], beta[k])


def test_mask_drops_unlabelled_pairs():
    z, beta, prod, _ = _planted(N=3000)
    mask = np.ones_like(z, dtype=bool)
    mask[::3, 2:] = False
    y = prod.copy()
    y[~mask] = 1.0 - y[~mask]                               # garbage where masked
    fit = sts_fit(z, y, mask, BETAS, 16)
    np.testing.assert_allclose(fit["inv_temp"], beta)


def test_ece_matches_scikit_learn_and_the_accumulator():
    rng = np.random.default_rng(4)
    p = rng.uniform(0.001, 0.999, 5000)
    y = (rng.uniform(size=p.size) < p ** 1.3).astype(float)
    n_bins = 10
    prob_true, prob_pred = calibration_curve(y, p, n_bins=n_bins, strategy="uniform")
    cnt = np.bincount(np.minimum((p * n_bins).astype(int), n_bins - 1), minlength=n_bins)
    cnt = cnt[cnt > 0]
    ref = float(np.sum(cnt / p.size * np.abs(prob_true - prob_pred)))
    assert ece_of(p, y, n_bins) == pytest.approx(ref, abs=1e-12)
    bins = np.zeros((n_bins, 3), dtype=object)
    for pi, yi in zip(p.astype(np.float32), y):
        i = min(int(np.floor(float(pi) * n_bins)), n_bins - 1)
        bins[i] += [1, int(np.floor(float(pi) * P_SCALE)), int(yi)]
    assert oracle.ece(bins) == pytest.approx(ece_of(p.astype(np.float32), y, n_bins), abs=1e-7)


def test_temperature_keeps_the_ranking():
    z, _, _, _ = _planted(N=500)
    c = apply(z, [0.3, 0.7, 1.0, 2.5, 3.9])["conf"]
    for k in range(z.shape[1]):
        assert np.array_equal(np.argsort(z[:, k], kind="stable"), np.argsort(c[:, k], kind="stable"))


def test_confidence_logit_reproduces_confidence():
    spec = synth.small_spec("cal", R=6, gamma=4, V=200, r=8, d=16, dtype="f32", seed=2)
    inp = synth.generate(spec)
    tokens = np.random.default_rng(0).integers(0, spec.V, (spec.R, spec.gamma))
    inv = np.array([0.5, 1.0, 1.7, 3.0])
    c = oracle.confidence(inp["h"], inp["W1"], inp["anchor"], tokens, inp["w"], float(inp["b"]), inv)
    np.testing.assert_allclose(apply(c["logit"], inv)["conf"], c["conf"], rtol=1e-13)
    np.testing.assert_allclose(apply(c["logit"], inv)["surv"], c["surv"], rtol=1e-12)
