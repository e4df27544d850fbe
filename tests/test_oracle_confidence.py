"""Pins of the oracle's confidence head and prefix survival: closed forms with
scipy's logistic function, the concatenation order [h_k ; W1[x_{k-1}]], the
previous-token index (the anchor at slot 1) and monotone survival."""
import numpy as np
from scipy import special

import synth
from oracle.confidence import confidence


def _inputs(R=3, gamma=4, d=5, r=3, V=20, seed=0):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, 1, (R, gamma, d)).astype(np.float32)
    W1 = rng.normal(0, 1, (V, r)).astype(np.float32)
    anchor = rng.integers(0, V, R)
    tokens = rng.integers(0, V, (R, gamma))
    return h, W1, anchor, tokens


def test_zero_logit_gives_halves():
    h, W1, anchor, tokens = _inputs()
    w = np.zeros(h.shape[2] + W1.shape[1])
    out = confidence(h, W1, anchor, tokens, w, 0.0)
    assert np.all(out["conf"] == 0.5)
    assert out["surv"].tolist() == [[0.5, 0.25, 0.125, 0.0625]] * 3


def test_hidden_part_comes_first():
    h, W1, anchor, tokens = _inputs()
    d, r = h.shape[2], W1.shape[1]
    w = np.zeros(d + r)
    w[2] = 1.0                                      # third hidden component
    out = confidence(h, W1, anchor, tokens, w, 0.3)
    np.testing.assert_allclose(out["conf"], special.expit(h[:, :, 2].astype(np.float64) + 0.3), rtol=1e-14)


def test_markov_part_reads_previous_token():
    h, W1, anchor, tokens = _inputs()
    d, r = h.shape[2], W1.shape[1]
    w = np.zeros(d + r)
    w[d + 1] = 1.0                                  # second Markov component
    out = confidence(h, W1, anchor, tokens, w, -0.2)
    prev = np.concatenate([anchor[:, None], tokens[:, :-1]], axis=1)
    np.testing.assert_allclose(out["conf"], special.expit(W1[prev, 1].astype(np.float64) - 0.2), rtol=1e-14)


def test_survival_is_running_product_and_monotone():
    sp = synth.small_spec(R=6, gamma=7, V=300, r=16, d=32, dtype="bf16")
    inp = synth.generate(sp)
    rng = np.random.default_rng(1)
    tokens = rng.integers(0, sp.V, (sp.R, sp.gamma))
    out = confidence(inp["h"], inp["W1"], inp["anchor"], tokens, inp["w"], float(inp["b"]))
    c, a = out["conf"], out["surv"]
    np.testing.assert_allclose(a[:, 0], c[:, 0], rtol=0)
    np.testing.assert_allclose(a, np.cumprod(c, axis=1), rtol=1e-14)
    assert np.all(np.diff(a, axis=1) <= 0)
    a32 = a.astype(np.float32)
    assert np.all(np.diff(a32, axis=1) <= 0)        # still monotone after rounding


def test_inverse_temperature_scales_the_logit():
    h, W1, anchor, tokens = _inputs()
    rng = np.random.default_rng(4)
    w = rng.normal(0, 1, h.shape[2] + W1.shape[1])
    base = confidence(h, W1, anchor, tokens, w, 0.1)
    it = np.array([2.0, 0.5, 1.0, 3.0])
    sc = confidence(h, W1, anchor, tokens, w, 0.1, inv_temp=it)
    z = special.logit(base["conf"])
    np.testing.assert_allclose(sc["conf"], special.expit(z * it[None, :]), rtol=1e-9)
