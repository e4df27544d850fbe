"""Pins of the oracle's Markov draft head.

* inverse CDF: brute-force hand cases;
* softmax / log-sum-exp: against scipy;
* row lookup by the previous token: a full-rank head (W1 = identity) must add
  row x_{k-1} of W2 to the base logits;
* sampling: chi-square of drafted tokens against scipy's softmax, per slot and
  conditioned on the previous token, with a Markov head strong enough to matter.
"""
import numpy as np
import pytest
from scipy import special, stats

import synth
from oracle.markov import inverse_cdf, markov_step, markov_draft, widen, markov_logits


def test_inverse_cdf_hand_cases():
    w = np.array([1.0, 2.0, 3.0, 4.0])          # C = 1, 3, 6, 10
    assert inverse_cdf(w, 0.0) == 0
    assert inverse_cdf(w, 0.999) == 0
    assert inverse_cdf(w, 1.0) == 1             # strict: C_0 = 1 is not > 1
    assert inverse_cdf(w, 2.5) == 1
    assert inverse_cdf(w, 3.0) == 2
    assert inverse_cdf(w, 9.999) == 3
    assert inverse_cdf(w, 10.0) == 3            # past the end: last positive id
    w0 = np.array([0.0, 1.0, 0.0, 2.0, 0.0])    # zero weights are never drawn
    assert inverse_cdf(w0, 0.0) == 1
    assert inverse_cdf(w0, 1.0) == 3
    assert inverse_cdf(w0, 3.0) == 3


def test_widen_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3E80, 0x4049], dtype=np.uint16)
    assert widen(bits).tolist() == [1.0, -2.0, 0.0, 0.25, 3.140625]


def test_step_probabilities_match_scipy():
    rng = np.random.default_rng(1)
    R, V, r = 5, 300, 16
    U = rng.normal(0, 3, (R, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.5, (r, V)).astype(np.float32)
    x_prev = rng.integers(0, V, R)
    u = rng.uniform(0, 1, R)
    rec = markov_step(U, W1, W2, x_prev, u)
    for i in range(R):
        z = U[i].astype(np.float64) + W1[x_prev[i]].astype(np.float64) @ W2.astype(np.float64)
        p = special.softmax(z)
        np.testing.assert_allclose(rec["p"][i], p[rec["tokens"][i]], rtol=1e-12)
        np.testing.assert_allclose(rec["lse"][i], special.logsumexp(z), rtol=1e-13)
        # the draw sits where the cumulative probability crosses u
        c = np.cumsum(p)
        x = rec["tokens"][i]
        assert (c[x - 1] if x else 0.0) <= u[i] + 1e-12 and c[x] > u[i] - 1e-12


def test_zero_markov_factor_is_plain_categorical():
    rng = np.random.default_rng(2)
    V = 40
    U = rng.normal(0, 2, (1, V))
    W1 = np.zeros((V, 8))
    W2 = rng.normal(0, 1, (8, V))
    rec = markov_step(U, W1, W2, [3], [0.37])
    p = special.softmax(U[0])
    assert rec["tokens"][0] == int(np.searchsorted(np.cumsum(p), 0.37, side="right"))
    np.testing.assert_allclose(rec["p"][0], p[rec["tokens"][0]], rtol=1e-12)


def test_row_lookup_uses_previous_token():
    # W1 = identity (r = V): the bias is row x_prev of W2, not a column.
    rng = np.random.default_rng(3)
    V = 12
    U = rng.normal(0, 1, (V,))
    W1 = np.eye(V)
    Bm = rng.normal(0, 1, (V, V))
    for x_prev in (0, 5, 11):
        z = markov_logits(U, W1, Bm, x_prev)
        np.testing.assert_allclose(z, U + Bm[x_prev], rtol=0, atol=1e-15)
        assert not np.allclose(z, U + Bm[:, x_prev])


def _chisq(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.concatenate([counts[keep], [counts[~keep].sum()]])
    e = np.concatenate([exp[keep], [exp[~keep].sum()]])
    if e[-1] == 0:
        obs, e = obs[:-1], e[:-1]
    return stats.chisquare(obs, e).pvalue


@pytest.mark.slow
def test_draft_chi_square_per_slot_and_conditional():
    """Many requests share one block of logits and one anchor; their Philox
    streams differ by request id. Slot-1 tokens must follow
    softmax(U_1 + W1[x_0] W2); slot-2 tokens, grouped by x_1, must follow
    softmax(U_2 + W1[x_1] W2) (a strong head so the dependence is visible)."""
    rng = np.random.default_rng(11)
    N, V, r, gamma = 12000, 16, 8, 2
    U1 = rng.normal(0, 1.5, (gamma, V))
    W1 = rng.normal(0, 0.7, (V, r))
    W2 = rng.normal(0, 0.7, (r, V))
    U = np.broadcast_to(U1, (N, gamma, V)).copy()
    anchor = np.full(N, 4)
    out = markov_draft(U, W1, W2, anchor, seed=9, step=0, req_ids=np.arange(N))
    x1, x2 = out["tokens"][:, 0], out["tokens"][:, 1]
    p1 = special.softmax(U1[0] + W1[4] @ W2)
    assert _chisq(np.bincount(x1, minlength=V).astype(float), p1) > 1e-4
    for v in np.argsort(-np.bincount(x1, minlength=V))[:3]:
        sel = x2[x1 == v]
        p2 = special.softmax(U1[1] + W1[v] @ W2)
        assert _chisq(np.bincount(sel, minlength=V).astype(float), p2) > 1e-4
    # and the dependence is real: the conditionals differ between x_1 values
    a, b = np.argsort(-np.bincount(x1, minlength=V))[:2]
    pa = special.softmax(U1[1] + W1[a] @ W2)
    pb = special.softmax(U1[1] + W1[b] @ W2)
    assert 0.5 * np.abs(pa - pb).sum() > 0.05


def test_draft_teacher_forcing_conditions_on_given_tokens():
    sp = synth.small_spec(R=3, gamma=3, V=200, r=8, d=8, dtype="f32")
    inp = synth.generate(sp)
    teacher = np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9]])
    out = markov_draft(inp["U"], inp["W1"], inp["W2"], inp["anchor"], 0, 0, inp["req_ids"],
                       teacher_tokens=teacher)
    assert out["steps"][1]["x_prev"].tolist() == teacher[:, 0].tolist()
    assert out["steps"][2]["x_prev"].tolist() == teacher[:, 1].tolist()
    assert out["steps"][0]["x_prev"].tolist() == inp["anchor"].tolist()
