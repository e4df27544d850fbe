"""GPU parity of sequential temperature scaling (dspark_sts_fit, and the
confidence head's logit output and inverse temperatures), through the C ABI.

* The head's logits and tempered confidences match the oracle teacher-forced
  on the GPU's drafts (1e-5).
* The fit: soft labels planted from known inverse temperatures are
  recovered exactly; on hard labels each position's ECE curve matches the
  oracle's, teacher-forced on the GPU's choices for the earlier positions
  (tolerance from the arithmetic: float32 products, plus the pairs that sit
  within 1e-5 of a bin edge), and the GPU's choice is a minimiser of the
  oracle's curve up to that tolerance.
* End to end: a decode loop's logits and analytic acceptances c* give soft
  labels prod c*; the fitted temperatures, fed back to the head, lower the
  ECE of the survivals against those labels.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.calibrate import sts_fit as oracle_fit, ece_of, apply
from tests.gpu_util import log, upload, to_dev, TOL

pytestmark = pytest.mark.gpu

# inverse temperatures 0.25 .. 3.97 in steps of 10%, and 1, as float32 values
BETAS = sorted({float(np.float32(0.25 * 1.1 ** i)) for i in range(30)} | {1.0})
N_BINS = 16


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()
    return dv


def _edge_allowance(a, n_bins):
    s = np.asarray(a, dtype=np.float64) * n_bins
    near = np.abs(s - np.round(s)) < 1e-5 * n_bins
    return (2.0 * near.sum() + 1.0) / max(len(a), 1)


def check_fit(dv, z, y, mask, label):
    import torch
    zt, yt = to_dev(z.astype(np.float32)), to_dev(y.astype(np.float32))
    mt = None if mask is None else to_dev(mask.astype(np.uint8))
    bt = to_dev(np.array(BETAS, dtype=np.float32))
    inv, ece = dv.sts_fit(zt, yt, bt, n_bins=N_BINS, mask=mt)
    torch.cuda.synchronize()
    inv, ece = inv.cpu().numpy(), ece.cpu().numpy()
    m = np.ones_like(z, dtype=bool) if mask is None else mask.astype(bool)
    # teacher-forced: the oracle's curve at position k uses the GPU's betas before k
    ref = oracle_fit(z.astype(np.float32), y, m, BETAS, N_BINS, fixed=inv)
    a_prev = np.ones(z.shape[0])
    for k in range(z.shape[1]):
        a_best = a_prev * 1.0 / (1.0 + np.exp(-z[:, k].astype(np.float64) * inv[k]))
        tol = 1e-5 + _edge_allowance(a_best[m[:, k]], N_BINS)
        for j, beta in enumerate(BETAS):
            aj = a_prev * 1.0 / (1.0 + np.exp(-z[:, k].astype(np.float64) * beta))
            tj = 1e-5 + _edge_allowance(aj[m[:, k]], N_BINS)
            assert abs(ece[k, j] - ref["ece"][k, j]) <= tj, (label, k, j, ece[k, j], ref["ece"][k, j])
        assert float(inv[k]) in BETAS, (label, k, inv[k])
        j = BETAS.index(float(inv[k]))
        assert ref["ece"][k, j] <= ref["ece"][k].min() + 2 * tol, (label, k, inv[k])
        a_prev = a_best
    return inv, ece


def test_soft_labels_recover_planted_temperatures(dv):
    rng = np.random.default_rng(0)
    z = rng.normal(1.0, 2.0, (20000, 5)).astype(np.float32)
    beta = np.array([BETAS[i] for i in (3, 10, 15, 7, 21)], dtype=np.float32)
    y = apply(z, beta)["surv"].astype(np.float32)
    inv, ece = check_fit(dv, z, y, None, "planted")
    np.testing.assert_array_equal(inv, beta)
    log(f"[sts] planted: recovered {inv.tolist()}, ECE at the fit {ece.min(axis=1).tolist()}")


@pytest.mark.parametrize("N", [1, 777, 50000])
def test_hard_labels_match_the_oracle(dv, N):
    rng = np.random.default_rng(N)
    z = rng.normal(0.5, 2.5, (N, 6)).astype(np.float32)
    prod = apply(z, [0.6, 1.3, 0.9, 2.0, 0.4, 1.1])["surv"]
    y = (rng.uniform(size=prod.shape) < prod).astype(np.float32)
    mask = rng.uniform(size=z.shape) < 0.85
    check_fit(dv, z, y, mask, f"hard N={N}")


def test_logits_and_tempered_confidence(dv):
    import torch
    spec = synth.small_spec("sts", R=20, gamma=5, V=3000, r=64, d=96, dtype="bf16", seed=5)
    inp = synth.generate(spec)
    dev, _ = upload(inp, spec)
    inv = np.array([0.5, 0.8, 1.0, 1.6, 2.5], dtype=np.float32)
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=spec.budgets[0], verify_mode=0,
                  inv_temp=to_dev(inv), keep_logits=True)
    ch.run()
    torch.cuda.synchronize()
    res = ch.results()
    ref = oracle.confidence(inp["h"], inp["W1"], inp["anchor"], res["tokens"], inp["w"],
                            float(inp["b"]), inv)
    np.testing.assert_allclose(res["logit"], ref["logit"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(res["conf"], ref["conf"], rtol=0, atol=TOL)
    np.testing.assert_allclose(res["surv"], ref["surv"], rtol=0, atol=TOL)


def test_fit_on_a_decode_loop_lowers_the_ece(dv):
    import torch
    spec = synth.small_spec("sts_loop", R=64, gamma=5, V=3000, r=64, d=96, dtype="bf16", seed=9,
                            W_std=0.3, b=1.5)
    inp = synth.generate(spec)
    dev, _ = upload(inp, spec)
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=spec.budgets[0],
                  verify_mode=2, analytic=True, keep_logits=True, seed=1, step=0)
    steps = ch.decode(24, lag=2, record=True)
    torch.cuda.synchronize()
    z = np.concatenate([s["logit"] for s in steps]).astype(np.float32)
    y = np.cumprod(np.concatenate([s["cstar"] for s in steps]), axis=1).astype(np.float32)
    assert np.all(np.isfinite(y))                      # cap-accept verifies every slot
    inv, _ = check_fit(dv, z, y, None, "loop")
    surv0 = apply(z, np.ones(spec.gamma))["surv"]
    surv1 = apply(z, inv)["surv"]
    e0 = [ece_of(surv0[:, k], y[:, k], N_BINS) for k in range(spec.gamma)]
    e1 = [ece_of(surv1[:, k], y[:, k], N_BINS) for k in range(spec.gamma)]
    assert sum(e1) < sum(e0)
    # the chain with the fitted temperatures reproduces those survivals
    ch2 = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=spec.budgets[0], verify_mode=2,
                   inv_temp=to_dev(inv), seed=1, step=0)
    ch2.run()
    torch.cuda.synchronize()
    r2 = ch2.results()
    np.testing.assert_allclose(r2["surv"], apply(steps[0]["logit"], inv)["surv"], rtol=0, atol=TOL)
    log(f"[sts] decode-loop fit: inv_temp {inv.tolist()}, ECE per position {np.round(e0, 4).tolist()}"
        f" -> {np.round(e1, 4).tolist()}")
