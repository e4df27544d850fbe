"""GPU parity of the observability outputs, through the C ABI.

* dspark_analytic_accept: c* of every verified slot against the oracle's
  1 - 1/2 |p_d - p_t|_1, teacher-forced on the GPU's drafts, windows and
  packing (1e-5); NaN exactly on the slots no packed row verifies.
* dspark_observe: after several decode steps the device block equals, word
  for word, the oracle accumulator fed the GPU's own per-step outputs (all
  counts are integers); a graph-replayed loop leaves the same block and the
  same c* as the eager loop.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import log, upload, PackedView, sample_requests, factors64, TOL

pytestmark = pytest.mark.gpu

MODES = {"static": 0, "compact": 1, "cap_accept": 2}
N_BINS = 16


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()
    return dv


def _oracle_block(steps, R, gamma):
    st = oracle.new_stats(R, gamma, N_BINS)
    for s in steps:
        oracle.observe(st, conf=s["conf"], surv=s["surv"], win_len=s["win_len"],
                       accept_len=s["accept_len"], ceiling_len=s["ceiling_len"],
                       cu_seqlens=s["cu_seqlens"])
    return st


def _compare_block(got, ref, label):
    for key in ("steps", "req_steps", "committed", "accepted", "ceiling", "window", "verified"):
        assert got[key] == ref[key], (label, key, got[key], ref[key])
    for key in ("hist_window", "hist_accept", "hist_ceiling", "req_accepted", "req_ceiling",
                "req_window", "bins"):
        assert np.array_equal(np.asarray(got[key], dtype=object), np.asarray(ref[key], dtype=object)), (label, key)


def _check_cstar(steps, inp, reqs, label):
    W1, W2 = factors64(inp)
    for t, s in enumerate(steps):
        rows = PackedView(inp["target"], s["cu_seqlens"])
        ref = oracle.analytic_acceptance(rows, s["cu_seqlens"], s["anchor"], s["tokens"], inp["U"],
                                         W1, W2, requests=[int(r) for r in reqs])
        got = s["cstar"]
        for r in reqs:
            nan_g, nan_o = np.isnan(got[r]), np.isnan(ref[r])
            assert np.array_equal(nan_g, nan_o), (label, t, r, got[r], ref[r])
            np.testing.assert_allclose(got[r][~nan_g], ref[r][~nan_o], rtol=0, atol=TOL,
                                       err_msg=f"{label} t{t} r{r}")


def run_observed(dv, spec, vmode, lag, n_steps, sample=None, graph_check=True):
    import torch
    label = f"{spec.name}/{vmode}/lag{lag}"
    log(f"[observe] {label}: R={spec.R} gamma={spec.gamma} V={spec.V} r={spec.r} "
        f"dtype={spec.dtype} steps={n_steps}")
    inp = synth.generate(spec)
    dev, sps = upload(inp, spec)
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=spec.budgets[0],
                  verify_mode=MODES[vmode], seed=9, step=50, observe_bins=N_BINS, analytic=True)
    steps = ch.decode(n_steps, lag=lag, record=True)
    torch.cuda.synchronize()
    reqs = np.arange(spec.R) if sample is None else sample_requests(spec.R, sample)
    _check_cstar(steps, inp, reqs, label)
    got = ch.observe_summary()
    _compare_block(got, _oracle_block(steps, spec.R, spec.gamma), label)
    log(f"[observe] {label}: c* and block ok; utilisation {got['utilisation']:.3f}, "
        f"ECE conditional {got['ece_conditional']:.4f} prefix {got['ece_prefix']:.4f}")
    if graph_check:
        eager_block = ch.obs_block.cpu().numpy().copy()
        ch.reset()
        ch.obs_block.zero_()
        graphed = ch.decode(n_steps, lag=lag, graph=True, record=True)
        torch.cuda.synchronize()
        assert np.array_equal(ch.obs_block.cpu().numpy(), eager_block), label
        for e, g in zip(steps, graphed):
            assert np.array_equal(e["cstar"], g["cstar"], equal_nan=True), label
        log(f"[observe] {label}: graph replays leave the same block and c*")
    return got


SMALL = dict(R=20, gamma=5, V=3000, r=64, d=96, seed=31, W_std=0.3, b=0.5)


@pytest.mark.parametrize("vmode,dtype", [("cap_accept", "bf16"), ("compact", "bf16"),
                                         ("static", "f32"), ("compact", "f32")])
def test_small_observed_decode(dv, vmode, dtype):
    spec = synth.small_spec(f"obs_{dtype}", dtype=dtype, **SMALL)
    got = run_observed(dv, spec, vmode, 2, 5)
    if vmode == "static":
        assert got["accepted"] == got["ceiling"]


def test_ragged_rank_and_vocab(dv):
    spec = synth.small_spec("obs_ragged", R=33, gamma=4, V=2950, r=100, d=40, dtype="bf16", seed=8,
                            W_std=0.3, b=0.5)
    run_observed(dv, spec, "compact", 1, 3)


@pytest.mark.parametrize("name,vmode", [("qwen3", "cap_accept"), ("mixed", "compact")])
def test_full_size_observed(dv, name, vmode):
    run_observed(dv, synth.CONFIGS[name], vmode, 2, 3, graph_check=False)
