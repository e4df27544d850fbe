"""Pins of the oracle's rejection-sampling verification.

* closed form: the probability that slot 1 is accepted equals
  1 - 1/2 ||p_d - p_t||_1 (the analytic acceptance rate the DSpark digest uses
  as the confidence head's target, "Verification scheduling (system side)"),
  checked empirically within a binomial band;
* lossless: committed tokens are distributed as the target (chi-square at a
  16-entry vocabulary), at slot 1 and at slot 2 given slot 1 accepted, in static
  mode, compact mode with windows fixed in advance, and compact mode with
  greedy (non-anticipating) windows;
* special cases: p_d = p_t accepts everything; disjoint supports reject slot 1
  and resample from the target; an empty window is plain target sampling;
* cap-accept commits exactly what compact commits (SGLang DSpark blog, "Verify
  modes").
"""
import numpy as np
import pytest
from scipy import special, stats

import synth
import oracle
from oracle.markov import markov_draft
from oracle.pack import pack_ragged
from oracle.verify import verify, VERIFY_STATIC, VERIFY_COMPACT, VERIFY_CAP_ACCEPT


def _chisq(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.concatenate([counts[keep], [counts[~keep].sum()]])
    e = np.concatenate([exp[keep], [exp[~keep].sum()]])
    if e[-1] == 0:
        obs, e = obs[:-1], e[:-1]
    return stats.chisquare(obs, e).pvalue


def _shared_block(N, V, gamma, seed, draft_noise=0.8, r=4, Wstd=0.3):
    """N requests sharing one block of target and draft logits (their Philox
    streams differ by request id)."""
    rng = np.random.default_rng(seed)
    T = rng.normal(0, 1.5, (gamma + 1, V))
    U1 = T[:gamma] + rng.normal(0, draft_noise, (gamma, V))
    W1 = rng.normal(0, Wstd, (V, r))
    W2 = rng.normal(0, Wstd, (r, V))
    return {
        "target": np.broadcast_to(T, (N, gamma + 1, V)),
        "U": np.broadcast_to(U1, (N, gamma, V)),
        "W1": W1, "W2": W2, "anchor": np.full(N, 2), "req_ids": np.arange(N),
        "T": T, "U1": U1,
    }


def _packed(target, cu):
    N = len(cu) - 1
    rows = np.concatenate([target[i, :cu[i + 1] - cu[i]] for i in range(N)], axis=0)
    return rows


def _run(blk, win, mode, seed=1, step=0):
    N, gamma, V = blk["U"].shape
    d = markov_draft(blk["U"], blk["W1"], blk["W2"], blk["anchor"], seed, step, blk["req_ids"])
    pk = pack_ragged(blk["anchor"], d["tokens"], None if mode != VERIFY_COMPACT else win,
                     [N * (gamma + 1)], N * (gamma + 1))
    rows = _packed(blk["target"], pk["cu_seqlens"])
    v = verify(rows, pk["cu_seqlens"], blk["anchor"], d["tokens"], d["p_draft"], blk["U"],
               blk["W1"], blk["W2"], win, mode, seed, step, blk["req_ids"])
    return d, v


@pytest.mark.slow
def test_acceptance_rate_closed_form():
    N, V, gamma = 12000, 16, 1
    blk = _shared_block(N, V, gamma, seed=3, draft_noise=1.0)
    d, v = _run(blk, None, VERIFY_STATIC)
    pt = special.softmax(blk["T"][0])
    pd = special.softmax(blk["U1"][0] + blk["W1"][2] @ blk["W2"])
    closed = 1.0 - 0.5 * np.abs(pd - pt).sum()
    rate = (v["accept_len"] >= 1).mean()
    sigma = np.sqrt(closed * (1 - closed) / N)
    assert abs(rate - closed) < 4 * sigma, (rate, closed)


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["static", "compact_fixed", "compact_greedy"])
def test_lossless_chi_square(mode):
    N, V, gamma = 10000, 16, 3
    blk = _shared_block(N, V, gamma, seed=5)
    pt1 = special.softmax(blk["T"][0])
    if mode == "static":
        d, v = _run(blk, None, VERIFY_STATIC)
    elif mode == "compact_fixed":
        win = np.random.default_rng(8).integers(0, gamma + 1, N)
        d, v = _run(blk, win, VERIFY_COMPACT)
    else:
        # windows from the greedy scheduler over confidences that depend on
        # the drafted tokens (a synthetic head)
        d = markov_draft(blk["U"], blk["W1"], blk["W2"], blk["anchor"], 1, 0, blk["req_ids"])
        rng = np.random.default_rng(9)
        h = rng.normal(0, 1, (N, gamma, 4)).astype(np.float32)
        w = rng.normal(0, 0.8, 4 + blk["W1"].shape[1]).astype(np.float32)
        c = oracle.confidence(h, blk["W1"].astype(np.float32), blk["anchor"], d["tokens"], w, 1.0)
        M_max = N * (gamma + 1)
        sps = [max(2_000_000 - 40 * m, 1) for m in range(M_max + 1)]
        sch = oracle.schedule_topb(c["surv"].astype(np.float32), sps, N * gamma, oracle.SCHED_GREEDY)
        win = np.array(sch["win_len"])
        assert 0 < win.mean() < gamma
        pk = pack_ragged(blk["anchor"], d["tokens"], win, [M_max], M_max)
        rows = _packed(blk["target"], pk["cu_seqlens"])
        v = verify(rows, pk["cu_seqlens"], blk["anchor"], d["tokens"], d["p_draft"], blk["U"],
                   blk["W1"], blk["W2"], win, VERIFY_COMPACT, 1, 0, blk["req_ids"])
    first = v["out_tokens"][:, 0]
    assert _chisq(np.bincount(first, minlength=V).astype(float), pt1) > 1e-4
    # slot 2 given slot 1 committed as a draft (n_out >= 2): target row 1
    sel = v["n_out"] >= 2
    second = v["out_tokens"][sel, 1]
    pt2 = special.softmax(blk["T"][1])
    assert sel.sum() > 2000
    assert _chisq(np.bincount(second, minlength=V).astype(float), pt2) > 1e-4


def test_equal_distributions_accept_everything():
    N, V, gamma = 200, 30, 4
    rng = np.random.default_rng(1)
    T = rng.normal(0, 2, (gamma + 1, V))
    blk = {"target": np.broadcast_to(T, (N, gamma + 1, V)),
           "U": np.broadcast_to(T[:gamma], (N, gamma, V)),
           "W1": np.zeros((V, 3)), "W2": np.zeros((3, V)),
           "anchor": np.zeros(N, dtype=int), "req_ids": np.arange(N)}
    d, v = _run(blk, None, VERIFY_STATIC)
    assert np.all(v["accept_len"] == gamma)
    assert np.all(v["out_tokens"][:, :gamma] == d["tokens"])


@pytest.mark.slow
def test_disjoint_supports_reject_and_resample_target():
    N, V, gamma = 8000, 16, 2
    T = np.zeros((gamma + 1, V))
    T[:, :V // 2] = -1e4                      # target lives on the upper half
    T[:, V // 2:] = np.random.default_rng(2).normal(0, 1, (gamma + 1, V // 2))
    U1 = np.full((gamma, V), -1e4)
    U1[:, :V // 2] = 0.0                      # draft lives on the lower half
    blk = {"target": np.broadcast_to(T, (N, gamma + 1, V)),
           "U": np.broadcast_to(U1, (N, gamma, V)),
           "W1": np.zeros((V, 2)), "W2": np.zeros((2, V)),
           "anchor": np.zeros(N, dtype=int), "req_ids": np.arange(N)}
    d, v = _run(blk, None, VERIFY_STATIC)
    assert np.all(v["accept_len"] == 0)
    first = v["out_tokens"][:, 0]
    assert np.all(first >= V // 2)
    assert _chisq(np.bincount(first, minlength=V).astype(float), special.softmax(T[0])) > 1e-4


@pytest.mark.slow
def test_empty_window_is_plain_target_sampling():
    N, V, gamma = 8000, 16, 3
    blk = _shared_block(N, V, gamma, seed=6)
    d, v = _run(blk, np.zeros(N, dtype=int), VERIFY_COMPACT)
    assert np.all(v["accept_len"] == 0) and np.all(v["n_out"] == 1)
    assert all(t["kind"] == "bonus" and t["slot"] == 1 for t in v["trace"].values())
    first = v["out_tokens"][:, 0]
    assert _chisq(np.bincount(first, minlength=V).astype(float), special.softmax(blk["T"][0])) > 1e-4


def test_cap_accept_commits_what_compact_commits():
    sp = synth.small_spec(R=24, gamma=6, V=500, r=16, d=16, dtype="bf16", seed=12)
    inp = synth.generate(sp)
    common = dict(tiers=sp.tiers, staircase=sp.staircase, B_cap=sp.R * sp.gamma)
    comp = oracle.chain(inp, verify_mode=VERIFY_COMPACT, **common)
    cap = oracle.chain(inp, verify_mode=VERIFY_CAP_ACCEPT, **common)
    stat = oracle.chain(inp, verify_mode=VERIFY_STATIC, **common)
    assert np.array_equal(comp["verify"]["out_tokens"], cap["verify"]["out_tokens"])
    assert np.array_equal(comp["verify"]["accept_len"], cap["verify"]["accept_len"])
    # the cap-accept ceiling is what a full-block verify accepts
    assert np.array_equal(cap["verify"]["ceiling"], stat["verify"]["accept_len"])
    win = np.array(comp["sched"]["win_len"])
    assert np.array_equal(cap["verify"]["accept_len"], np.minimum(stat["verify"]["accept_len"], win))
    assert 0 < win.sum() < sp.R * sp.gamma
