"""Pins of the oracle's multi-step decode loop and of the causal-budget claim
behind it (DSpark digest, "Verification scheduling (system side)" and "Infra
(online production @ DeepSeek-V4)").

* Exact enumeration (no sampling): a request's first committed token is
  distributed exactly as the target when its window is decided without looking
  at the token being verified -- a budget from older confidences (any array
  fixed before the step's draws), the greedy scheduler with its early stop, or
  a fixed K -- and not in general when ARGMAX sizes the budget from the step's
  own survivals, whose later slots depend on the slot-1 draft. The constructed
  case has a closed-form answer (total variation 0.15 from the target).
* Special case: lag 0 is the single-step chain repeated with x_0 moved to the
  last committed token and the Philox step counting up.
* Lag semantics: a step at t >= lag takes its budget from step t - lag; the
  earlier steps run greedy; the selection is always by the step's own
  survivals.
* Monte Carlo: every step of a lag-2 ARGMAX loop commits a first token
  distributed as the target row of slot 1 (chi-square over many seeds).
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth
from oracle.schedule import schedule_topb, SCHED_ARGMAX, SCHED_GREEDY, SCHED_FIXED


# ---------------------------------------------------------------------------
# exact enumeration of the first committed token
# ---------------------------------------------------------------------------

# two requests, gamma = 2, V = 3. Request 0: c_1 = 0.5 and c_2 depends on the
# slot-1 draft x (0.9 for x = 0, 0.1 otherwise). Request 1 ranks last.
PD0 = np.array([0.5, 0.3, 0.2])
PT0 = np.array([0.2, 0.3, 0.5])
PD1 = np.array([0.6, 0.2, 0.2])
PT1 = np.array([0.1, 0.6, 0.3])
C2_0 = np.array([0.9, 0.1, 0.1])
C2_1 = np.array([0.5, 0.5, 0.5])
# steps per second (x1000) at M = 0..6: with R = 2, K = 0 gives 2000 (x 2^20),
# K = 1 gives 1975, K = 2 gives 2065 when request 0's second survival is 0.45
# and 1785 when it is 0.05; K = 3, 4 never win
SPS = [2000, 1500, 1000, 790, 700, 600, 500]


def _survivals(x0, x1, c1_1):
    a = np.array([[0.5, 0.5 * C2_0[x0]], [c1_1, c1_1 * C2_1[x1]]], dtype=np.float32)
    return a


def _first_token_dist(req, mode, budget=None, K_fixed=0, c1_1=0.01):
    """Exact distribution of request `req`'s first committed token, summed over
    both requests' slot-1 drafts (the only draws the survivals depend on)."""
    pd, pt = (PD0, PT0) if req == 0 else (PD1, PT1)
    res = np.maximum(pt - pd, 0.0)
    res /= res.sum()
    out = np.zeros(3)
    for x0 in range(3):
        for x1 in range(3):
            prob = PD0[x0] * PD1[x1]
            s = schedule_topb(_survivals(x0, x1, c1_1), SPS, 4, mode, K_fixed, budget)
            x = (x0, x1)[req]
            if s["win_len"][req] >= 1:
                acc = min(1.0, pt[x] / pd[x])
                dist = (1.0 - acc) * res
                dist[x] += acc
            else:
                dist = pt
            out += prob * dist
    return out


def test_same_step_argmax_budget_is_anticipating():
    d = _first_token_dist(0, SCHED_ARGMAX)
    # K = 2 exactly when x0 = 0 (probability 0.5), else K = 0:
    # 0.5 (0.4 e_0 + 0.6 e_2) + 0.5 p_t
    np.testing.assert_allclose(d, [0.3, 0.15, 0.55], atol=1e-12)
    assert 0.5 * np.abs(d - PT0).sum() == pytest.approx(0.15, abs=1e-12)


@pytest.mark.parametrize("c1_1", [0.01, 0.3])
def test_causal_windows_are_lossless(c1_1):
    stale = _survivals(0, 0, c1_1)          # confidences fixed before the step's draws
    cases = [(SCHED_ARGMAX, stale, 0), (SCHED_GREEDY, None, 0), (SCHED_FIXED, None, 1),
             (SCHED_FIXED, None, 2)]
    for mode, budget, K in cases:
        for req, pt in ((0, PT0), (1, PT1)):
            d = _first_token_dist(req, mode, budget, K, c1_1)
            np.testing.assert_allclose(d, pt, atol=1e-12, err_msg=str((mode, K, req, c1_1)))


def test_competing_requests_share_the_stale_budget():
    # with request 1 at c_1 = 0.3, a K = 2 budget goes to request 0's second
    # slot or to request 1's first slot depending on request 0's draft
    stale = _survivals(0, 0, 0.3)
    wins = {schedule_topb(_survivals(x0, 0, 0.3), SPS, 4, SCHED_ARGMAX, 0, stale)["win_len"][1]
            for x0 in range(3)}
    assert wins == {0, 1}


# ---------------------------------------------------------------------------
# the loop itself
# ---------------------------------------------------------------------------

def _inputs(R=6, gamma=4, V=200, seed=3, **kw):
    spec = synth.small_spec("decode", R=R, gamma=gamma, V=V, r=16, d=32, dtype="f32", seed=seed,
                            **kw)
    return spec, synth.generate(spec)


# Markov factors and head bias that make the survivals depend strongly on the
# drafted tokens, and a smooth cost curve, so that K and the windows vary from
# step to step
VARIED = dict(cost=("linear_sps", 2_000_000, 120_000), staircase=False, W_std=1.0, b=0.5)


def _loop(inp, spec, steps, lag, vmode, smode=SCHED_ARGMAX, seed=5, step0=11):
    return oracle.decode(inp, steps=steps, lag=lag, tiers=spec.tiers, staircase=spec.staircase,
                         B_cap=spec.budgets[0], verify_mode=vmode, sched_mode=smode, seed=seed,
                         step0=step0)


@pytest.mark.parametrize("vmode", [oracle.VERIFY_STATIC, oracle.VERIFY_COMPACT])
def test_lag0_is_the_single_step_chain_repeated(vmode):
    spec, inp = _inputs()
    steps = _loop(inp, spec, 4, 0, vmode)
    anchor = inp["anchor"].astype(np.int32)
    for t, res in enumerate(steps):
        ref = oracle.chain({**inp, "anchor": anchor}, tiers=spec.tiers, staircase=spec.staircase,
                           B_cap=spec.budgets[0], verify_mode=vmode, seed=5, step=11 + t)
        assert res["anchor"].tolist() == anchor.tolist()
        assert res["draft"]["tokens"].tolist() == ref["draft"]["tokens"].tolist()
        assert res["sched"]["win_len"] == ref["sched"]["win_len"]
        v = ref["verify"]
        assert res["verify"]["out_tokens"].tolist() == v["out_tokens"].tolist()
        # the next x_0 is the last committed token
        anchor = np.array([v["out_tokens"][r, v["n_out"][r] - 1] for r in range(spec.R)],
                          dtype=np.int32)
    # the anchors moved: later steps drafted from committed tokens
    assert steps[-1]["anchor"].tolist() != inp["anchor"].tolist()


@pytest.mark.parametrize("lag", [1, 2])
def test_budget_comes_from_lag_steps_back(lag):
    spec, inp = _inputs(R=3, gamma=3, V=50, **VARIED)
    steps = _loop(inp, spec, 8, lag, oracle.VERIFY_COMPACT)
    assert len({res["sched"]["K"] for res in steps}) >= 2
    for t, res in enumerate(steps):
        surv = res["conf"]["surv"].astype(np.float32)
        if t < lag:
            assert res["surv_budget"] is None and res["sched_mode"] == SCHED_GREEDY
            ref = schedule_topb(surv, res["sps_milli"], spec.budgets[0], SCHED_GREEDY)
        else:
            old = steps[t - lag]["conf"]["surv"].astype(np.float32)
            assert np.array_equal(res["surv_budget"], old) and res["sched_mode"] == SCHED_ARGMAX
            ref = schedule_topb(surv, res["sps_milli"], spec.budgets[0], SCHED_ARGMAX, 0, old)
            # K is the budget array's argmax, the selection the current top-K
            K_old = schedule_topb(old, res["sps_milli"], spec.budgets[0], SCHED_ARGMAX)["K"]
            assert ref["K"] == K_old
        assert res["sched"]["win_len"] == ref["win_len"] and res["sched"]["K"] == ref["K"]


@pytest.mark.slow
def test_stale_budget_loop_commits_target_distributed_tokens():
    # V = 6 so that a chi-square over every id has power; the first committed
    # token of every request at every step must follow softmax(target[r, 0])
    spec, inp = _inputs(R=3, gamma=3, V=6, seed=9, **VARIED)
    counts = np.zeros((spec.R, spec.V))
    Ks, wins = set(), set()
    for sd in range(60):
        for res in _loop(inp, spec, 12, 2, oracle.VERIFY_COMPACT, seed=1000 + sd, step0=0):
            first = res["verify"]["out_tokens"][:, 0]
            counts[np.arange(spec.R), first] += 1
            Ks.add(res["sched"]["K"])
            wins.update(res["sched"]["win_len"])
    assert len(Ks) >= 2 and {0, 1, 2, 3} <= wins       # the windows really vary
    for r in range(spec.R):
        pt = special.softmax(synth_target_row(inp, r))
        p = stats.chisquare(counts[r], pt * counts[r].sum()).pvalue
        assert p > 1e-4, (r, counts[r], pt)


def synth_target_row(inp, r):
    return oracle.widen(inp["target"][r, 0])
