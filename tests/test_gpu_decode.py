"""GPU parity of the multi-step decode loop (Chain.decode over dspark_advance),
through the C ABI.

Every step is checked teacher-forced against the oracle on the GPU's own state
at the start of that step (its x_0, Philox step and budget array), with the
same tolerance rules as the single-step chain; the loop's own bookkeeping is
bit-exact: the Philox step counts up, x_0 of step t+1 is the token step t
committed last, and the budget array of step t is the GPU's survival array of
step t - lag. A graph-replayed loop must reproduce the eager loop bit for bit
at every replay (with host copies and synchronisation between replays).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (log, upload, PackedView, check_draft, check_confidence,
                            check_schedule, check_pack, check_verify, sample_requests, factors64)

pytestmark = pytest.mark.gpu

MODES = {"static": 0, "compact": 1, "cap_accept": 2}


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()          # raises if the HIP library is missing
    return dv


def check_loop(steps, inp, spec, vmode, lag, seed, step0, B, reqs, label, smode=oracle.SCHED_ARGMAX):
    flips = 0
    R = spec.R
    factors64(inp)                 # widened once; every step's view shares them
    for t, res in enumerate(steps):
        lab = f"{label}/t{t}"
        step = int(res["step"][0])
        assert step == step0 + t, lab
        inp_t = {**inp, "anchor": res["anchor"]}
        if t == 0:
            assert res["anchor"].tolist() == inp["anchor"].tolist(), lab
        else:
            prev = steps[t - 1]
            last = prev["out_tokens"][np.arange(R), prev["accept_len"]]
            assert res["anchor"].tolist() == last.tolist(), lab
        if lag > 0 and t >= lag:
            assert np.array_equal(res["surv_budget"], steps[t - lag]["surv"]), lab
            assert res["sched_mode"] == smode, lab
        else:
            assert res["surv_budget"] is None, lab
            want = oracle.SCHED_GREEDY if (lag > 0 and smode == oracle.SCHED_ARGMAX) else smode
            assert res["sched_mode"] == want, lab
        flips += check_draft(res, inp_t, seed, step, reqs, lab)
        check_confidence(res, inp_t, reqs, lab)
        sps = [int(x) for x in res["sps"]]
        ref_s = check_schedule(res, sps, B, res["sched_mode"], 0, lab, res["surv_budget"])
        full = vmode in ("static", "cap_accept")
        check_pack(res, inp_t, None if full else ref_s["win_len"], spec.tiers, R * (spec.gamma + 1), lab)
        rows = PackedView(inp["target"], res["cu_seqlens"])
        flips += check_verify(res, inp_t, rows, MODES[vmode], res["win_len"], seed, step, reqs, lab)
    return flips


def run_loop(dv, spec, vmode, lag, n_steps, *, seed=7, step0=100, sample=None, graph_check=True):
    import torch
    label = f"{spec.name}/{vmode}/lag{lag}"
    log(f"[decode] {label}: R={spec.R} gamma={spec.gamma} V={spec.V} r={spec.r} "
        f"dtype={spec.dtype} steps={n_steps}")
    inp = synth.generate(spec)
    dev, sps = upload(inp, spec)
    B = spec.budgets[0]
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=B, verify_mode=MODES[vmode],
                  seed=seed, step=step0)
    eager = ch.decode(n_steps, lag=lag, record=True)
    torch.cuda.synchronize()
    for e in eager:
        e["sps"] = sps
    reqs = np.arange(spec.R) if sample is None else sample_requests(spec.R, sample)
    flips = check_loop(eager, inp, spec, vmode, lag, seed, step0, B, reqs, label)
    Ks = [int(e["K"][0]) for e in eager]
    log(f"[decode] {label}: eager ok, K per step {Ks}, "
        f"mean A {np.mean([e['accept_len'].mean() for e in eager]):.2f}, excused flips {flips}")
    if graph_check:
        ch.reset()
        graphed = ch.decode(n_steps, lag=lag, graph=True, record=True)
        torch.cuda.synchronize()
        assert ch._graph is not None
        for t, (e, g) in enumerate(zip(eager, graphed)):
            for k, v in e.items():
                if k == "sps":
                    continue
                if v is None or isinstance(v, int):
                    assert g[k] == v, (label, "graph", t, k)
                else:
                    assert np.array_equal(g[k], v), (label, "graph", t, k)
        log(f"[decode] {label}: graph replays match the eager loop")
    return eager


SMALL = dict(R=20, gamma=5, V=3000, r=64, d=96, seed=21, W_std=0.3, b=0.5)


@pytest.mark.parametrize("vmode,lag,dtype", [("compact", 2, "bf16"), ("compact", 1, "f32"),
                                             ("static", 2, "bf16"), ("cap_accept", 0, "bf16")])
def test_small_decode(dv, vmode, lag, dtype):
    spec = synth.small_spec(f"decode_{dtype}", dtype=dtype, **SMALL)
    steps = run_loop(dv, spec, vmode, lag, 6)
    if lag:
        # the stale budget changed K in at least one step of the compact loops
        assert len({int(s["K"][0]) for s in steps}) >= 2 or vmode != "compact"


def test_decode_survives_a_lag_change(dv):
    # lag 2 then lag 0 on one chain: new history, new graph; state carries over
    import torch
    spec = synth.small_spec("decode_switch", dtype="bf16", **SMALL)
    inp = synth.generate(spec)
    dev, sps = upload(inp, spec)
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=spec.budgets[0],
                  verify_mode=MODES["compact"], seed=3, step=0)
    a = ch.decode(3, lag=2, graph=True, record=True)
    b = ch.decode(3, lag=0, graph=True, record=True)
    torch.cuda.synchronize()
    assert [int(s["step"][0]) for s in a + b] == list(range(6))
    last = a[-1]["out_tokens"][np.arange(spec.R), a[-1]["accept_len"]]
    assert b[0]["anchor"].tolist() == last.tolist()
    assert all(s["surv_budget"] is None for s in b)


@pytest.mark.parametrize("name,vmode", [("qwen3", "compact"), ("mixed", "compact")])
def test_full_size_decode(dv, name, vmode):
    run_loop(dv, synth.CONFIGS[name], vmode, 2, 4)
