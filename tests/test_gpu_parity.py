"""GPU parity of every stage against the oracle (teacher-forced stage by
stage on the GPU's own chain outputs), through the C ABI.

Small workloads span several 16-request blocks, several 64-entry vocabulary
tiles and ragged tails in both; the five named workloads run at full size in
the configuration bench.py times, with the oracle checking every request of
every stage.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import log, upload, run_and_check, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()          # raises if the HIP library is missing
    return dv


# ---------------------------------------------------------------------------
# diagnostic: the matrix-core logits tile against the oracle's logits
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,V,r,R", [("f32", 1000, 32, 20), ("bf16", 3000, 64, 20),
                                          ("bf16", 2950, 256, 33), ("bf16", 517, 100, 5),
                                          ("f32", 640, 128, 16)])
def test_markov_logits_tile(dv, dtype, V, r, R):
    import torch
    log(f"[logits] dtype={dtype} V={V} r={r} R={R}")
    sp = synth.small_spec(R=R, gamma=2, V=V, r=r, d=8, dtype=dtype, W_std=0.3)
    inp = synth.generate(sp)
    dev, _ = upload(inp, sp)
    W2p = dv.prepack_w2(dev["W2"])
    x_prev = to_dev(inp["anchor"])
    z = dv.markov_logits(dev["U"], sp.gamma * V, dev["W1"], W2p, x_prev, R=R, V=V, r=r)
    torch.cuda.synchronize()
    ref = oracle.markov_logits(inp["U"][:, 0], inp["W1"], inp["W2"], inp["anchor"])
    np.testing.assert_allclose(z.cpu().numpy(), ref, rtol=0, atol=2e-5)


# ---------------------------------------------------------------------------
# small workloads: every stage, every mode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("vmode", ["static", "compact", "cap_accept"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_chain(dv, vmode, dtype):
    sp = synth.small_spec(R=20, gamma=5, V=3000, r=64, d=96, dtype=dtype)
    run_and_check(dv, sp, vmode)


@pytest.mark.parametrize("dtype,R,r", [("bf16", 300, 32), ("f32", 150, 100)])
def test_request_groups(dv, dtype, R, r):
    # more requests than one GEMM launch holds (256 for bfloat16, 128 for
    # float32): the draft and residual passes run one launch per group
    sp = synth.small_spec(R=R, gamma=2, V=1200, r=r, d=24, dtype=dtype, seed=13)
    run_and_check(dv, sp, "compact")


@pytest.mark.parametrize("smode", [oracle.SCHED_GREEDY, oracle.SCHED_FIXED])
def test_small_chain_sched_modes(dv, smode):
    sp = synth.small_spec(R=37, gamma=4, V=1777, r=48, d=40, dtype="bf16", seed=5)
    run_and_check(dv, sp, "compact", smode=smode, K_fixed=50)


def test_small_chain_ragged_rank_and_vocab(dv):
    # rank not a multiple of 8 (scalar staging), vocabulary not a multiple of 8
    sp = synth.small_spec(R=18, gamma=3, V=997, r=45, d=33, dtype="bf16", seed=9)
    run_and_check(dv, sp, "compact")


def test_cap_accept_commits_match_compact(dv):
    sp = synth.small_spec(R=40, gamma=6, V=2048, r=32, d=64, dtype="bf16", seed=21)
    inp = synth.generate(sp)
    comp, _ = run_and_check(dv, sp, "compact", inp=inp)
    cap, _ = run_and_check(dv, sp, "cap_accept", inp=inp)
    assert np.array_equal(comp["tokens"], cap["tokens"])
    assert np.array_equal(comp["win_len"], cap["win_len"])
    assert np.array_equal(comp["accept_len"], cap["accept_len"])
    assert np.array_equal(comp["out_tokens"], cap["out_tokens"])
    assert np.all(cap["ceiling_len"] >= cap["accept_len"])


def test_determinism(dv):
    import torch
    sp = synth.small_spec(R=24, gamma=5, V=3000, r=64, d=32, dtype="bf16", seed=3)
    inp = synth.generate(sp)
    dev, _ = upload(inp, sp)
    outs = []
    for _ in range(2):
        ch = dv.Chain(dev, b=float(inp["b"]), tiers=sp.tiers, B_cap=sp.R * sp.gamma, verify_mode=1)
        ch.run()
        torch.cuda.synchronize()
        outs.append(ch.results())
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_step_and_seed_change_draws(dv):
    sp = synth.small_spec(R=16, gamma=4, V=1000, r=32, d=16, dtype="bf16", seed=4)
    inp = synth.generate(sp)
    a, _ = run_and_check(dv, sp, "static", inp=inp, seed=0, step=0)
    b, _ = run_and_check(dv, sp, "static", inp=inp, seed=0, step=1)
    c, _ = run_and_check(dv, sp, "static", inp=inp, seed=7, step=0)
    assert not np.array_equal(a["tokens"], b["tokens"])
    assert not np.array_equal(a["tokens"], c["tokens"])


def _random_chain_shapes(n, seed):
    """n seeded (R, gamma, V, r, d, dtype, verify mode, scheduler mode) draws:
    request counts on and around the engine's 16-request blocks and its
    one-, two- and multi-group shapes (1 .. 300), vocabularies from one tile to
    several row-pass chunks with ragged tails (64 .. 33000), ranks from 16 to
    256 (some not a multiple of the vector width), hidden sizes up to 520."""
    rng = np.random.default_rng(seed)
    modes = ["static", "compact", "cap_accept"]
    out = []
    for case in range(n):
        while True:
            R = int(rng.choice([1, 3, 17, 64, 129, 150, 200, 256, 300]))
            gamma = int(rng.integers(1, 9))
            if R * (gamma + 1) <= 4096:
                break
        V = int(rng.choice([64, 700, 1500, 2047, 3000, 16400, 33000]))
        r = int(rng.choice([16, 32, 64, 100, 256]))
        d = int(rng.choice([8, 40, 96, 520]))
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        if dtype == "f32" and r > 128:
            r = 100
        out.append(dict(R=R, gamma=gamma, V=V, r=r, d=d, dtype=dtype, vmode=modes[case % 3],
                        smode=int(rng.integers(0, 3)), K_fixed=int(rng.integers(0, R * gamma + 1)),
                        sseed=int(rng.integers(1, 10**6)), seed=int(rng.integers(0, 1000)),
                        step=int(rng.integers(0, 1000))))
    return out


@pytest.mark.parametrize("case", _random_chain_shapes(10, 11), ids=lambda c: (
    f"R{c['R']}-g{c['gamma']}-V{c['V']}-r{c['r']}-{c['dtype']}-{c['vmode']}-s{c['smode']}"))
def test_random_small_chains(dv, case):
    """Seeded random shapes, every request of every stage against the oracle."""
    sp = synth.small_spec(f"rand{case['sseed']}", R=case["R"], gamma=case["gamma"], V=case["V"],
                          r=case["r"], d=case["d"], dtype=case["dtype"], seed=case["sseed"])
    run_and_check(dv, sp, case["vmode"], smode=case["smode"], K_fixed=case["K_fixed"],
                  seed=case["seed"], step=case["step"])


# ---------------------------------------------------------------------------
# edge cases: degenerate sizes, an empty budget, the row limit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [dict(R=1, gamma=1, V=1, r=1, d=4, dtype="f32"),
                                   dict(R=1, gamma=16, V=65, r=8, d=8, dtype="bf16"),
                                   dict(R=3, gamma=2, V=64, r=32, d=16, dtype="bf16")],
                         ids=["V1-gamma1-r1", "gamma16-V65", "one-tile"])
def test_degenerate_sizes(dv, shape):
    # a one-entry vocabulary (every draft is token 0 with probability 1, every
    # accept test passes), the longest block, exactly one vocabulary tile; each
    # in every verify mode, with an empty budget and with the full one
    sp = synth.small_spec("edge", seed=3, **shape)
    inp = synth.generate(sp)
    for vmode in ("static", "compact", "cap_accept"):
        for B in (0, sp.R * sp.gamma):
            res, _ = run_and_check(dv, sp, vmode, B_cap=B, inp=inp)
            if B == 0:
                assert int(res["K"][0]) == 0 and np.all(res["win_len"] == 0)
            if shape["V"] == 1:
                assert np.all(res["tokens"] == 0) and np.allclose(res["p_draft"], 1.0)


def test_row_limit(dv):
    # R (gamma + 1) = 4096 packed rows, the documented maximum: 3840 scheduler
    # keys, the largest pack; a cheap per-token cost so that K is large
    sp = synth.small_spec("rowlimit", R=256, gamma=15, V=700, r=32, d=16, dtype="bf16", seed=6,
                          cost=("stair_T", 2e-3, 1e-8, 0.005))
    inp = synth.generate(sp)
    res, _ = run_and_check(dv, sp, "static", inp=inp)
    assert int(res["totals"][0]) == 4096
    res, _ = run_and_check(dv, sp, "compact", inp=inp, check_draft_conf=False)
    assert int(res["K"][0]) > 1000


# ---------------------------------------------------------------------------
# the five named workloads at full size
# ---------------------------------------------------------------------------

def test_tiny_all_modes(dv):
    sp = synth.CONFIGS["tiny"]
    inp = synth.generate(sp)
    for vmode in ("static", "compact", "cap_accept"):
        for smode in (oracle.SCHED_ARGMAX, oracle.SCHED_GREEDY, oracle.SCHED_FIXED):
            if vmode != "compact" and smode != oracle.SCHED_ARGMAX:
                continue
            run_and_check(dv, sp, vmode, smode=smode, K_fixed=6, inp=inp)


@pytest.mark.parametrize("vmode", ["static", "compact"])
def test_qwen3(dv, vmode):
    run_and_check(dv, synth.CONFIGS["qwen3"], vmode)


def test_dsv4_compact(dv):
    run_and_check(dv, synth.CONFIGS["dsv4"], "compact")


@pytest.mark.parametrize("vmode", ["cap_accept", "compact"])
def test_mixed(dv, vmode):
    run_and_check(dv, synth.CONFIGS["mixed"], vmode)


def test_long_budget_sweep(dv):
    sp = synth.CONFIGS["long"]
    inp = synth.generate(sp)
    # the draft and confidence do not depend on the budget: checked once
    for i, B in enumerate(sp.budgets):
        run_and_check(dv, sp, "compact", B_cap=B, inp=inp, check_draft_conf=i == 0)
