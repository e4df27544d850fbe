"""GPU edge cases and distribution checks, through the C ABI.

* Many requests over a one- or two-tile vocabulary: the draft GEMM then runs
  on one or two workgroups, which must still draw every request's uniform.
  Every request is compared with the oracle.
* More than 128 requests at rank 256 (bf16): the GEMM engine's shape with
  eight rank chunks and two 16-request blocks per wave, at a small size.
* Disjoint draft and target supports (DSpark digest, "Architecture
  (drafter)": rejection sampling is exact): every slot-1 draft has p_t = 0 and
  is rejected, and the correction is drawn from p_t, the residual.
* No residual mass left after a reject (rounding only in exact arithmetic):
  the correction falls back to p_t, in the verify kernels and in the oracle.
* NaN and out-of-range survivals in the scheduler (read as 0, clamped to
  [0, 1]) against the oracle's integer scheduler.
* Losslessness on the GPU: committed slot-1 tokens of 10240 requests that
  share one set of logits (V = 48) follow the target's slot-1 distribution
  (chi-square), and the slot-1 drafts follow the draft distribution.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (log, upload, to_dev, run_and_check, check_verify, PackedView,
                            factors64, MODES)

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
# engine shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,R,V", [("bf16", 256, 64), ("bf16", 256, 128), ("bf16", 300, 64),
                                       ("f32", 150, 64), ("f32", 128, 100)])
def test_many_requests_small_vocab(dv, dtype, R, V):
    # 64 R > 64 ceil(V / 64): fewer GEMM workgroups than 64-request groups
    sp = synth.small_spec(f"smallvocab_{dtype}", R=R, gamma=3, V=V, r=32, d=16, dtype=dtype,
                          seed=17, W_std=0.3)
    for vmode in ("static", "compact"):
        run_and_check(dv, sp, vmode)


@pytest.mark.parametrize("R,V", [(200, 1500), (256, 2047)])
def test_wide_rank_two_blocks_per_wave(dv, R, V):
    # bf16, rank 256 (eight 32-rank chunks), more than eight 16-request blocks
    sp = synth.small_spec("rank256", R=R, gamma=3, V=V, r=256, d=32, dtype="bf16", seed=19,
                          W_std=0.05)
    run_and_check(dv, sp, "cap_accept")


# ---------------------------------------------------------------------------
# verify special cases
# ---------------------------------------------------------------------------

NEG = -30000.0   # exp(NEG - max) is 0 in float32 and float64


def _rows(inp, key):
    return synth.bf16_bits_to_f32(inp[key]) if inp[key].dtype == np.uint16 else inp[key]


def test_disjoint_supports(dv):
    sp = synth.small_spec("disjoint", R=40, gamma=3, V=1000, r=32, d=16, dtype="bf16", seed=23,
                          W_std=0.0)
    inp = synth.generate(sp)
    half = sp.V // 2
    tgt = _rows(inp, "target").copy()
    U = _rows(inp, "U").copy()
    tgt[..., half:] = NEG         # the target lives on [0, V/2)
    U[..., :half] = NEG           # the draft on [V/2, V)
    inp["target"] = synth.to_bf16_bits(tgt)
    inp["U"] = synth.to_bf16_bits(U)
    for vmode in ("static", "compact", "cap_accept"):
        res, _ = run_and_check(dv, sp, vmode, inp=inp)
        assert np.all(res["tokens"][:, 0] >= half), vmode          # drafts from p_d's support
        verified = res["cu_seqlens"][1:] - res["cu_seqlens"][:-1] - 1
        rej = verified > 0
        assert np.all(res["accept_len"][rej] == 0), vmode           # p_t(x) = 0: always rejected
        assert np.all(res["out_tokens"][:, 0] < half), vmode        # correction from p_t's support


def test_zero_residual_falls_back_to_target(dv):
    import torch
    sp = synth.small_spec("zeroresid", R=64, gamma=3, V=2000, r=32, d=8, dtype="bf16", seed=29,
                          W_std=0.0)
    inp = synth.generate(sp)
    R, g, V = sp.R, sp.gamma, sp.V
    inp["U"] = np.ascontiguousarray(inp["target"][:, :g, :])       # draft logits = target logits
    W1, W2 = factors64(inp)
    Uw = oracle.widen(inp["U"])
    m = Uw.max(axis=2)
    lse = m + np.log(np.exp(Uw - m[..., None]).sum(axis=2))
    rng = np.random.default_rng(5)
    tokens = rng.integers(0, V, size=(R, g)).astype(np.int32)
    # p_draft = 1 makes a reject likely at slot 1 (ratio = p_t(x)); a draft
    # normaliser 0.01 below the true one makes p_d > p_t at every entry on the
    # GPU, so no residual mass is left; the oracle recomputes p_d = p_t exactly
    p_draft = np.ones((R, g), dtype=np.float32)
    lse_draft = (lse - 0.01).astype(np.float32)
    dev, _ = upload(inp, sp)
    cu = np.arange(R + 1, dtype=np.int32) * (g + 1)
    W2p = dv.prepack_w2(dev["W2"])
    out = dv.verify(dev["target"].view(R * (g + 1), V), to_dev(cu), dev["anchor"], to_dev(tokens),
                    to_dev(p_draft), to_dev(lse_draft), dev["U"], dev["W1"], W2p, r=sp.r,
                    mode=MODES["static"], seed=3, step=11, req_ids=dev["req_ids"])
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res.update({"tokens": tokens, "p_draft": p_draft, "cu_seqlens": cu})
    rows = PackedView(inp["target"], cu)
    flips = check_verify(res, inp, rows, MODES["static"], None, 3, 11, np.arange(R), "zeroresid")
    ref = oracle.verify(rows, cu, inp["anchor"], tokens, p_draft, inp["U"], W1, W2, None,
                        MODES["static"], 3, 11, inp["req_ids"])
    kinds = [ref["trace"][r]["kind"] for r in range(R)]
    n_fb = sum(k == "residual->target" for k in kinds)
    assert all(k in ("residual->target", "bonus") for k in kinds), kinds
    assert n_fb >= R // 2, n_fb
    log(f"[edge] zero residual: {n_fb} of {R} corrections fell back to p_t; excused flips {flips}")


# ---------------------------------------------------------------------------
# scheduler: NaN and out-of-range survivals
# ---------------------------------------------------------------------------

def test_scheduler_nan_and_out_of_range_survivals(dv):
    import torch
    R, g = 30, 5
    sp = synth.small_spec("nansurv", R=R, gamma=g, V=100, r=8, d=8, dtype="f32", seed=31,
                          cost=("stair_T", 2e-3, 40e-6, 0.005))
    sps = dv.cost_table_prepare(synth.raw_step_time(sp), sp.tiers, sp.staircase)
    rng = np.random.default_rng(7)
    c = rng.uniform(0.3, 1.0, size=(R, g)).astype(np.float32)
    surv = np.cumprod(c, axis=1).astype(np.float32)
    surv[3, 2] = np.nan                  # NaN mid-row: read as 0, and 0 for the rest of the row
    surv[5, 0] = np.nan
    surv[7, :] = np.nan
    surv[9, 1] = np.inf                  # clamped to 1 (then the row's running minimum)
    surv[11, 0] = 1.5
    surv[13, 3] = -0.25                  # clamped to 0
    budget = surv[::-1].copy()
    budget[0, 0] = np.nan
    d_surv, d_budget, d_sps = to_dev(surv), to_dev(budget), to_dev(sps)
    spsl = [int(x) for x in sps]
    for mode in (oracle.SCHED_ARGMAX, oracle.SCHED_GREEDY, oracle.SCHED_FIXED):
        for bud in (None, budget):
            for B in (R * g, 37):
                win, K = dv.schedule_topb(d_surv, d_sps, B_cap=B, mode=mode, K_fixed=61,
                                          surv_budget=None if bud is None else d_budget)
                torch.cuda.synchronize()
                ref = oracle.schedule_topb(surv, spsl, B, mode, 61, bud)
                assert win.cpu().numpy().tolist() == ref["win_len"], (mode, bud is None, B)
                assert int(K.cpu()[0]) == ref["K"], (mode, bud is None, B)
    assert ref["win_len"][7] == 0


# ---------------------------------------------------------------------------
# chi-square of committed slot-1 tokens on the GPU
# ---------------------------------------------------------------------------

def _chi2_p(counts: np.ndarray, probs: np.ndarray) -> float:
    """Pearson chi-square p-value, cells with expected count < 5 pooled."""
    from scipy.stats import chisquare
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    obs_c, exp_c, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= 5.0:
            obs_c.append(acc_o)
            exp_c.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0 and exp_c:
        obs_c[-1] += acc_o
        exp_c[-1] += acc_e
    obs_c, exp_c = np.asarray(obs_c), np.asarray(exp_c)
    return float(chisquare(obs_c, exp_c * obs_c.sum() / exp_c.sum()).pvalue)


@pytest.mark.parametrize("vmode,smode", [("static", oracle.SCHED_ARGMAX),
                                         ("compact", oracle.SCHED_GREEDY)])
def test_committed_slot1_tokens_follow_target(dv, vmode, smode):
    import torch
    R, V, steps = 2048, 48, 5
    sp = synth.small_spec("chi2", R=R, gamma=1, V=V, r=16, d=8, dtype="bf16", seed=37,
                          W_std=0.3, target_std=1.5, zipf_s=None, noise=("const", 1.2), b=0.0)
    inp = synth.generate(sp)
    for key in ("U", "target", "h"):     # one set of logits shared by every request
        inp[key] = np.ascontiguousarray(np.broadcast_to(inp[key][:1], inp[key].shape))
    inp["anchor"] = np.full(R, inp["anchor"][0], dtype=np.int32)
    dev, _ = upload(inp, sp)
    committed, drafts = [], []
    for s in range(steps):
        ch = dv.Chain(dev, b=float(inp["b"]), tiers=sp.tiers, B_cap=R, verify_mode=MODES[vmode],
                      sched_mode=smode, seed=0, step=1000 + s)
        ch.run(gather=True)
        torch.cuda.synchronize()
        res = ch.results()
        committed.append(res["out_tokens"][:, 0])
        drafts.append(res["tokens"][:, 0])
    committed, drafts = np.concatenate(committed), np.concatenate(drafts)
    W1, W2 = factors64(inp)
    zt = oracle.widen(inp["target"][0, 0])
    p_t = np.exp(zt - zt.max())
    p_t /= p_t.sum()
    zd = oracle.markov_logits(inp["U"][0, 0], W1, W2, int(inp["anchor"][0]))
    p_d = np.exp(zd - zd.max())
    p_d /= p_d.sum()
    tv = 0.5 * np.abs(p_t - p_d).sum()
    p_commit = _chi2_p(np.bincount(committed, minlength=V).astype(float), p_t)
    p_draft = _chi2_p(np.bincount(drafts, minlength=V).astype(float), p_d)
    log(f"[edge] chi2 {vmode}: {committed.size} requests, TV(p_d, p_t) = {tv:.3f}, "
        f"p-value committed vs p_t {p_commit:.4f}, drafts vs p_d {p_draft:.4f}")
    assert tv > 0.1                       # the draft really differs from the target
    assert p_commit > 1e-4 and p_draft > 1e-4
    # the committed tokens do not follow the draft distribution
    assert _chi2_p(np.bincount(committed, minlength=V).astype(float), p_d) < 1e-6
