"""Helpers for GPU parity tests: device upload of synth inputs, the tolerance
rules, and stage-by-stage comparison of the HIP chain against the oracle.

Tolerances:
  * ids, lengths, selection and packing: bit-exact;
  * probabilities, log-sum-exps, confidences, survivals: 1e-5 absolute;
  * an accept/reject decision may differ only where |u - p_t/p_d| < 1e-5;
  * an inverse-CDF draw may differ only where every oracle cumulative
    boundary between the two ids lies within 1e-5 * S of the threshold u * S.
"""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np

import oracle
import synth

TOL = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray):
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    if arr.dtype == np.uint32:
        return torch.from_numpy(arr.view(np.int32)).cuda()
    return torch.from_numpy(arr).cuda()


def upload(inp: Dict[str, np.ndarray], spec: synth.Spec):
    import draft_verify_sampling_markov_amd as dv
    dev = {k: to_dev(inp[k]) for k in ("U", "W1", "W2", "target", "h", "anchor", "w")}
    dev["req_ids"] = to_dev(inp["req_ids"])
    sps = dv.cost_table_prepare(inp["raw_T"], spec.tiers, spec.staircase)
    dev["sps_milli"] = to_dev(sps)
    return dev, sps


class PackedView:
    """Packed target rows read lazily from a [R, gamma+1, V] source."""

    def __init__(self, target: np.ndarray, cu: Sequence[int]):
        self.target = target
        self.cu = np.asarray(cu)

    def __getitem__(self, i: int):
        r = int(np.searchsorted(self.cu, i, side="right")) - 1
        return self.target[r, i - int(self.cu[r])]


def factors64(inp):
    """W1 and W2 widened to float64 once per input dict (the oracle widens
    stored values exactly and passes float64 through, so its results are the
    same; this only avoids re-widening the whole factors on every call)."""
    if "_W64" not in inp:
        inp["_W64"] = (oracle.widen(inp["W1"]), oracle.widen(inp["W2"]))
    return inp["_W64"]


def draw_ok(w: np.ndarray, t: float, g: int, o: int, tol: float = TOL) -> bool:
    """GPU id g vs oracle id o for weights w and threshold t."""
    if g == o:
        return True
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    S = C[-1]
    lo, hi = min(g, o), max(g, o)
    return bool(np.all(np.abs(C[lo:hi] - t) <= tol * S))


def check_draft(res, inp, seed, step, reqs, label="") -> int:
    """Teacher-forced per slot: slot k is conditioned on the GPU's x_{k-1}.
    Returns the number of (excused) draw flips."""
    tokens, p, lse = res["tokens"], res["p_draft"], res["lse_draft"]
    R, gamma = tokens.shape
    flips = 0
    reqs = np.asarray(reqs)
    W1, W2 = factors64(inp)
    for k in range(1, gamma + 1):
        x_prev = inp["anchor"][reqs] if k == 1 else tokens[reqs, k - 2]
        u = [oracle.uniforms(seed, step, int(inp["req_ids"][r]), k)[oracle.PURPOSE_DRAFT] for r in reqs]
        rec = oracle.markov_step(inp["U"][reqs, k - 1], W1, W2, x_prev, u)
        for i, r in enumerate(reqs):
            g, o = int(tokens[r, k - 1]), int(rec["tokens"][i])
            assert 0 <= g < inp["U"].shape[2], (label, r, k, g)
            assert draw_ok(rec["w"][i], rec["t"][i], g, o), (label, "draft", r, k, g, o)
            flips += g != o
            p_ref = rec["w"][i, g] / rec["S"][i]
            assert abs(float(p[r, k - 1]) - p_ref) <= TOL, (label, "p_draft", r, k, p[r, k - 1], p_ref)
            assert abs(float(lse[r, k - 1]) - rec["lse"][i]) <= TOL, (label, "lse", r, k, lse[r, k - 1], rec["lse"][i])
    return flips


def check_confidence(res, inp, reqs, label=""):
    reqs = np.asarray(reqs)
    ref = oracle.confidence(inp["h"][reqs], factors64(inp)[0], inp["anchor"][reqs], res["tokens"][reqs],
                            inp["w"], float(inp["b"]))
    np.testing.assert_allclose(res["conf"][reqs], ref["conf"], rtol=0, atol=TOL, err_msg=label)
    np.testing.assert_allclose(res["surv"][reqs], ref["surv"], rtol=0, atol=TOL, err_msg=label)
    assert np.all(np.diff(res["surv"], axis=1) <= 0), label


def check_schedule(res, sps, B_cap, mode, K_fixed=0, label="", budget=None):
    ref = oracle.schedule_topb(res["surv"], [int(x) for x in sps], B_cap, mode, K_fixed, budget)
    assert res["win_len"].tolist() == ref["win_len"], label
    assert int(res["K"][0]) == ref["K"], label
    return ref


def check_pack(res, inp, win, tiers, M_cap, label=""):
    ref = oracle.pack_ragged(inp["anchor"], res["tokens"], win, tiers, M_cap)
    assert res["cu_seqlens"].tolist() == ref["cu_seqlens"], label
    assert res["packed_tokens"].tolist() == ref["packed_tokens"], label
    assert res["packed_req"].tolist() == ref["packed_req"], label
    assert res["packed_slot"].tolist() == ref["packed_slot"], label
    assert res["totals"].tolist() == [ref["M"], ref["M_pad"]], label
    return ref


def check_verify(res, inp, target_rows, mode, win_len, seed, step, reqs, label="") -> int:
    """Teacher-forced: the oracle verifies the GPU's drafts with the GPU's
    p_draft and packing. Returns the number of excused flips."""
    cu = res["cu_seqlens"]
    W1, W2 = factors64(inp)
    ref = oracle.verify(target_rows, cu, inp["anchor"], res["tokens"], res["p_draft"], inp["U"],
                        W1, W2, win_len, mode, seed, step, inp["req_ids"],
                        requests=[int(r) for r in reqs])
    flips = 0
    for r in reqs:
        r = int(r)
        tr = ref["trace"][r]
        cg, co = int(res["ceiling_len"][r]), int(ref["ceiling"][r])
        if cg != co:
            k0 = min(cg, co)
            assert abs(tr["u_accept"][k0] - tr["ratios"][k0]) < TOL, (label, "accept", r, k0, cg, co)
            flips += 1
            continue
        A = int(ref["accept_len"][r])
        assert int(res["accept_len"][r]) == A, (label, "A", r)
        assert int(res["n_out"][r]) == A + 1, (label, "n_out", r)
        assert res["out_tokens"][r, :A].tolist() == ref["out_tokens"][r, :A].tolist(), (label, r)
        assert np.all(res["out_tokens"][r, A + 1:] == -1), (label, "pad", r)
        g, o = int(res["out_tokens"][r, A]), int(ref["out_tokens"][r, A])
        assert 0 <= g < inp["U"].shape[2], (label, r, g)
        assert draw_ok(tr["weights"], tr["t"], g, o), (label, "corr", tr["kind"], r, g, o)
        flips += g != o
    return flips


def sample_requests(R: int, n: int, seed: int = 0) -> np.ndarray:
    if R <= n:
        return np.arange(R)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(R, size=n - 2, replace=False).tolist()) | {0, R - 1}
    return np.array(sorted(pick))


MODES = {"static": 0, "compact": 1, "cap_accept": 2}


def run_and_check(dv, spec, vmode: str, smode: int = oracle.SCHED_ARGMAX, B_cap=None, K_fixed=0,
                  sample=None, seed=0, step=0, inp=None, check_draft_conf: bool = True):
    """One chain step on the GPU (Chain.run), then every stage teacher-forced
    against the oracle. sample=None checks every request; check_draft_conf=
    False skips the draft and confidence checks (a caller that already checked
    them on the same inputs, seed and step, e.g. a budget sweep)."""
    import torch
    label = f"{spec.name}/{vmode}/sched{smode}/B{B_cap}"
    log(f"[parity] {label}: R={spec.R} gamma={spec.gamma} V={spec.V} r={spec.r} dtype={spec.dtype}")
    if inp is None:
        inp = synth.generate(spec)
    dev, sps = upload(inp, spec)
    B = spec.budgets[0] if B_cap is None else B_cap
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=B, verify_mode=MODES[vmode],
                  sched_mode=smode, K_fixed=K_fixed, seed=seed, step=step)
    ch.run(gather=True)
    torch.cuda.synchronize()
    res = ch.results()
    reqs = np.arange(spec.R) if sample is None else sample_requests(spec.R, sample)
    flips = 0
    if check_draft_conf:
        flips += check_draft(res, inp, seed, step, reqs, label)
        check_confidence(res, inp, reqs, label)
    ref_s = check_schedule(res, sps, B, smode, K_fixed, label)
    full = vmode in ("static", "cap_accept")
    check_pack(res, inp, None if full else ref_s["win_len"], spec.tiers, ch.M_cap, label)
    rows = PackedView(inp["target"], res["cu_seqlens"])
    flips += check_verify(res, inp, rows, MODES[vmode], res["win_len"], seed, step, reqs, label)
    log(f"[parity] {label}: ok over {len(reqs)} requests, K={int(res['K'][0])} "
        f"M={res['totals'].tolist()} mean A={res['accept_len'].mean():.2f} excused flips={flips}")
    return res, ch
