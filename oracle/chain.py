"""The whole draft -> confidence -> schedule -> pack -> verify chain (oracle),
and the multi-step decode loop built from it.

One decode step of the chain as the DSpark pages describe it (DSpark digest,
"Architecture (drafter)" and "Verification scheduling (system side)"; SGLang
DSpark blog, "Verify modes" and "Ragged verify under full CUDA graphs"), with a
stand-in for the target forward: the target logits of request r, slot j+1 are
given as target[r, j] and gathered into packed order.

The decode loop (DSpark digest, "Infra (online production @ DeepSeek-V4)":
the cut length comes from confidences two steps back while the candidates are
ranked by the latest ones; vLLM adaptive verification page, "DSpark
confidence-scheduling mechanism": the budget comes from the previous step's
confidences) repeats the step with
  * x_0 of step t+1 = the last token step t committed for the request (the
    correction or bonus token, out_tokens[r, A_r]);
  * Philox step = step0 + t;
  * budget survivals of step t = the survivals of step t - lag (lag 0: the
    step's own survivals, as in a single step).
Reading: in the first `lag` steps no confidences that old exist yet. Those
steps run the non-anticipating greedy scheduler with its early stop over their
own survivals when the loop's mode is ARGMAX (the digest's "Verification
scheduling" algorithm, whose early stop is what keeps a same-step budget
lossless); GREEDY and FIXED loops run unchanged.
The synthetic stand-ins for the drafter's base logits U, its hidden states h
and the target logits stay the same at every step (no model runs here); the
drafts still change from step to step because x_0 and the Philox step do.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .markov import markov_draft
from .confidence import confidence
from .schedule import cost_table_prepare, schedule_topb, SCHED_ARGMAX, SCHED_GREEDY
from .pack import pack_ragged
from .verify import verify, VERIFY_STATIC, VERIFY_COMPACT, VERIFY_CAP_ACCEPT


def chain(inp: Dict[str, np.ndarray], *, tiers: Sequence[int], staircase: bool, B_cap: int,
          verify_mode: int, sched_mode: int = SCHED_ARGMAX, K_fixed: int = 0,
          seed: int = 0, step: int = 0,
          surv_budget: Optional[np.ndarray] = None) -> Dict[str, object]:
    U, W1, W2, anchor = inp["U"], inp["W1"], inp["W2"], inp["anchor"]
    req_ids = inp["req_ids"]
    R, gamma, V = U.shape
    d = markov_draft(U, W1, W2, anchor, seed, step, req_ids)
    c = confidence(inp["h"], W1, anchor, d["tokens"], inp["w"], float(inp["b"]))
    surv32 = c["surv"].astype(np.float32)
    sps = cost_table_prepare(inp["raw_T"], tiers, staircase)
    sched = schedule_topb(surv32, sps, B_cap, sched_mode, K_fixed, surv_budget)
    M_cap = R * (gamma + 1)
    win = None if verify_mode in (VERIFY_STATIC, VERIFY_CAP_ACCEPT) else sched["win_len"]
    pk = pack_ragged(anchor, d["tokens"], win, tiers, M_cap)
    target = inp["target"]
    rows = np.zeros((M_cap, V), dtype=target.dtype)
    cu = pk["cu_seqlens"]
    for r in range(R):
        n = cu[r + 1] - cu[r]
        rows[cu[r]:cu[r + 1]] = target[r, :n]
    v = verify(rows, cu, anchor, d["tokens"], d["p_draft"], U, W1, W2, sched["win_len"],
               verify_mode, seed, step, req_ids)
    return {"draft": d, "conf": c, "sps_milli": sps, "sched": sched, "pack": pk,
            "verify": v, "target_packed": rows}


def decode(inp: Dict[str, np.ndarray], *, steps: int, lag: int, tiers: Sequence[int],
           staircase: bool, B_cap: int, verify_mode: int, sched_mode: int = SCHED_ARGMAX,
           K_fixed: int = 0, seed: int = 0, step0: int = 0) -> List[Dict[str, object]]:
    """`steps` chain steps in a row; returns each step's chain() result with the
    step's anchor, budget survivals and scheduler mode added under "anchor",
    "surv_budget" and "sched_mode"."""
    if lag < 0:
        raise ValueError("lag must be >= 0")
    R = inp["U"].shape[0]
    anchor = np.array(inp["anchor"], dtype=np.int32)
    history: List[np.ndarray] = []     # survivals of the steps so far, oldest first
    out: List[Dict[str, object]] = []
    for t in range(steps):
        budget = history[t - lag] if (lag > 0 and t >= lag) else None
        mode_t = sched_mode
        if lag > 0 and t < lag and sched_mode == SCHED_ARGMAX:
            mode_t = SCHED_GREEDY
        res = chain({**inp, "anchor": anchor}, tiers=tiers, staircase=staircase, B_cap=B_cap,
                    verify_mode=verify_mode, sched_mode=mode_t, K_fixed=K_fixed, seed=seed,
                    step=step0 + t, surv_budget=budget)
        res["sched_mode"] = mode_t
        res["anchor"] = anchor
        res["surv_budget"] = budget
        out.append(res)
        history.append(res["conf"]["surv"].astype(np.float32))
        v = res["verify"]
        anchor = np.array([v["out_tokens"][r, v["accept_len"][r]] for r in range(R)],
                          dtype=np.int32)
    return out
