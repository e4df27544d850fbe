"""The whole draft -> confidence -> schedule -> pack -> verify chain (oracle).

One decode step of the chain as the DSpark pages describe it (DSpark digest,
"Architecture (drafter)" and "Verification scheduling (system side)"; SGLang
DSpark blog, "Verify modes" and "Ragged verify under full CUDA graphs"), with a
stand-in for the target forward: the target logits of request r, slot j+1 are
given as target[r, j] and gathered into packed order.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .markov import markov_draft
from .confidence import confidence
from .schedule import cost_table_prepare, schedule_topb, SCHED_ARGMAX
from .pack import pack_ragged
from .verify import verify, VERIFY_STATIC, VERIFY_COMPACT, VERIFY_CAP_ACCEPT


def chain(inp: Dict[str, np.ndarray], *, tiers: Sequence[int], staircase: bool, B_cap: int,
          verify_mode: int, sched_mode: int = SCHED_ARGMAX, K_fixed: int = 0,
          seed: int = 0, step: int = 0) -> Dict[str, object]:
    U, W1, W2, anchor = inp["U"], inp["W1"], inp["W2"], inp["anchor"]
    req_ids = inp["req_ids"]
    R, gamma, V = U.shape
    d = markov_draft(U, W1, W2, anchor, seed, step, req_ids)
    c = confidence(inp["h"], W1, anchor, d["tokens"], inp["w"], float(inp["b"]))
    surv32 = c["surv"].astype(np.float32)
    sps = cost_table_prepare(inp["raw_T"], tiers, staircase)
    sched = schedule_topb(surv32, sps, B_cap, sched_mode, K_fixed)
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
