"""Ragged verify packing (oracle).

SGLang DSpark blog, "Ragged verify under full CUDA graphs": the per-request
verify windows are packed front to back into one compact buffer that is a
cu_seqlens-style variable-length input, and the packed total is rounded up to
the nearest captured tier, so a trimmed batch replays a genuinely smaller
graph. vLLM adaptive verification page, "Technical implementation & CUDA
graphs": padding makes cost a staircase (121 tokens cost the 128-token graph);
"Configuration & reproduction": the largest verify batch is
(num_speculative_tokens + 1) * max_num_seq.

Each request r contributes 1 + L_r rows: its anchor x_0, then drafts
x_1..x_{L_r}. cu[0] = 0, cu[r+1] = cu[r] + 1 + L_r, M = cu[R], M_pad = the
smallest tier >= M, or -1 when M exceeds every tier (reading: the pages give no
rule for overflow). Rows [M, M_cap) hold token 0, request -1, slot -1.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def pack_ragged(anchor: Sequence[int], tokens: np.ndarray, win_len: Optional[Sequence[int]],
                tiers: Sequence[int], M_cap: int) -> Dict[str, object]:
    tokens = np.asarray(tokens)
    R, gamma = tokens.shape
    L = [gamma] * R if win_len is None else [int(x) for x in win_len]
    cu = [0]
    for r in range(R):
        cu.append(cu[-1] + 1 + L[r])
    M = cu[-1]
    M_pad = -1
    for t in tiers:
        if t >= M:
            M_pad = int(t)
            break
    ptok = [0] * M_cap
    preq = [-1] * M_cap
    pslot = [-1] * M_cap
    for r in range(R):
        for j in range(L[r] + 1):
            i = cu[r] + j
            ptok[i] = int(anchor[r]) if j == 0 else int(tokens[r, j - 1])
            preq[i] = r
            pslot[i] = j
    return {"cu_seqlens": cu, "packed_tokens": ptok, "packed_req": preq,
            "packed_slot": pslot, "M": M, "M_pad": M_pad}
