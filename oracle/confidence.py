"""Confidence head and prefix survival (oracle, float64).

DSpark digest, "Verification scheduling (system side)": the confidence head
scores every draft slot with c_k in (0, 1), the probability that draft k passes
verification given that its whole prefix was accepted; it is a sigmoid of a
linear projection of the concatenation [h_k ; W1[x_{k-1}]] (the hidden state of
slot k, then the Markov embedding of the previous token). The prefix survival
of slot j of request r is the running product a_{r,j} = prod_{i <= j} c_{r,i}.

Sequential temperature scaling calibrates these scores per position; the pages
give no formula, so an optional per-position inverse temperature multiplies the
logit (c = sigmoid(z * inv_temp_k)); with none given it is 1.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .markov import widen


def confidence(h: np.ndarray, W1: np.ndarray, anchor: np.ndarray, tokens: np.ndarray,
               w: np.ndarray, b: float, inv_temp: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """h [R, gamma, d]; W1 [V, r]; anchor [R]; tokens [R, gamma]; w [d + r]; b.

    Returns conf, surv and logit (the head's pre-temperature logit z) [R, gamma]
    in float64."""
    hh = widen(h)
    W1w = widen(W1)
    ww = np.asarray(w, dtype=np.float64)
    R, gamma, d = hh.shape
    conf = np.empty((R, gamma), dtype=np.float64)
    surv = np.empty((R, gamma), dtype=np.float64)
    logit = np.empty((R, gamma), dtype=np.float64)
    for r in range(R):
        a = 1.0
        for k in range(1, gamma + 1):
            prev = int(anchor[r]) if k == 1 else int(tokens[r, k - 2])
            feat = np.concatenate([hh[r, k - 1], W1w[prev]])
            z = float(feat @ ww) + float(b)
            logit[r, k - 1] = z
            if inv_temp is not None:
                z *= float(inv_temp[k - 1])
            c = 1.0 / (1.0 + np.exp(-z))
            a = a * c
            conf[r, k - 1] = c
            surv[r, k - 1] = a
    return {"conf": conf, "surv": surv, "logit": logit}
