"""Markov sequential draft head (oracle, float64).

DSpark digest, "Architecture (drafter)": a parallel backbone emits base logits
U_1..U_gamma for a gamma-token block in one forward (the anchor x_0 fills the
first input position); a light sequential head then adds a prefix-dependent
transition bias, giving the causal factorisation
    p_k(v | x_0, x_<k) = softmax_v( U_k(v) + B_k(x_0, x_<k, v) ),
sampled left to right at inference. The Markov head makes the bias depend on
the previous token only, with the low-rank factorisation B = W1 W2: W1 in
R^{V x r} is read as a row lookup by the previous token and W2 in R^{r x V}
projects that row back to the vocabulary. Sampling temperature is 1 (the
digest's "Benchmark" section drafts chains at temperature 1.0).

Sampling is by inverse CDF over ascending vocabulary ids with a strict
comparison: x = min{ v : C_v > u * S }, C_v = sum_{i <= v} w_i, w = exp(z - max z),
S = sum w; if rounding leaves no such v, the largest id with w_v > 0 is taken.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .philox import uniforms, PURPOSE_DRAFT


def widen(a: np.ndarray) -> np.ndarray:
    """Stored input -> float64. uint16 arrays are bfloat16 bit patterns (the
    value is the top half of a float32); float32 arrays are widened exactly;
    float64 arrays (inputs a caller widened once) are returned as they are."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype == np.float64:
        return a                                 # already widened: no copy
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


def markov_logits(U_k: np.ndarray, W1: np.ndarray, W2: np.ndarray, x_prev) -> np.ndarray:
    """z = U_k + W1[x_prev] @ W2 in float64.

    U_k: [..., V] base logits of slot k; W1 [V, r]; W2 [r, V]; x_prev: token(s)
    at slot k-1 (the anchor when k = 1)."""
    e = widen(W1)[np.asarray(x_prev)]           # row lookup, [..., r]
    return widen(U_k) + e @ widen(W2)           # projection, [..., V]


def inverse_cdf(w: np.ndarray, t: float) -> int:
    """First id whose inclusive cumulative weight exceeds t; fallback: the last
    id with positive weight."""
    C = np.cumsum(w)
    idx = int(np.searchsorted(C, t, side="right"))
    if idx >= w.shape[0]:
        pos = np.nonzero(w > 0)[0]
        idx = int(pos[-1])
    return idx


def markov_step(U_k: np.ndarray, W1: np.ndarray, W2: np.ndarray, x_prev: Sequence[int],
                u: Sequence[float]) -> Dict[str, np.ndarray]:
    """One draft slot for a batch of requests.

    U_k [R, V]; x_prev [R]; u [R] draft uniforms. Returns tokens [R],
    p [R] (draft probability of the sampled token), lse [R] (max + ln S), and
    the per-row weights w [R, V] with their sums S [R] so that a test can judge
    how close a draw was to a cumulative boundary."""
    z = markov_logits(U_k, W1, W2, x_prev)
    R = z.shape[0]
    m = z.max(axis=1)
    w = np.exp(z - m[:, None])
    S = w.sum(axis=1)
    tokens = np.empty(R, dtype=np.int64)
    p = np.empty(R, dtype=np.float64)
    for i in range(R):
        t = float(u[i]) * S[i]
        x = inverse_cdf(w[i], t)
        tokens[i] = x
        p[i] = w[i, x] / S[i]
    return {"tokens": tokens, "p": p, "lse": m + np.log(S), "w": w, "S": S,
            "t": np.asarray(u, dtype=np.float64) * S}


def markov_draft(U: np.ndarray, W1: np.ndarray, W2: np.ndarray, anchor: np.ndarray,
                 seed: int, step: int, req_ids: np.ndarray,
                 teacher_tokens: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Draft a whole block: slots k = 1..gamma, left to right.

    U [R, gamma, V]; anchor [R] is x_0. The draft uniform of slot k of request
    r is word 0 of the Philox block (k, req_ids[r], step).

    teacher_tokens [R, gamma] (optional): condition slot k on
    teacher_tokens[:, k-1] instead of this oracle's own draw, so that each slot
    can be checked on its own against another implementation's chain.

    Returns tokens [R, gamma] int64, p_draft and lse_draft [R, gamma] float64,
    and per-slot step records (list of markov_step dicts) in "steps"."""
    R, gamma, V = U.shape
    tokens = np.empty((R, gamma), dtype=np.int64)
    p = np.empty((R, gamma), dtype=np.float64)
    lse = np.empty((R, gamma), dtype=np.float64)
    steps = []
    prev = np.asarray(anchor, dtype=np.int64)
    for k in range(1, gamma + 1):
        u = [uniforms(seed, step, int(req_ids[i]), k)[PURPOSE_DRAFT] for i in range(R)]
        rec = markov_step(U[:, k - 1, :], W1, W2, prev, u)
        tokens[:, k - 1] = rec["tokens"]
        p[:, k - 1] = rec["p"]
        lse[:, k - 1] = rec["lse"]
        rec["x_prev"] = prev.copy()
        steps.append(rec)
        prev = rec["tokens"] if teacher_tokens is None else np.asarray(teacher_tokens[:, k - 1], dtype=np.int64)
    return {"tokens": tokens, "p_draft": p, "lse_draft": lse, "steps": steps}
