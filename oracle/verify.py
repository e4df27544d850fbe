"""Lossless rejection-sampling verification (oracle, float64).

DSpark digest, summary and "Architecture (drafter)": the target verifies a
drafted block in one forward and accepts, by rejection sampling, the longest
prefix that conforms; this is lossless because the Markov head keeps every
per-token draft probability an exact softmax.

SGLang DSpark blog, "Verify modes":
  * static     -- verify the whole drafted block every step;
  * compact    -- verify only each request's scheduled window (production);
  * cap-accept -- verify the whole block but commit only up to the window; it
                  commits exactly what compact commits and exposes what a full
                  verification would have accepted (the ceiling).

Per request r (the standard speculative-sampling rule):
  slot k = 1..Lv:  accept x_k when u1 < p_t(x_k) / p_d(x_k)   (i.e. with
                   probability min(1, p_t/p_d)); stop at the first rejection.
  first rejection at slot A+1 inside the commit window:
                   resample from the normalised residual max(0, p_t - p_d),
                   with p_d the draft distribution of that slot recomputed from
                   U, W1[x_A], W2; if rounding leaves no residual mass, sample
                   from p_t instead (exact arithmetic never gets there).
  whole commit window accepted:
                   sample a bonus token from p_t of slot L_commit + 1.
Packed target row cu[r] + j is the target distribution of slot j + 1 (row j
of a request holds token x_j, anchor first).

Uniforms: words 1 (accept), 2 (residual), 3 (bonus) of Philox block
(k, req_id, step) at the slot k they decide.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .markov import widen, markov_logits, inverse_cdf
from .philox import uniforms, PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_BONUS

VERIFY_STATIC = 0
VERIFY_COMPACT = 1
VERIFY_CAP_ACCEPT = 2


def _softmax(z: np.ndarray) -> np.ndarray:
    m = z.max()
    w = np.exp(z - m)
    return w / w.sum()


def verify(target_packed: np.ndarray, cu_seqlens: Sequence[int], anchor: Sequence[int],
           tokens: np.ndarray, p_draft: np.ndarray, U: np.ndarray, W1: np.ndarray,
           W2: np.ndarray, win_len: Optional[Sequence[int]], mode: int, seed: int, step: int,
           req_ids: Sequence[int], requests: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """target_packed [rows, V] (stored dtype); cu_seqlens [R+1]; tokens [R, gamma];
    p_draft [R, gamma]; U [R, gamma, V]; win_len [R] (CAP_ACCEPT only).

    requests: optional subset of request indices to verify (others are left at
    their fill values). Returns accept_len, out_tokens [R, gamma+1] (-1 fill),
    n_out, ceiling (leading accepts over every verified slot) and a per-request
    trace for tolerance checks."""
    tokens = np.asarray(tokens)
    R, gamma = tokens.shape
    pd_in = np.asarray(p_draft, dtype=np.float64)
    accept_len = np.full(R, -1, dtype=np.int64)
    n_out = np.full(R, -1, dtype=np.int64)
    ceiling = np.full(R, -1, dtype=np.int64)
    out = np.full((R, gamma + 1), -1, dtype=np.int64)
    trace: Dict[int, Dict[str, object]] = {}
    todo = range(R) if requests is None else requests
    for r in todo:
        rows = int(cu_seqlens[r + 1]) - int(cu_seqlens[r])
        Lv = rows - 1
        if mode == VERIFY_CAP_ACCEPT:
            L_commit = min(int(win_len[r]), Lv)
        else:
            L_commit = Lv
        rid = int(req_ids[r])
        ratios: List[float] = []
        us: List[float] = []
        A_full = 0
        for k in range(1, Lv + 1):
            zt = widen(target_packed[int(cu_seqlens[r]) + k - 1])
            pt = _softmax(zt)
            x = int(tokens[r, k - 1])
            ratio = pt[x] / pd_in[r, k - 1]
            u1 = uniforms(seed, step, rid, k)[PURPOSE_ACCEPT]
            ratios.append(float(ratio))
            us.append(u1)
            if u1 < ratio:
                A_full += 1
            else:
                break
        A = min(A_full, L_commit)
        if A < L_commit:
            slot = A + 1
            pt = _softmax(widen(target_packed[int(cu_seqlens[r]) + A]))
            x_prev = int(anchor[r]) if A == 0 else int(tokens[r, A - 1])
            pd = _softmax(markov_logits(U[r, A], W1, W2, x_prev))
            q = np.maximum(0.0, pt - pd)
            kind = "residual"
            if not q.sum() > 0.0:
                q = pt
                kind = "residual->target"
            u = uniforms(seed, step, rid, slot)[PURPOSE_RESIDUAL]
        else:
            slot = L_commit + 1
            q = _softmax(widen(target_packed[int(cu_seqlens[r]) + L_commit]))
            kind = "bonus"
            u = uniforms(seed, step, rid, slot)[PURPOSE_BONUS]
        t = u * q.sum()
        tok = inverse_cdf(q, t)
        out[r, :A] = tokens[r, :A]
        out[r, A] = tok
        accept_len[r] = A
        n_out[r] = A + 1
        ceiling[r] = A_full
        trace[r] = {"ratios": ratios, "u_accept": us, "kind": kind, "slot": slot,
                    "weights": q, "t": t, "token": tok, "A": A, "A_full": A_full,
                    "L_commit": L_commit}
    return {"accept_len": accept_len, "out_tokens": out, "n_out": n_out,
            "ceiling": ceiling, "trace": trace}
