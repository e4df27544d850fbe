"""Vocabulary-sharded Markov draft, with G ranks' calls issued on one device.

SGLang DSpark blog, "Performance optimisation and zero-overhead scheduling":
the block drafter's matmul is sharded. Rank g owns vocabulary columns
[b_g, b_{g+1}) with b_g = floor(g V / G): its slice of W2 (pre-packed on its
own) and of U. Per draft slot each rank runs the GEMM pass on its columns and
summarises them per request; the summaries are all-gathered; each rank runs
the shard select, where exactly one rank finds the token; a MAX / SUM
all-reduce hands every rank the token and its probability for the next slot.

Here every rank's buffers live on the one device, so the all-gather is the
shared [G, R, 2] summary buffer itself, and the two all-reduces are stood in
for by torch reductions over the rank axis (a multi-GPU build issues them as
RCCL collectives; they are not part of this library). Every other step runs
in the library's kernels.
"""
from __future__ import annotations

from typing import List, Optional

from . import (prepack_w2, new_workspace, markov_shard_partials, markov_shard_summary,
               markov_shard_select, CALL_MARKOV_DRAFT)


class ShardedDraft:
    """G-way vocabulary-sharded draft of a [R, gamma, V] block.

    U [R, gamma, V], W1 [V, r], W2 [r, V] device tensors (float32 or bfloat16).
    """

    def __init__(self, U, W1, W2, G: int):
        import torch
        self.t = torch
        self.U, self.W1 = U, W1
        self.R, self.gamma, self.V = U.shape
        self.r = W1.shape[1]
        self.G = int(G)
        if not 1 <= self.G <= min(64, self.V):
            raise ValueError("need 1 <= G <= min(64, V)")
        V, R, g, dev = self.V, self.R, self.gamma, U.device
        self.bounds = [s * V // self.G for s in range(self.G + 1)]
        self.W2p = [prepack_w2(W2[:, b0:b1].contiguous())
                    for b0, b1 in zip(self.bounds[:-1], self.bounds[1:])]
        self.ws = [new_workspace(CALL_MARKOV_DRAFT, R, 1, b1 - b0, self.r, dev)
                   for b0, b1 in zip(self.bounds[:-1], self.bounds[1:])]
        f32, i32 = torch.float32, torch.int32
        self.summaries = torch.empty((self.G, R, 2), dtype=f32, device=dev)
        self.tok_parts = torch.empty((self.G, R), dtype=i32, device=dev)
        self.p_parts = torch.empty((self.G, R), dtype=f32, device=dev)
        self.lse_parts = torch.empty((self.G, R), dtype=f32, device=dev)
        self.out = (torch.empty((R, g), dtype=i32, device=dev),
                    torch.empty((R, g), dtype=f32, device=dev),
                    torch.empty((R, g), dtype=f32, device=dev))

    def rank_slot(self, rank: int, k: int, x_prev, xstride: int, *, seed: int, step: int,
                  req_ids, phase: str, step_dev=None):
        """One rank's calls of slot k: phase "partials" (GEMM pass + summary)
        or "select"."""
        b0, b1 = self.bounds[rank], self.bounds[rank + 1]
        V, g = self.V, self.gamma
        Uk = self.U.view(-1)[(k - 1) * V + b0:]
        if phase == "partials":
            markov_shard_partials(Uk, g * V, self.W1, self.W2p[rank], x_prev, xstride, R=self.R,
                                  V_g=b1 - b0, V=V, r=self.r, part=self.ws[rank])
            markov_shard_summary(self.ws[rank], R=self.R, V_g=b1 - b0, out=self.summaries[rank])
        else:
            markov_shard_select(Uk, g * V, self.W1, self.W2p[rank], x_prev, xstride,
                                self.ws[rank], self.summaries, G=self.G, g=rank, v0=b0, k=k,
                                R=self.R, V_g=b1 - b0, V=V, r=self.r, seed=seed, step=step,
                                req_ids=req_ids, tok_out=self.tok_parts[rank],
                                p_out=self.p_parts[rank], lse_out=self.lse_parts[rank],
                                step_dev=step_dev)

    def draft(self, anchor, *, seed: int = 0, step: int = 0, req_ids=None, step_dev=None,
              owners: Optional[List] = None):
        """All gamma slots; returns (tokens, p_draft, lse_draft) like
        markov_draft. owners: optional list that receives, per slot, a device
        copy of the [G, R] per-rank token ids (-1 where a rank did not own
        the draw)."""
        torch = self.t
        if req_ids is None:
            req_ids = torch.arange(self.R, dtype=torch.int32, device=self.U.device)
        tok, p, lse = self.out
        tf = tok.view(-1)
        for k in range(1, self.gamma + 1):
            x_prev, xs = (anchor, 1) if k == 1 else (tf[k - 2:], self.gamma)
            for rank in range(self.G):
                self.rank_slot(rank, k, x_prev, xs, seed=seed, step=step, req_ids=req_ids,
                               phase="partials", step_dev=step_dev)
            # all-gather of the summaries: the shared buffer already holds them
            for rank in range(self.G):
                self.rank_slot(rank, k, x_prev, xs, seed=seed, step=step, req_ids=req_ids,
                               phase="select", step_dev=step_dev)
            # all-reduce stand-ins (MAX of the ids, SUM of the probabilities)
            tok[:, k - 1].copy_(self.tok_parts.amax(dim=0))
            p[:, k - 1].copy_(self.p_parts.sum(dim=0))
            lse[:, k - 1].copy_(self.lse_parts[0])
            if owners is not None:
                owners.append(self.tok_parts.clone())
        return self.out
