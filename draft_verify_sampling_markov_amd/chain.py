"""One decode step of the DSpark chain over preallocated device buffers.

draft (dspark_markov_draft) -> confidence (dspark_confidence) -> schedule
(dspark_schedule_topb) -> pack (dspark_pack_ragged) -> [target forward] ->
verify (dspark_verify), all enqueued on one stream with no host read-back.

The target forward is outside this library. ``gather_target`` stands in for
it: it copies the target logits of each packed row (request r, slot j) from a
[R, gamma+1, V] source into packed order with one torch index_select. For the
full-block modes (static, cap-accept) the packed order is the source's own
row order, so the source is used as is.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

from . import (markov_draft, markov_partials, markov_select, confidence, schedule_topb,
               pack_ragged, verify, prepack_w2, new_workspace, CALL_MARKOV_DRAFT, CALL_VERIFY,
               VERIFY_STATIC, VERIFY_CAP_ACCEPT, SCHED_ARGMAX)


class Chain:
    """Buffers and calls for repeated chain steps on one batch.

    inputs: dict of device tensors U [R, gamma, V], W1 [V, r], W2 [r, V],
    target [R, gamma+1, V] (same dtype), h [R, gamma, d], anchor [R] int32,
    w [d+r] f32, req_ids [R] int32, sps_milli [M_max+1] int32 (uint32 bits).
    """

    def __init__(self, inputs: Dict[str, "object"], *, b: float, tiers: Sequence[int],
                 B_cap: int, verify_mode: int, sched_mode: int = SCHED_ARGMAX, K_fixed: int = 0,
                 seed: int = 0, step: int = 0, W2p=None):
        import torch
        self.t = torch
        self.inp = inputs
        U = inputs["U"]
        self.R, self.gamma, self.V = U.shape
        self.r = inputs["W1"].shape[1]
        self.b = float(b)
        self.tiers = list(tiers)
        self.B_cap = int(B_cap)
        self.verify_mode = int(verify_mode)
        self.sched_mode = int(sched_mode)
        self.K_fixed = int(K_fixed)
        self.seed, self.step = int(seed), int(step)
        dev = U.device
        R, g, V, r = self.R, self.gamma, self.V, self.r
        self.M_cap = R * (g + 1)
        self.W2p = W2p if W2p is not None else prepack_w2(inputs["W2"])
        i32, f32, u8 = torch.int32, torch.float32, torch.uint8
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.draft_out = (e((R, g), i32), e((R, g), f32), e((R, g), f32))
        self.conf_out = (e((R, g), f32), e((R, g), f32))
        self.sched_out = (e((R,), i32), e((1,), i32))
        self.pack_out = {"cu_seqlens": e((R + 1,), i32), "packed_tokens": e((self.M_cap,), i32),
                         "packed_req": e((self.M_cap,), i32), "packed_slot": e((self.M_cap,), i32),
                         "totals": e((2,), i32)}
        self.verify_out = {"accept_len": e((R,), i32), "out_tokens": e((R, g + 1), i32),
                           "n_out": e((R,), i32), "ceiling_len": e((R,), i32)}
        self.ws_draft = new_workspace(CALL_MARKOV_DRAFT, R, g, V, r, dev)
        self.ws_verify = new_workspace(CALL_VERIFY, R, g, V, r, dev)
        self.full_block = self.verify_mode in (VERIFY_STATIC, VERIFY_CAP_ACCEPT)
        self.target_packed = (inputs["target"].view(self.M_cap, V) if self.full_block
                              else e((self.M_cap, V), U.dtype))

    # -- stages ------------------------------------------------------------
    def draft(self):
        i = self.inp
        return markov_draft(i["U"], i["W1"], self.W2p, i["anchor"], r=self.r, seed=self.seed,
                            step=self.step, req_ids=i["req_ids"], out=self.draft_out,
                            ws=self.ws_draft)

    def draft_split(self, events=None):
        """The draft as its two per-slot passes -- the same launches draft()
        makes through dspark_markov_draft. ``events``: optional list of gamma
        (start, end) torch.cuda.Event pairs recorded around each slot's GEMM +
        partials launch, on the current stream."""
        i = self.inp
        U, W1 = i["U"], i["W1"]
        tok, p, lse = self.draft_out
        g, V = self.gamma, self.V
        Uf, tf, pf, lf = U.view(-1), tok.view(-1), p.view(-1), lse.view(-1)
        for k in range(1, g + 1):
            Uk = Uf[(k - 1) * V:]
            x_prev, xs = (i["anchor"], 1) if k == 1 else (tf[k - 2:], g)
            if events is not None:
                events[k - 1][0].record()
            markov_partials(Uk, g * V, W1, self.W2p, x_prev, xs, R=self.R, V=V, r=self.r,
                            part=self.ws_draft)
            if events is not None:
                events[k - 1][1].record()
            markov_select(Uk, g * V, W1, self.W2p, x_prev, xs, self.ws_draft, k=k, R=self.R, V=V,
                          r=self.r, seed=self.seed, step=self.step, req_ids=i["req_ids"],
                          tok_out=tf[k - 1:], p_out=pf[k - 1:], lse_out=lf[k - 1:], ostride=g)

    def confidence(self):
        i = self.inp
        return confidence(i["h"], i["W1"], i["anchor"], self.draft_out[0], i["w"], self.b,
                          out=self.conf_out)

    def schedule(self):
        return schedule_topb(self.conf_out[1], self.inp["sps_milli"], B_cap=self.B_cap,
                             mode=self.sched_mode, K_fixed=self.K_fixed, out=self.sched_out)

    def pack(self):
        win = None if self.full_block else self.sched_out[0]
        return pack_ragged(self.inp["anchor"], self.draft_out[0], win, self.tiers, self.M_cap,
                           out=self.pack_out)

    def gather_target(self):
        """Stand-in for the target forward (not part of the chain)."""
        if self.full_block:
            return self.target_packed
        t = self.t
        req = self.pack_out["packed_req"].clamp(min=0).long()
        slot = self.pack_out["packed_slot"].clamp(min=0).long()
        idx = req * (self.gamma + 1) + slot
        src = self.inp["target"].view(self.R * (self.gamma + 1), self.V)
        t.index_select(src, 0, idx, out=self.target_packed)
        return self.target_packed

    def verify(self):
        i = self.inp
        d = self.draft_out
        return verify(self.target_packed, self.pack_out["cu_seqlens"], i["anchor"], d[0], d[1],
                      d[2], i["U"], i["W1"], self.W2p, r=self.r, mode=self.verify_mode,
                      win_len=self.sched_out[0], seed=self.seed, step=self.step,
                      req_ids=i["req_ids"], out=self.verify_out, ws=self.ws_verify)

    def run(self, gather: bool = True):
        """One whole step; ``gather`` re-runs the target stand-in between pack
        and verify (needed whenever the windows may have changed)."""
        self.draft()
        self.confidence()
        self.schedule()
        self.pack()
        if gather:
            self.gather_target()
        self.verify()

    def results(self) -> Dict[str, "object"]:
        """Host copies of every stage output (synchronises)."""
        d, c, s = self.draft_out, self.conf_out, self.sched_out
        out = {"tokens": d[0], "p_draft": d[1], "lse_draft": d[2], "conf": c[0], "surv": c[1],
               "win_len": s[0], "K": s[1], **self.pack_out, **self.verify_out}
        return {k: v.cpu().numpy() for k, v in out.items()}
