"""Decode steps of the DSpark chain over preallocated device buffers.

draft and confidence (dspark_markov_draft_confidence, or dspark_markov_draft
then dspark_confidence) -> schedule and pack (dspark_schedule_pack, or
dspark_schedule_topb then dspark_pack_ragged) -> [target forward] -> verify
(dspark_verify), all enqueued on one stream with no host read-back.
``decode`` repeats the step, carrying x_0, the Philox step and a short
survival history from one step to the next on the device (dspark_advance), so
that the verify budget can come from confidences ``lag`` steps old (DSpark
digest, "Infra": two steps back; vLLM adaptive verification page, "Execution
pipeline": the previous step); the steady-state step can be captured once
into a HIP graph and replayed.

The target forward is outside this library. ``gather_target`` stands in for
it: it copies the target logits of each packed row (request r, slot j) from a
[R, gamma+1, V] source into packed order with one torch index_select. For the
full-block modes (static, cap-accept) the packed order is the source's own
row order, so the source is used as is.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

from . import (markov_draft, markov_draft_confidence, markov_partials, markov_select, confidence,
               schedule_topb, schedule_pack,
               pack_ragged, verify, advance, observe, new_observe_block, parse_observe,
               analytic_accept, prepack_w2, new_workspace, CALL_MARKOV_DRAFT, CALL_VERIFY,
               CALL_ANALYTIC_ACCEPT, VERIFY_STATIC, VERIFY_CAP_ACCEPT, SCHED_ARGMAX, SCHED_GREEDY)


class Chain:
    """Buffers and calls for repeated chain steps on one batch.

    inputs: dict of device tensors U [R, gamma, V], W1 [V, r], W2 [r, V],
    target [R, gamma+1, V] (same dtype), h [R, gamma, d], anchor [R] int32,
    w [d+r] f32, req_ids [R] int32, sps_milli [M_max+1] int32 (uint32 bits).
    The chain keeps its own copy of the anchors (``self.anchor``), which
    ``decode`` moves on from step to step.

    inv_temp: optional f32 [gamma] device tensor of per-position inverse
    temperatures for the confidence head (sequential temperature scaling,
    from sts_fit); keep_logits=True also keeps the head's pre-temperature
    logits in ``logit_out``.

    Optional observability, run after every verify when enabled:
    observe_bins > 0 accumulates dspark_observe counts into ``obs_block``
    (read with ``observe_summary``); analytic=True writes the analytic
    acceptance c* of every verified slot into ``cstar``.
    """

    def __init__(self, inputs: Dict[str, "object"], *, b: float, tiers: Sequence[int],
                 B_cap: int, verify_mode: int, sched_mode: int = SCHED_ARGMAX, K_fixed: int = 0,
                 seed: int = 0, step: int = 0, W2p=None, observe_bins: int = 0,
                 analytic: bool = False, inv_temp=None, keep_logits: bool = False):
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
        self.anchor = inputs["anchor"].clone()
        self.step_dev = torch.tensor([self.step], dtype=torch.int64, device=dev)
        self.surv_hist = None
        self._graph = None
        self._hist_steps = 0      # steps whose survivals the history holds (at most lag)
        self._lag = None          # history depth the buffers and graph were made for
        self._warm = False        # an eager decode step has run (every kernel loaded)
        R, g, V, r = self.R, self.gamma, self.V, self.r
        self.M_cap = R * (g + 1)
        self.W2p = W2p if W2p is not None else prepack_w2(inputs["W2"])
        i32, f32, u8 = torch.int32, torch.float32, torch.uint8
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.draft_out = (e((R, g), i32), e((R, g), f32), e((R, g), f32))
        self.conf_out = (e((R, g), f32), e((R, g), f32))
        self.inv_temp = inv_temp
        self.logit_out = e((R, g), f32) if keep_logits else None
        self.sched_out = (e((R,), i32), e((1,), i32))
        self.pack_out = {"cu_seqlens": e((R + 1,), i32), "packed_tokens": e((self.M_cap,), i32),
                         "packed_req": e((self.M_cap,), i32), "packed_slot": e((self.M_cap,), i32),
                         "totals": e((2,), i32)}
        self.verify_out = {"accept_len": e((R,), i32), "out_tokens": e((R, g + 1), i32),
                           "n_out": e((R,), i32), "ceiling_len": e((R,), i32)}
        self.ws_draft = new_workspace(CALL_MARKOV_DRAFT, R, g, V, r, dev)
        self.ws_verify = new_workspace(CALL_VERIFY, R, g, V, r, dev)
        self.n_bins = int(observe_bins)
        self.obs_block = new_observe_block(R, g, self.n_bins, dev) if self.n_bins else None
        self.analytic = bool(analytic)
        self.cstar = e((R, g), f32) if self.analytic else None
        self.ws_accept = (new_workspace(CALL_ANALYTIC_ACCEPT, R, g, V, r, dev) if self.analytic
                          else None)
        self.full_block = self.verify_mode in (VERIFY_STATIC, VERIFY_CAP_ACCEPT)
        self.target_packed = (inputs["target"].view(self.M_cap, V) if self.full_block
                              else e((self.M_cap, V), U.dtype))

    # -- stages ------------------------------------------------------------
    def draft(self):
        i = self.inp
        return markov_draft(i["U"], i["W1"], self.W2p, self.anchor, r=self.r, seed=self.seed,
                            step=self.step, req_ids=i["req_ids"], out=self.draft_out,
                            ws=self.ws_draft)

    def draft_confidence(self, step_dev=None):
        """The draft and the confidence head in one call (dspark_markov_draft_
        confidence): each slot's GEMM launch also scores the slot."""
        i = self.inp
        markov_draft_confidence(i["U"], i["W1"], self.W2p, self.anchor, i["h"], i["w"], self.b,
                                r=self.r, inv_temp=self.inv_temp, seed=self.seed,
                                step=self.step, step_dev=step_dev, req_ids=i["req_ids"],
                                out=self.draft_out, conf_out=self.conf_out, logit=self.logit_out,
                                ws=self.ws_draft)

    def draft_split(self, events=None, passes=("partials", "select")):
        """The draft as its two per-slot passes, through the split calls: the
        same GEMM and select kernels dspark_markov_draft launches, except that
        the slot's draft uniform is drawn in the select rather than in the
        GEMM's prologue. ``events``: optional list of gamma (start, end)
        torch.cuda.Event pairs recorded around each slot's GEMM + partials
        launch, on the current stream. ``passes``: ("select",) re-runs only
        the selects over the partials already in the workspace (repeatable:
        a select reads the partials and leaves the tile queue at zero)."""
        i = self.inp
        U, W1 = i["U"], i["W1"]
        tok, p, lse = self.draft_out
        g, V = self.gamma, self.V
        Uf, tf, pf, lf = U.view(-1), tok.view(-1), p.view(-1), lse.view(-1)
        for k in range(1, g + 1):
            Uk = Uf[(k - 1) * V:]
            x_prev, xs = (self.anchor, 1) if k == 1 else (tf[k - 2:], g)
            if "partials" in passes:
                if events is not None:
                    events[k - 1][0].record()
                markov_partials(Uk, g * V, W1, self.W2p, x_prev, xs, R=self.R, V=V, r=self.r,
                                part=self.ws_draft)
                if events is not None:
                    events[k - 1][1].record()
            if "select" in passes:
                markov_select(Uk, g * V, W1, self.W2p, x_prev, xs, self.ws_draft, k=k, R=self.R,
                              V=V, r=self.r, seed=self.seed, step=self.step,
                              req_ids=i["req_ids"], tok_out=tf[k - 1:], p_out=pf[k - 1:],
                              lse_out=lf[k - 1:], ostride=g)

    def confidence(self):
        i = self.inp
        return confidence(i["h"], i["W1"], self.anchor, self.draft_out[0], i["w"], self.b,
                          inv_temp=self.inv_temp, out=self.conf_out, logit=self.logit_out)

    def schedule(self):
        return schedule_topb(self.conf_out[1], self.inp["sps_milli"], B_cap=self.B_cap,
                             mode=self.sched_mode, K_fixed=self.K_fixed, out=self.sched_out)

    def schedule_and_pack(self, mode=None, budget=None):
        """The scheduler and the pack in one launch (dspark_schedule_pack)."""
        schedule_pack(self.conf_out[1], self.inp["sps_milli"], self.anchor, self.draft_out[0],
                      self.tiers, self.M_cap, B_cap=self.B_cap,
                      mode=self.sched_mode if mode is None else mode, K_fixed=self.K_fixed,
                      surv_budget=budget, pack_windows=not self.full_block,
                      sched_out=self.sched_out, pack_out=self.pack_out)

    def pack(self):
        win = None if self.full_block else self.sched_out[0]
        return pack_ragged(self.anchor, self.draft_out[0], win, self.tiers, self.M_cap,
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
        return verify(self.target_packed, self.pack_out["cu_seqlens"], self.anchor, d[0], d[1],
                      d[2], i["U"], i["W1"], self.W2p, r=self.r, mode=self.verify_mode,
                      win_len=self.sched_out[0], seed=self.seed, step=self.step,
                      req_ids=i["req_ids"], out=self.verify_out, ws=self.ws_verify)

    def observe_step(self):
        """Add the current step's outputs to ``obs_block``."""
        v = self.verify_out
        observe(self.conf_out[0], self.conf_out[1], self.sched_out[0], v["accept_len"],
                v["ceiling_len"], self.pack_out["cu_seqlens"], self.obs_block, n_bins=self.n_bins)

    def analytic_step(self):
        """c* of the current step's verified slots into ``cstar``."""
        i, d = self.inp, self.draft_out
        return analytic_accept(self.target_packed, self.pack_out["cu_seqlens"], self.anchor, d[0],
                               d[2], i["U"], i["W1"], self.W2p, r=self.r, out=self.cstar,
                               ws=self.ws_accept)

    def _extras(self):
        if self.analytic:
            self.analytic_step()
        if self.obs_block is not None:
            self.observe_step()

    def observe_summary(self) -> Dict[str, object]:
        """Host copy of ``obs_block``, split and summarised (synchronises)."""
        return parse_observe(self.obs_block.cpu().numpy(), self.R, self.gamma, self.n_bins)

    def run(self, gather: bool = True):
        """One whole step; ``gather`` re-runs the target stand-in between pack
        and verify (needed whenever the windows may have changed)."""
        self.draft_confidence()
        self.schedule_and_pack()
        if gather:
            self.gather_target()
        self.verify()
        self._extras()

    def results(self) -> Dict[str, "object"]:
        """Host copies of every stage output (synchronises)."""
        d, c, s = self.draft_out, self.conf_out, self.sched_out
        out = {"tokens": d[0], "p_draft": d[1], "lse_draft": d[2], "conf": c[0], "surv": c[1],
               "win_len": s[0], "K": s[1], **self.pack_out, **self.verify_out}
        if self.analytic:
            out["cstar"] = self.cstar
        if self.logit_out is not None:
            out["logit"] = self.logit_out
        return {k: v.cpu().numpy() for k, v in out.items()}

    # -- decode loop -------------------------------------------------------
    def _decode_step(self, budget, mode: int):
        """One step of the loop, every launch on the current stream: the draft
        and verify read the Philox step from ``step_dev``; dspark_advance then
        moves x_0, the step and the survival history on."""
        i, d = self.inp, self.draft_out
        self.draft_confidence(step_dev=self.step_dev)
        self.schedule_and_pack(mode=mode, budget=budget)
        if not self.full_block:
            self.gather_target()
        verify(self.target_packed, self.pack_out["cu_seqlens"], self.anchor, d[0], d[1], d[2],
               i["U"], i["W1"], self.W2p, r=self.r, mode=self.verify_mode,
               win_len=self.sched_out[0], seed=self.seed, step_dev=self.step_dev,
               req_ids=i["req_ids"], out=self.verify_out, ws=self.ws_verify)
        self._extras()
        v = self.verify_out
        advance(self.anchor, v["accept_len"], v["out_tokens"], step_dev=self.step_dev,
                surv_hist=self.surv_hist,
                surv=self.conf_out[1] if self.surv_hist is not None else None)

    def reset(self, anchor=None, step: Optional[int] = None):
        """Put x_0 (default: the inputs' anchors) and the Philox step (default:
        the constructor's) back, and forget the survival history and graph."""
        self.anchor.copy_(self.inp["anchor"] if anchor is None else anchor)
        self.step_dev.fill_(self.step if step is None else int(step))
        self.surv_hist = None
        self._graph = None
        self._hist_steps = 0
        self._lag = None

    def save_state(self):
        """Device copies of the loop state (x_0, Philox step, survival history)."""
        return {"anchor": self.anchor.clone(), "step": self.step_dev.clone(),
                "hist": None if self.surv_hist is None else self.surv_hist.clone(),
                "hist_steps": self._hist_steps, "lag": self._lag}

    def load_state(self, st):
        """Restore a save_state() snapshot in place (a captured graph stays valid)."""
        if st["lag"] != self._lag:
            raise ValueError("the snapshot was taken with another history depth")
        self.anchor.copy_(st["anchor"])
        self.step_dev.copy_(st["step"])
        if st["hist"] is not None:
            self.surv_hist.copy_(st["hist"])
        self._hist_steps = st["hist_steps"]

    def decode(self, steps: int, *, lag: int = 2, graph: bool = False, record: bool = False):
        """Run ``steps`` decode steps from the current state.

        Step t sizes its budget from the survivals of step t - lag (lag 0: its
        own). The first ``lag`` steps have no survivals that old and, when the
        mode is ARGMAX, run the greedy scheduler with its early stop instead.
        graph=True captures the first step that uses the history into a HIP
        graph and replays it for every later step (eager steps before it load
        every kernel). record=True returns, per step, device copies of its
        x_0, Philox step, budget array and every output (taken between steps,
        outside any graph); otherwise returns None."""
        torch = self.t
        R, g = self.R, self.gamma
        if lag < 0 or lag > 8:
            raise ValueError("lag must be in [0, 8]")
        if lag != self._lag:   # new history depth: new buffers, new graph
            self.surv_hist = (torch.zeros((lag, R, g), dtype=torch.float32, device=self.anchor.device)
                              if lag > 0 else None)
            self._graph = None
            self._hist_steps = 0
            self._lag = lag
        log = [] if record else None
        for _ in range(steps):
            steady = self._hist_steps >= lag
            budget = self.surv_hist[lag - 1] if (lag > 0 and steady) else None
            mode = self.sched_mode
            if not steady and mode == SCHED_ARGMAX:
                mode = SCHED_GREEDY
            if record:
                snap = {"anchor": self.anchor.clone(), "step": self.step_dev.clone(),
                        "surv_budget": None if budget is None else budget.clone(),
                        "sched_mode": mode}
            if graph and steady and self._graph is not None:
                self._graph.replay()
            elif graph and steady and self._warm:
                self._graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(self._graph):
                    self._decode_step(budget, mode)
                self._graph.replay()
            else:
                self._decode_step(budget, mode)
                self._warm = True
            self._hist_steps = min(self._hist_steps + 1, lag)
            if record:
                d, c, s, v = self.draft_out, self.conf_out, self.sched_out, self.verify_out
                snap.update({"tokens": d[0].clone(), "p_draft": d[1].clone(),
                             "lse_draft": d[2].clone(), "conf": c[0].clone(), "surv": c[1].clone(),
                             "win_len": s[0].clone(), "K": s[1].clone(),
                             **{k: t.clone() for k, t in self.pack_out.items()},
                             **{k: t.clone() for k, t in v.items() if t is not None}})
                if self.analytic:
                    snap["cstar"] = self.cstar.clone()
                if self.logit_out is not None:
                    snap["logit"] = self.logit_out.clone()
                log.append(snap)
        if not record:
            return None
        return [{k: (x.cpu().numpy() if hasattr(x, "cpu") else x) for k, x in e.items()}
                for e in log]
