#!/usr/bin/env python3
"""Throughput of the DSpark draft-head-and-verify chain on one MI355X.

One step = one pass of the whole chain over one batch: Markov draft (gamma
slots), confidence + survival, global top-B schedule, ragged pack, and
rejection-sampling verify, all on the GPU with inputs resident in HBM. The
target forward that sits between pack and verify in a serving engine is not
part of the chain; its output (the packed target logits) is prepared once
before timing -- every timed step processes the same batch, so the schedule
and pack are the same each step, and this is checked after timing.

The headline workload is the largest one: mixed traffic (R = 256, gamma = 7,
V = 151936) in cap-accept verify, every block verified whole (1792 verified
draft slots per step). Prints one JSON line: the metric (verified draft
slots per second over exactly --steps steps), per-step statistics over
individually timed steps (median, p10, p90; warm and after a 512 MiB cache
flush), the roofline of the dominant kernel (the per-slot bias GEMM +
softmax-partials pass, timed with HIP events on the chain's stream) with its
algorithmic bytes counting W2 once per block, the verify stage against the
bytes of its two passes, the same figures for the other named workloads
(without the stage timings), the bandwidth and matrix rate this GPU reaches (two probe
kernels of the library), and the CPU oracle timed on a bounded sample of the
headline workload on this host.

Each timed region follows W untimed steps (default 200, about 0.1 s): on
MI355X the step time drifts by about 5% over the first few dozen steps of
sustained load before it settles, and a serving loop runs at the settled
rate.

    python bench.py [--steps K] [--warmup W] [--config mixed] [--mode cap_accept]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft slots/s (draft+schedule+verify chain) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16, published
MFMA_F32_PEAK_TFS = 157.3


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev(arr):
    import numpy as np
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    if arr.dtype == np.uint32:
        return torch.from_numpy(arr.view(np.int32)).cuda()
    return torch.from_numpy(arr).cuda()


PMC_SOURCES = ("draft_verify_sampling_markov_amd/csrc/markov.hip",
               "draft_verify_sampling_markov_amd/csrc/tile_engine.hpp",
               "draft_verify_sampling_markov_amd/csrc/dspark_device.hpp")


def _pmc_fields(config_name: str):
    """The key: value lines of the committed counter summary of the draft GEMM
    kernel for this workload, or None (no summary, or sources changed since)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"markov_partials_{config_name}_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith(("|", "#", " ", "-")):
            k, v = ln.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in PMC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return fields


def measured_traffic(config_name: str):
    """HBM bytes per launch of the draft GEMM kernel from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a 256 MiB copy), or
    None when no summary exists for this workload or the kernel's sources have
    changed since the counters were taken."""
    f = _pmc_fields(config_name)
    if f is None or "traffic_bytes_per_launch" not in f:
        return None
    return int(f["traffic_bytes_per_launch"])


def measured_mfma_busy(config_name: str):
    """Matrix-core busy fraction of the draft GEMM kernel from the same counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES over the kernel's SIMD cycles), or None."""
    f = _pmc_fields(config_name)
    if f is None or "mfma_busy_frac" not in f:
        return None
    return float(f["mfma_busy_frac"])


def cpu_baseline(spec, inp, mode_name: str, n_req: int = 8, runs: int = 3, target_s: float = 3.5):
    """The oracle as it stands, on the first n requests of the workload: one
    sizing step on n_req requests, n scaled so that a step takes about
    target_s seconds (at most R), then `runs` timed chain steps, the median
    reported (about 10 s of CPU work in all)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    vmode = {"static": oracle.VERIFY_STATIC, "compact": oracle.VERIFY_COMPACT,
             "cap_accept": oracle.VERIFY_CAP_ACCEPT}[mode_name]

    def step(n):
        sub = {k: inp[k][:n] for k in ("U", "target", "h", "anchor", "req_ids")}
        sub.update({k: inp[k] for k in ("W1", "W2", "w", "b", "raw_T")})
        t0 = time.perf_counter()
        out = oracle.chain(sub, tiers=spec.tiers, staircase=spec.staircase,
                           B_cap=min(spec.budgets[0], n * spec.gamma), verify_mode=vmode)
        dt = time.perf_counter() - t0
        return dt, (n * spec.gamma if vmode != oracle.VERIFY_COMPACT else int(out["sched"]["K"]))

    n = min(n_req, spec.R)
    t_size, _ = step(n)
    n = int(min(spec.R, max(n, round(n * target_s / max(t_size, 1e-3)))))
    times, slots = [], 0
    for _ in range(runs):
        dt, slots = step(n)
        times.append(dt)
    dt = float(np.median(times))
    return {"value": slots / dt, "unit": "slots/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {spec.R} requests of the {spec.name} workload, full "
                      f"vocabulary V={spec.V}, {mode_name} verify; median of {runs} oracle chain "
                      f"steps ({', '.join(f'{t:.1f}' for t in times)} s; float64 numpy, "
                      f"{cores} cores in the affinity mask, BLAS threads={blas})"}


def measure_decode(dv, dev, inp, spec, B_cap: int, steps: int, lag: int):
    """The decode loop in compact mode: each step drafts from the token the
    previous one committed, sizes its budget from the survivals of `lag` steps
    before, and verifies the scheduled windows. Its target stand-in (a gather
    of the windows' target rows, which a serving engine's target forward would
    write) runs inside every step and is timed on its own as well. Times
    `steps` steps run eagerly and as replays of one captured graph, from the
    same state, and counts the tokens they commit with a recorded rerun."""
    import numpy as np
    import torch
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=B_cap,
                  verify_mode=dv.VERIFY_COMPACT, seed=1, step=1000)
    ch.decode(lag + 3, lag=lag)                      # fills the history, loads every kernel
    ch.decode(1, lag=lag, graph=True)                # captures the steady-state step
    torch.cuda.synchronize()
    st = ch.save_state()
    out = {"lag": lag, "steps": steps, "verify": "compact"}
    for name, graph in (("eager", False), ("graph", True)):
        ch.load_state(st)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ch.decode(steps, lag=lag, graph=graph)
        torch.cuda.synchronize()
        out[f"{name}_ms_per_step"] = round((time.perf_counter() - t0) * 1e3 / steps, 4)
    ch.load_state(st)
    rec = ch.decode(steps, lag=lag, record=True)
    torch.cuda.synchronize()
    committed = float(np.mean([r["n_out"].sum() for r in rec]))
    slots = float(np.mean([int(r["K"][0]) for r in rec]))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        ch.gather_target()
    ev[1].record()
    torch.cuda.synchronize()
    out["target_standin_ms"] = round(ev[0].elapsed_time(ev[1]) / steps, 4)
    out["committed_tokens_per_step"] = round(committed, 2)
    out["verified_slots_per_step"] = round(slots, 1)
    out["committed_tokens_per_s_graph"] = round(committed / (out["graph_ms_per_step"] * 1e-3), 1)
    log(f"[bench] decode loop: eager {out['eager_ms_per_step']} ms/step, graph "
        f"{out['graph_ms_per_step']} ms/step (target stand-in {out['target_standin_ms']} ms), "
        f"{committed:.1f} tokens and {slots:.0f} verified slots per step")
    return out


def measure_observability(dv, dev, inp, spec, B_cap: int, steps: int):
    """The two observability calls on a cap-accept step of the workload (the
    mode that verifies the whole block while committing the window): the
    accumulator (dspark_observe) and the analytic acceptance pass
    (dspark_analytic_accept), each timed with HIP events over `steps` calls on
    the chain's stream. The analytic pass's algorithmic bytes are the packed
    target rows once for their log-sum-exps, then the U row and target row of
    every verified slot, and W2 once per group of rows the GEMM engine holds.
    Then 32 decode steps of the same chain give a calibration set (the head's
    logits, soft labels prod c*) for one timed sequential-temperature fit
    (dspark_sts_fit) over a grid of 31 inverse temperatures."""
    import numpy as np
    import torch
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=B_cap,
                  verify_mode=dv.VERIFY_CAP_ACCEPT, observe_bins=16, analytic=True,
                  keep_logits=True)
    ch.run(gather=False)
    torch.cuda.synchronize()
    res = ch.results()
    out = {"mode": "cap_accept", "calls": steps}
    for name, fn in (("analytic", ch.analytic_step), ("observe", ch.observe_step)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        out[f"{name}_us"] = round(ev[0].elapsed_time(ev[1]) * 1e3 / steps, 2)
    b = 2 if spec.dtype == "bf16" else 4
    R, g, V, r = spec.R, spec.gamma, spec.V, spec.r
    M = int(res["totals"][0])
    verified = int(np.isfinite(res["cstar"]).sum())
    groups = -(-(R * (g + 1)) // (256 if spec.dtype == "bf16" else 128))
    nbytes = M * V * b + 2 * verified * V * b + groups * r * V * b
    out["analytic_bytes"] = nbytes
    out["analytic_gbs"] = round(nbytes / (out["analytic_us"] * 1e-6) / 1e9, 1)
    summ = ch.observe_summary()
    out["mean_cstar"] = round(float(np.nanmean(res["cstar"])), 4)
    out["mean_conf"] = round(float(res["conf"].mean()), 4)
    out["utilisation"] = round(summ["utilisation"], 4)
    out["ece_conditional"] = round(summ["ece_conditional"], 4)
    log(f"[bench] observability: analytic c* pass {out['analytic_us']} us "
        f"({out['analytic_gbs']} GB/s), accumulator {out['observe_us']} us")

    # sequential temperature scaling on a calibration set from the decode
    # loop: the head's logits against soft labels prod c* (analytic acceptance)
    rec = ch.decode(32, lag=2, record=True)
    torch.cuda.synchronize()
    z = torch.from_numpy(np.concatenate([r_["logit"] for r_ in rec])).cuda()
    y = torch.from_numpy(np.cumprod(np.concatenate([r_["cstar"] for r_ in rec]), axis=1)
                         .astype(np.float32)).cuda()
    betas_l = sorted({float(np.float32(0.25 * 1.1 ** i)) for i in range(30)} | {1.0})
    betas = torch.tensor(betas_l, dtype=torch.float32, device="cuda")
    dv.sts_fit(z, y, betas)                            # loads the kernels
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    inv, ece = dv.sts_fit(z, y, betas)
    ev[1].record()
    torch.cuda.synchronize()
    inv_l, ece_np = inv.cpu().numpy(), ece.cpu().numpy()
    j1 = betas_l.index(1.0)
    picked = [betas_l.index(float(b_)) for b_ in inv_l]
    out["sts"] = {"samples": int(z.shape[0]), "grid": len(betas_l), "fit_us": round(ev[0].elapsed_time(ev[1]) * 1e3, 1),
                  "inv_temp": [round(float(b_), 4) for b_ in inv_l],
                  "ece_beta1": [round(float(ece_np[k, j1]), 4) for k in range(spec.gamma)],
                  "ece_fit": [round(float(ece_np[k, picked[k]]), 4) for k in range(spec.gamma)],
                  "labels": "soft: prod of analytic acceptance c* over the prefix"}
    log(f"[bench] temperature fit over {out['sts']['samples']} samples x {len(betas_l)} candidates: "
        f"{out['sts']['fit_us']} us; prefix ECE {out['sts']['ece_beta1']} -> {out['sts']['ece_fit']}")
    return out


def measure_shards(dv, dev, spec, G: int, reps: int):
    """One rank's draft kernels at the vocabulary-shard shape V/G (rank 0 of
    G; same R, r and gamma): per slot the GEMM pass over the rank's columns,
    the per-request summary, and the shard select, after one full sharded
    draft has laid out every rank's summaries. Each is timed by replaying a
    captured graph of the gamma slots (`reps` replays, HIP events around
    them), so the figures are GPU time, not the host's launch rate: one graph
    holds the whole per-rank slot (GEMM + summary + select), one the summaries
    alone and one the selects alone; the GEMM figure is the difference. The
    collectives between them (an all-gather of G x R x 8 bytes and an
    all-reduce of R ids and probabilities per slot) are not measured."""
    import torch
    sd = dv.ShardedDraft(dev["U"], dev["W1"], dev["W2"], G)
    sd.draft(dev["anchor"], seed=3, step=5, req_ids=dev["req_ids"])
    torch.cuda.synchronize()
    tf = sd.out[0].view(-1)
    Vg = sd.bounds[1] - sd.bounds[0]

    def slots(phases):
        for k in range(1, spec.gamma + 1):
            x_prev, xs = (dev["anchor"], 1) if k == 1 else (tf[k - 2:], spec.gamma)
            for ph in phases:
                if ph == "gemm":
                    Uk = dev["U"].view(-1)[(k - 1) * spec.V:]
                    dv.markov_shard_partials(Uk, spec.gamma * spec.V, dev["W1"], sd.W2p[0], x_prev,
                                             xs, R=spec.R, V_g=Vg, V=spec.V, r=spec.r,
                                             part=sd.ws[0])
                elif ph == "summary":
                    dv.markov_shard_summary(sd.ws[0], R=spec.R, V_g=Vg, out=sd.summaries[0])
                else:
                    sd.rank_slot(0, k, x_prev, xs, seed=3, step=5, req_ids=dev["req_ids"],
                                 phase="select")

    def timed(phases):
        slots(phases)                     # eager once: loads every kernel
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            slots(phases)
        g.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / (reps * spec.gamma)

    whole = timed(("gemm", "summary", "select"))
    summ = timed(("summary",))
    sel = timed(("select",))
    gemm = whole - summ - sel
    b = 2 if spec.dtype == "bf16" else 4
    n_t = -(-Vg // 64)
    nbytes = spec.R * Vg * b + spec.r * Vg * b + spec.R * spec.r * b + n_t * spec.R * 8
    out = {"G": G, "V_g": Vg, "rank": 0, "per_slot_us": round(whole, 2), "gemm_us": round(gemm, 2),
           "summary_us": round(summ, 2), "select_us": round(sel, 2), "gemm_bytes": nbytes,
           "gemm_gbs": round(nbytes / (gemm * 1e-6) / 1e9, 1),
           "draft_us_per_rank": round(whole * spec.gamma, 1)}
    log(f"[bench] {G}-way vocabulary shard (V_g={Vg}), graph-replayed: per slot {out['per_slot_us']} "
        f"us = GEMM {out['gemm_us']} ({out['gemm_gbs']} GB/s) + summary {out['summary_us']} + "
        f"select {out['select_us']}")
    return out


def _spec_bytes(spec):
    return 2 if spec.dtype == "bf16" else 4


def draft_algorithmic(spec):
    """The Markov draft's algorithmic work per step: U_k streamed for every
    slot, W2 once per block, the gathered W1 rows per slot (bytes); the bias
    GEMM's 2 R r V flops per slot."""
    b = _spec_bytes(spec)
    R, g, V, r = spec.R, spec.gamma, spec.V, spec.r
    return {"bytes": g * R * V * b + r * V * b + g * R * r * b, "flops": 2 * g * R * r * V}


def verify_algorithmic(spec, res):
    """The verify's algorithmic bytes for one step's results: pass 1 reads every
    verified packed row (M_v = the pack's total), pass 2 one target row per
    request, the U row of each request whose correction is a residual (accept
    length below its commit window) and W2 once."""
    import numpy as np
    b = _spec_bytes(spec)
    R, g, V, r = spec.R, spec.gamma, spec.V, spec.r
    M_v = int(res["totals"][0])
    commit = np.clip(res["win_len"], 0, g) if res.get("win_len") is not None else np.full(R, g)
    R_rej = int(np.sum(res["accept_len"] < commit))
    return {"pass1": M_v * V * b, "pass2": (R + R_rej) * V * b + r * V * b, "rows": M_v,
            "residual_requests": R_rej}


def _stats(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def measure_chain(dv, spec, mode_name: str, B_cap: int, *, steps: int, warmup: int, samples: int,
                  cold_samples: int, profile_steps: int, stages: bool = True,
                  resident_compare: bool = True):
    """One workload: the whole-chain step time (exactly `steps` steps, eager
    launches and replays of one captured graph; the faster counts), per-step
    statistics over `samples` individually timed replays (warm) and
    `cold_samples` replays each after a 512 MiB write that evicts the caches,
    per-stage event times, and the roofline of the dominant kernel."""
    import numpy as np
    import torch
    import synth
    mode = dv.VERIFY_MODES[mode_name]
    t0 = time.time()
    inp = synth.generate(spec)
    log(f"[bench] generated {spec.name} inputs in {time.time() - t0:.1f} s")
    dev = {k: to_dev(inp[k]) for k in ("U", "W1", "W2", "target", "h", "anchor", "w", "req_ids")}
    sps = dv.cost_table_prepare(inp["raw_T"], spec.tiers, spec.staircase)
    dev["sps_milli"] = to_dev(sps)
    ch = dv.Chain(dev, b=float(inp["b"]), tiers=spec.tiers, B_cap=B_cap, verify_mode=mode)

    # one step with the target stand-in, to lay out the packed target rows
    ch.run(gather=True)
    torch.cuda.synchronize()
    first = ch.results()
    if first["totals"][1] < 0:
        raise RuntimeError(f"packed total {first['totals'][0]} exceeds every tier")
    K_sel = int(first["K"][0])
    slots_per_step = spec.R * spec.gamma if mode != dv.VERIFY_COMPACT else K_sel

    for _ in range(warmup):
        ch.run(gather=False)
    torch.cuda.synchronize()

    # ---- timed region 1: exactly `steps` steps, eager launches ----
    t_e = time.perf_counter()
    for _ in range(steps):
        ch.run(gather=False)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t_e) * 1e3 / steps

    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        ch.run(gather=False)
    for _ in range(max(warmup, 1)):
        step_graph.replay()
    torch.cuda.synchronize()

    # ---- timed region 2: exactly `steps` steps, graph replays ----
    t_start = time.perf_counter()
    for _ in range(steps):
        step_graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t_start) * 1e3 / steps
    use_graph = graph_ms <= eager_ms
    ms_per_step = graph_ms if use_graph else eager_ms

    # per-step statistics: individually timed replays, warm and cache-cold
    def replay_times(n, flush=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (e0, e1) in enumerate(ev):
            if flush is not None:
                flush.fill_(i & 255)
            e0.record()
            step_graph.replay()
            e1.record()
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    warm = replay_times(samples)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = replay_times(cold_samples, flush)
    del flush
    after = ch.results()
    for key in ("win_len", "cu_seqlens", "totals", "tokens", "p_draft", "accept_len", "out_tokens"):
        if not np.array_equal(first[key], after[key]):
            raise RuntimeError(f"{key} changed between steps: the pre-laid target rows are stale")
    value = slots_per_step / (ms_per_step * 1e-3)
    log(f"[bench] {spec.name}/{mode_name}: {steps} steps, graph replays {graph_ms:.4f} ms/step, "
        f"eager {eager_ms:.4f} ms/step; warm median {np.median(warm):.4f}, cache-cold median "
        f"{np.median(cold):.4f} ms")
    out = {"value": round(value, 1), "ms_per_step": round(ms_per_step, 4),
           "graph_ms_per_step": round(graph_ms, 4), "eager_ms_per_step": round(eager_ms, 4),
           "step_timing": ("replays of one captured HIP graph of the whole step" if use_graph else
                           "eager launches of the whole step (faster than graph replays here)"),
           "step_ms": _stats(warm), "step_ms_cache_cold": _stats(cold),
           "cache_flush_bytes": 512 << 20,
           "slots_per_step": slots_per_step, "packed_total": int(first["totals"][0]),
           "tier": int(first["totals"][1]),
           "accepted_tokens_per_s": round(float(first["n_out"].sum()) / (ms_per_step * 1e-3), 1),
           "mean_accept_len": round(float(first["accept_len"].mean()), 3)}

    # ---- per-stage event timing on the chain's stream ----
    P = profile_steps
    g = spec.gamma
    if stages:
        stage_names = ["draft", "confidence", "schedule", "pack", "verify"]
        st_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stage_names) + 1)]
                 for _ in range(P)]
        for s in range(P):
            ev = st_ev[s]
            ev[0].record()
            ch.draft_split()
            ev[1].record()
            ch.confidence()
            ev[2].record()
            ch.schedule()
            ev[3].record()
            ch.pack()
            ev[4].record()
            ch.verify()
            ev[5].record()
        torch.cuda.synchronize()
        out["stages_ms"] = {n: round(float(np.mean([st_ev[s][i].elapsed_time(st_ev[s][i + 1])
                                                     for s in range(P)])), 4)
                            for i, n in enumerate(stage_names)}
        prof = ch.results()
        if not np.array_equal(prof["tokens"], first["tokens"]):
            raise RuntimeError("the per-slot draft differs from the draft call")
        # the verify stage against the algorithmic bytes of its two passes; the
        # stage's time includes its latency launches (decide, residual draw)
        va = verify_algorithmic(spec, dict(first, win_len=first["win_len"] if mode != dv.VERIFY_STATIC else None))
        v_us = out["stages_ms"]["verify"] * 1e3
        v_gbs = (va["pass1"] + va["pass2"]) / (v_us * 1e-6) / 1e9
        out["verify_roofline"] = {
            "bound": "hbm", "achieved": round(v_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(v_gbs / HBM_PEAK_GBS, 4), "stage_us": round(v_us, 2),
            "pass1_bytes": va["pass1"], "pass2_bytes": va["pass2"], "verified_rows": va["rows"],
            "residual_requests": va["residual_requests"],
            "note": "whole verify stage (row pass, accept test, residual pass, residual draw) "
                    "timed with events; bytes: every verified target row, then one target row "
                    "per request, the U row of each residual request and W2"}

    # ---- the draft call alone, per kernel choice (graph of one call) ----
    def draft_call_ms(reps):
        ch.draft_confidence()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            ch.draft_confidence()
        gr.replay()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(reps):
            gr.replay()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / reps

    alg = draft_algorithmic(spec)
    drafts = {"per_slot_ms": round(draft_call_ms(P), 4)}
    if resident_compare:
        prev = dv.set_draft_path(dv.DRAFT_RESIDENT)
        try:
            drafts["resident_ms"] = round(draft_call_ms(P), 4)
            drafts["resident_status"] = dv.draft_status(ch.ws_draft, spec.R, spec.V)
        finally:
            dv.set_draft_path(prev)
    for k_ in [k_ for k_ in drafts if k_.endswith("_ms")]:
        drafts[k_.replace("_ms", "_gbs")] = round(alg["bytes"] / (drafts[k_] * 1e-3) / 1e9, 1)
    drafts["algorithmic_bytes_per_step"] = alg["bytes"]
    drafts["note"] = ("whole draft call (gamma slots, draws, confidence head), graph-replayed; "
                      "GB/s = the draft's algorithmic bytes (W2 once per block) / call time")
    out["draft_call"] = drafts

    # ---- the dominant kernel: replays of a graph of 4 gamma GEMM launches
    # (slot k = 1..gamma in turn, its own U_k and previous tokens), each on a
    # workspace of its own whose tile-queue counters are put back to zero
    # between replays, outside the timed intervals (in the chain the select
    # does that) ----
    n_gemm = 4 * g
    wss = [dv.new_workspace(dv.CALL_MARKOV_DRAFT, spec.R, g, spec.V, spec.r, dev["U"].device)
           for _ in range(n_gemm)]
    Uf, tf = dev["U"].view(-1), ch.draft_out[0].view(-1)

    def gemm_launches():
        for j in range(n_gemm):
            k = 1 + j % g
            x_prev, xs = (ch.anchor, 1) if k == 1 else (tf[k - 2:], g)
            dv.markov_partials(Uf[(k - 1) * spec.V:], g * spec.V, dev["W1"], ch.W2p, x_prev, xs,
                               R=spec.R, V=spec.V, r=spec.r, part=wss[j])

    gemm_launches()
    gr = torch.cuda.CUDAGraph()
    for w_ in wss:
        dv.workspace_init(w_)
    with torch.cuda.graph(gr):
        gemm_launches()
    for _ in range(max(1, warmup // 4)):  # untimed, as the steps before a timed region
        for w_ in wss:
            dv.workspace_init(w_)
        gr.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(P)]
    for e0, e1 in ev:
        for w_ in wss:
            dv.workspace_init(w_)
        e0.record()
        gr.replay()
        e1.record()
    torch.cuda.synchronize()
    gemm_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / (P * n_gemm)
    del wss

    b = _spec_bytes(spec)
    R, V, r = spec.R, spec.V, spec.r
    bytes_per_launch = alg["bytes"] / g           # W2 once per block, spread over the gamma launches
    flops_per_launch = alg["flops"] / g
    achieved_gbs = bytes_per_launch / (gemm_ms * 1e-3) / 1e9
    achieved_tfs = flops_per_launch / (gemm_ms * 1e-3) / 1e12
    mfma_peak = MFMA_BF16_PEAK_TFS if spec.dtype == "bf16" else MFMA_F32_PEAK_TFS
    traffic = measured_traffic(f"{spec.name}_{mode_name}")
    busy = measured_mfma_busy(f"{spec.name}_{mode_name}")
    out["roofline"] = {
        "kernel": "markov_partials_kernel (per-slot bias GEMM + U add + softmax partials)",
        "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
        "traffic_over_algorithmic": None if traffic is None else round(traffic / bytes_per_launch, 3),
        "algorithmic_bytes_per_launch": int(round(bytes_per_launch)),
        "algorithmic_bytes": "gamma R V b + r V b + gamma R r b per step (U_k every slot, W2 once "
                             "per block, W1 rows every slot), divided over the gamma launches",
        "avg_launch_us": round(gemm_ms * 1e3, 2),
        "timing": "HIP events around replays of a graph of 4 gamma GEMM launches",
        "launches_timed": P * n_gemm,
        "mfma": {"achieved": round(achieved_tfs, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                 "frac": round(achieved_tfs / mfma_peak, 4), "flops_per_launch": int(flops_per_launch),
                 "busy_frac_counter": busy}}
    return out, inp, dev


def measure_peaks(dv):
    """What this GPU reaches, beside the published peaks the rooflines use:
    streaming reads of a 2 GiB buffer (eight times the Infinity Cache, so from
    HBM), re-reads of one 77.8 MB buffer (the size of a slot's U_k or of W2,
    which the Infinity Cache can hold; a launch this short also pays its
    ramp), and the bf16 matrix-core rate of a loop of independent 16x16x32
    products, 32 waves per CU. Each is the median of HIP-event
    timed launches on the current stream."""
    import numpy as np
    import torch
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    big = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    small = torch.ones(77_791_232, dtype=torch.uint8, device="cuda")
    for b in (big, small):
        dv.probe_read(b, sink)
    torch.cuda.synchronize()
    t_big = timed(lambda: dv.probe_read(big, sink), 9)
    t_small = timed(lambda: dv.probe_read(small, sink), 21)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid, iters = 8 * cus, 512
    flops = dv.probe_mfma(sink, grid=grid, iters=iters)
    torch.cuda.synchronize()
    t_mfma = timed(lambda: dv.probe_mfma(sink, grid=grid, iters=iters), 9)
    del big, small
    torch.cuda.empty_cache()
    out = {"hbm_read_GBs": round((2 << 30) / t_big / 1e9, 1),
           "reread_77MB_GBs": round(77_791_232 / t_small / 1e9, 1),
           "mfma_bf16_TFLOPs": round(flops / t_mfma / 1e12, 1),
           "published": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFS},
           "note": ("dspark_probe_read / dspark_probe_mfma: 16-byte nontemporal grid-stride "
                    "reads of 2 GiB, 4 workgroups of 512 threads per CU; 8 independent "
                    "v_mfma_f32_16x16x32_bf16 chains per wave, 32 waves per CU; medians of "
                    "event-timed launches; rooflines stay priced against the published peaks")}
    log(f"[bench] measured peaks: HBM read {out['hbm_read_GBs']} GB/s (2 GiB), re-read of 77.8 MB "
        f"{out['reread_77MB_GBs']} GB/s, bf16 MFMA {out['mfma_bf16_TFLOPs']} TFLOP/s")
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before each timed region; under sustained load the "
                         "GPU's step time settles after a few dozen steps")
    ap.add_argument("--config", default="mixed")
    ap.add_argument("--mode", default="cap_accept", choices=["static", "compact", "cap_accept"])
    ap.add_argument("--budget", type=int, default=None, help="cap B on selected slots")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--samples", type=int, default=50,
                    help="individually timed steps for the median / p10 / p90")
    ap.add_argument("--cold-samples", type=int, default=20,
                    help="individually timed steps, each after a 512 MiB cache-evicting write")
    ap.add_argument("--profile-steps", type=int, default=10,
                    help="steps of per-stage and per-kernel event timing")
    ap.add_argument("--other-configs", default="tiny:static,qwen3:static,dsv4:compact,long:compact",
                    help="workload:mode list measured after the headline ('' skips)")
    ap.add_argument("--decode-steps", type=int, default=20,
                    help="steps of the multi-step decode loop (compact verify, budget from "
                         "survivals --lag steps old) timed eagerly and as graph replays; 0 skips")
    ap.add_argument("--lag", type=int, default=2)
    ap.add_argument("--shards", type=int, default=0,
                    help="G > 1: also time one rank's draft kernels at the V/G vocabulary-shard "
                         "shape (off by default, so that a kernel trace of the default run holds "
                         "only the full-vocabulary GEMM launches)")
    ap.add_argument("--observe-calls", type=int, default=10,
                    help="timed calls of each observability pass on a cap-accept step; 0 skips")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the peak probes (streaming read, matrix-core loop)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one 256 MiB device-to-device copy (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the chain has no "
              f"multi-GPU path (its sharding is a design only).", file=sys.stderr)
        return 2

    import torch
    import synth
    import draft_verify_sampling_markov_amd as dv

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    dv.load_library()
    spec = synth.CONFIGS[args.config]
    B_cap = spec.budgets[0] if args.budget is None else args.budget
    try:
        head, inp, dev = measure_chain(dv, spec, args.mode, B_cap, steps=args.steps,
                                       warmup=args.warmup, samples=args.samples,
                                       cold_samples=args.cold_samples,
                                       profile_steps=args.profile_steps)
    except RuntimeError as e:
        log(f"[bench] {e}: failed workload")
        return 1
    R, g, V, r = spec.R, spec.gamma, spec.V, spec.r
    line = {
        "metric": METRIC, "value": head["value"], "unit": "slots/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "step_timing": head["step_timing"],
        "graph_ms_per_step": head["graph_ms_per_step"], "eager_ms_per_step": head["eager_ms_per_step"],
        "step_ms": head["step_ms"], "step_ms_cache_cold": head["step_ms_cache_cold"],
        "cache": ("value and step_ms: inputs resident and re-read every step (the 256 MB "
                  "Infinity Cache may hold part of them); step_ms_cache_cold: each step after a "
                  "512 MiB write"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": f"{spec.name}: R={R} gamma={g} V={V} r={r} d={spec.d} {spec.dtype}, "
                               f"{args.mode} verify, B={B_cap}",
                   "R": R, "gamma": g, "V": V, "r": r, "d": spec.d, "mode": args.mode,
                   "B_cap": B_cap, "verified_slots_per_step": head["slots_per_step"],
                   "packed_total": head["packed_total"], "tier": head["tier"]},
        "accepted_tokens_per_s": head["accepted_tokens_per_s"],
        "mean_accept_len": head["mean_accept_len"],
        "stages_ms": head.get("stages_ms"),
        "verify_roofline": head.get("verify_roofline"),
        "draft_call": head["draft_call"],
        "roofline": head["roofline"],
    }
    if args.decode_steps > 0:
        line["decode"] = measure_decode(dv, dev, inp, spec, B_cap, args.decode_steps, args.lag)
    if args.shards > 1:
        line["vocab_shards"] = measure_shards(dv, dev, spec, args.shards, 20)
    if args.observe_calls > 0:
        line["observability"] = measure_observability(dv, dev, inp, spec, B_cap, args.observe_calls)
    if not args.no_peaks:
        pk = measure_peaks(dv)
        line["peaks_measured"] = pk
        # the dominant kernel also against what this GPU reaches (reported beside frac)
        rl = line["roofline"]
        rl["frac_of_measured_peak"] = round(rl["achieved"] / pk["hbm_read_GBs"], 4)
        if spec.dtype == "bf16":   # the probe measures the bf16 matrix rate
            rl["mfma"]["frac_of_measured_peak"] = round(rl["mfma"]["achieved"] / pk["mfma_bf16_TFLOPs"], 4)
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(spec, inp, args.mode)
    del dev, inp
    torch.cuda.empty_cache()

    others = {}
    for item in [x for x in args.other_configs.split(",") if x]:
        name, mode_name = item.split(":")
        sp = synth.CONFIGS[name]
        try:
            o, _, _ = measure_chain(dv, sp, mode_name, sp.budgets[-1], steps=20, warmup=args.warmup,
                                    samples=20, cold_samples=5, profile_steps=5, stages=False)
        except RuntimeError as e:
            log(f"[bench] {name}/{mode_name}: {e}")
            continue
        rl = o["roofline"]
        others[f"{name}:{mode_name}"] = {
            "workload": f"{name}: R={sp.R} gamma={sp.gamma} V={sp.V} r={sp.r} {sp.dtype}, "
                        f"{mode_name} verify, B={sp.budgets[-1]}",
            "value": o["value"], "unit": "slots/s", "ms_per_step": o["ms_per_step"],
            "step_ms": o["step_ms"], "step_ms_cache_cold": o["step_ms_cache_cold"],
            "slots_per_step": o["slots_per_step"], "draft_call": o["draft_call"],
            "gemm_roofline": {k: rl[k] for k in ("achieved", "peak", "unit", "frac",
                                                 "avg_launch_us", "traffic",
                                                 "traffic_over_algorithmic")},
            "gemm_mfma_frac": rl["mfma"]["frac"]}
        torch.cuda.empty_cache()
    line["other_workloads"] = others
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
