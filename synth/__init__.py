"""Seeded synthetic inputs for the DSpark draft-head-and-verify chain.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``draft_verify_sampling_markov_amd``). It holds input recipes only: shapes,
seeded random draws, host-side dtype rounding and raw (unprocessed) step-time
profiles. None of the method's arithmetic lives here -- no softmax, sampling,
survival product, scheduling, packing or verification.

Workload shapes follow the pages' two target families (a dense Qwen3-class model
with a 151936-entry vocabulary and a sparse DeepSeek-V4-class model with a
129280-entry vocabulary; the SGLang DSpark blog, opening section) and the
drafter's block sizes (gamma = 7 in the DSpark paper digest, "Benchmark";
gamma = 5 for the production drafter, "Infra"). The pages' mixed gsm8k /
arena-hard / poetry traffic (SGLang blog, "Per-request differentiation on mixed
traffic") is stood in for by three request classes with different draft noise.
No dataset item is used or reproduced.

Every array is drawn from its own child stream of ``numpy.random.SeedSequence``
(PCG64), so adding an array never shifts another.
"""
from __future__ import annotations

import dataclasses
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Spec", "CONFIGS", "CONFIG_ORDER", "generate", "to_bf16_bits",
    "bf16_bits_to_f32", "small_spec", "m_max",
]


@dataclass(frozen=True)
class Spec:
    """One synthetic workload.

    name        -- workload name
    R, gamma    -- requests, draft block length (slots k = 1..gamma)
    V, r, d     -- vocabulary, Markov rank, drafter hidden size
    dtype       -- "f32" or "bf16": storage type of U, target, W1, W2, h
    target_std  -- std of the i.i.d. normal part of the target logits
    zipf_s      -- exponent of the per-row Zipf log-pmf bias (None: no bias)
    noise       -- draft-vs-target logit noise:
                   ("const", s) | ("class", (s0, s1, s2)) by r mod 3 |
                   ("slot", a, b): std a + b*k for slot k = 1..gamma
    W_std       -- std of the Markov factors W1, W2
    w_std       -- std of the confidence-head weight (None: 1/sqrt(d+r))
    b           -- confidence-head bias
    cost        -- raw step-time profile recipe:
                   ("linear_sps", s0_milli, s1_milli): SPS*1000 = s0 - s1*M
                   ("linear_T", t0, t1): T(M) = t0 + t1*M seconds
                   ("stair_T", t0, t1, rel_noise): T(M) = (t0 + t1*M)*(1+eps),
                       eps ~ U(-rel_noise, rel_noise); the consumer rounds it
                       to capture tiers
    staircase   -- whether the cost table is rounded up to capture tiers
    tiers       -- ascending captured pack totals
    budgets     -- caps B on the number of selected draft slots
    modes       -- verify modes exercised on this workload
    seed        -- data seed (PCG64)
    """

    name: str
    R: int
    gamma: int
    V: int
    r: int
    d: int
    dtype: str
    target_std: float
    zipf_s: Optional[float]
    noise: Tuple
    W_std: float = 0.02
    w_std: Optional[float] = None
    b: float = 1.5
    cost: Tuple = ("linear_T", 5e-3, 8e-6)
    staircase: bool = False
    tiers: Tuple[int, ...] = ()
    budgets: Tuple[int, ...] = ()
    modes: Tuple[str, ...] = ("static",)
    seed: int = 1000

    @property
    def M_max(self) -> int:
        return m_max(self.R, self.gamma)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


def m_max(R: int, gamma: int) -> int:
    """Largest verify-forward size: every request verifies its whole block plus
    its anchor row (the vLLM adaptive-verification page, "Configuration &
    reproduction": capture size (num_speculative_tokens + 1) * max_num_seq)."""
    return R * (gamma + 1)


_STAIR_DS = (64, 128, 256, 512, 1024, 1536)

CONFIGS: Dict[str, Spec] = {
    "tiny": Spec(
        name="tiny", R=4, gamma=7, V=1024, r=32, d=64, dtype="f32",
        target_std=2.0, zipf_s=None, noise=("const", 0.5),
        W_std=0.02, w_std=0.1, b=0.0,
        cost=("linear_sps", 1_000_000, 20_000), staircase=False,
        tiers=(8, 16, 32), budgets=(12,),
        modes=("static", "compact", "cap_accept"), seed=1000),
    "qwen3": Spec(
        name="qwen3", R=64, gamma=7, V=151936, r=256, d=2560, dtype="bf16",
        target_std=3.0, zipf_s=1.1, noise=("const", 0.7),
        cost=("linear_T", 5e-3, 8e-6), staircase=False,
        tiers=(64, 128, 256, 512), budgets=(64 * 7,),
        modes=("static", "compact"), seed=1001),
    "dsv4": Spec(
        name="dsv4", R=256, gamma=5, V=129280, r=256, d=4096, dtype="bf16",
        target_std=3.0, zipf_s=1.1, noise=("const", 1.0),
        cost=("stair_T", 6e-3, 4e-6, 0.005), staircase=True,
        tiers=_STAIR_DS, budgets=(256 * 5,),
        modes=("compact",), seed=1002),
    "mixed": Spec(
        name="mixed", R=256, gamma=7, V=151936, r=256, d=2560, dtype="bf16",
        target_std=3.0, zipf_s=1.1, noise=("class", (0.3, 0.8, 1.5)),
        cost=("stair_T", 6e-3, 4e-6, 0.005), staircase=True,
        tiers=_STAIR_DS + (2048,), budgets=(256 * 7,),
        modes=("cap_accept", "compact"), seed=1003),
    "long": Spec(
        name="long", R=128, gamma=15, V=151936, r=256, d=4096, dtype="bf16",
        target_std=3.0, zipf_s=1.1, noise=("slot", 0.4, 0.1),
        cost=("stair_T", 6e-3, 4e-6, 0.005), staircase=True,
        tiers=(128, 256, 512, 1024, 1536, 2048),
        budgets=(128, 256, 512, 1024, 1920),
        modes=("compact",), seed=1004),
}
CONFIG_ORDER: List[str] = ["tiny", "qwen3", "dsv4", "mixed", "long"]


def small_spec(name: str = "small", *, R: int = 20, gamma: int = 5, V: int = 3000,
               r: int = 64, d: int = 96, dtype: str = "bf16", seed: int = 77,
               noise: Tuple = ("class", (0.3, 0.8, 1.5)), zipf_s: Optional[float] = 1.1,
               target_std: float = 3.0, W_std: float = 0.02, b: float = 1.5,
               tiers: Optional[Tuple[int, ...]] = None,
               cost: Tuple = ("stair_T", 2e-3, 40e-6, 0.005), staircase: bool = True,
               budgets: Optional[Tuple[int, ...]] = None) -> Spec:
    """A workload small enough for the oracle to finish in seconds that still
    spans several 16-request blocks, several 64-entry vocabulary tiles and a
    ragged tail in both (defaults: R = 20, V = 3000)."""
    mm = m_max(R, gamma)
    if tiers is None:
        t, tiers_l = 8, []
        while t < mm:
            tiers_l.append(t)
            t *= 2
        tiers_l.append(mm)
        tiers = tuple(tiers_l)
    if budgets is None:
        budgets = (R * gamma,)
    return Spec(name=name, R=R, gamma=gamma, V=V, r=r, d=d, dtype=dtype,
                target_std=target_std, zipf_s=zipf_s, noise=noise, W_std=W_std,
                b=b, cost=cost, staircase=staircase, tiers=tiers, budgets=budgets,
                modes=("static", "compact", "cap_accept"), seed=seed)


# --------------------------------------------------------------------------
# dtype helpers (storage conversion only)
# --------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns the 16-bit
    patterns as uint16. Inputs here are finite normals (no NaN handling).
    Uses torch's CPU conversion (the same rounding, multi-threaded) when torch
    is importable, else the bit-level definition below."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        return _to_bf16_bits_np(x)


def _to_bf16_bits_np(x: np.ndarray) -> np.ndarray:
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------

_STREAMS = ("anchor", "W1", "W2", "target", "zipf", "noise", "h", "w", "cost")


_CHUNK = 1 << 20          # elements per independently seeded chunk
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _rows_per_chunk(shape) -> Tuple[int, int]:
    rows = int(shape[0])
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    return rows, max(1, _CHUNK // max(1, inner))


def _normal(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    """N(0, std^2) float32 of `shape`, drawn in fixed row chunks along axis 0,
    chunk i from child stream i of `ss` (so the result does not depend on the
    number of threads)."""
    out = np.empty(shape, dtype=np.float32)
    rows, per = _rows_per_chunk(shape)
    starts = list(range(0, rows, per))
    kids = ss.spawn(len(starts))

    def fill(i):
        s0 = starts[i]
        s1 = min(rows, s0 + per)
        g = np.random.default_rng(kids[i])
        g.standard_normal(size=out[s0:s1].shape, dtype=np.float32, out=out[s0:s1])
        if std != 1.0:
            out[s0:s1] *= np.float32(std)

    list(_pool().map(fill, range(len(starts))))
    return out


def _noise_std(spec: Spec) -> np.ndarray:
    """[R, gamma] std of the draft-vs-target noise for (request, slot)."""
    kind = spec.noise[0]
    R, g = spec.R, spec.gamma
    if kind == "const":
        return np.full((R, g), spec.noise[1], dtype=np.float32)
    if kind == "class":
        stds = np.asarray(spec.noise[1], dtype=np.float32)
        return np.repeat(stds[np.arange(R) % len(stds)][:, None], g, axis=1)
    if kind == "slot":
        a, b = spec.noise[1], spec.noise[2]
        ks = np.arange(1, g + 1, dtype=np.float64)
        return np.broadcast_to((a + b * ks).astype(np.float32), (R, g)).copy()
    raise ValueError(f"unknown noise kind {kind!r}")


def raw_step_time(spec: Spec, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Raw (unprocessed) step-time profile T(M) in seconds for M = 0..M_max, as a
    start-up profiler would record it; monotone enforcement and tier rounding
    are the consumer's job."""
    M = np.arange(spec.M_max + 1, dtype=np.float64)
    kind = spec.cost[0]
    if kind == "linear_sps":
        s0, s1 = spec.cost[1], spec.cost[2]
        sps_milli = s0 - s1 * M
        if np.any(sps_milli <= 0):
            raise ValueError("linear SPS table reaches zero inside [0, M_max]")
        return 1000.0 / sps_milli
    if kind == "linear_T":
        return spec.cost[1] + spec.cost[2] * M
    if kind == "stair_T":
        t0, t1, rel = spec.cost[1], spec.cost[2], spec.cost[3]
        if rng is None:
            rng = np.random.default_rng(np.random.SeedSequence(spec.seed).spawn(len(_STREAMS))[8])
        eps = rng.uniform(-rel, rel, size=M.shape)
        return (t0 + t1 * M) * (1.0 + eps)
    raise ValueError(f"unknown cost kind {kind!r}")


def generate(spec: Spec, *, with_h: bool = True) -> Dict[str, np.ndarray]:
    """Draw every input of one chain step for ``spec``.

    Returns a dict of numpy arrays:
      anchor  int32   [R]            last committed token x_0 of each request
      W1      store   [V, r]         Markov lookup factor
      W2      store   [r, V]         Markov projection factor
      target  store   [R, gamma+1, V] target logits; row j is the target's
                                     distribution for slot j+1 (row gamma: bonus)
      U       store   [R, gamma, V]  drafter base logits for slots 1..gamma
                                     (= target rows 0..gamma-1 + noise)
      h       store   [R, gamma, d]  drafter hidden states
      w       float32 [d + r]        confidence-head weight (h part first)
      b       float32 scalar         confidence-head bias
      raw_T   float64 [M_max+1]      raw step-time profile (seconds)
      req_ids uint32  [R]            request ids 0..R-1
    "store" is float32 for dtype f32 and uint16 bfloat16 bit patterns for bf16.
    """
    R, g, V, r, d = spec.R, spec.gamma, spec.V, spec.r, spec.d
    ss = dict(zip(_STREAMS, np.random.SeedSequence(spec.seed).spawn(len(_STREAMS))))

    out: Dict[str, np.ndarray] = {}
    out["anchor"] = np.random.default_rng(ss["anchor"]).integers(0, V, size=R, dtype=np.int64).astype(np.int32)
    out["W1"] = _store(_normal(ss["W1"], (V, r), spec.W_std), spec.dtype)
    out["W2"] = _store(_normal(ss["W2"], (r, V), spec.W_std), spec.dtype)

    target = _normal(ss["target"], (R, g + 1, V), spec.target_std)
    rows = target.reshape(R * (g + 1), V)
    if spec.zipf_s is not None:
        # Zipf(s) log-pmf over a per-row random ranking of the vocabulary:
        # the token ranked i (0-based) gets -s * ln(1 + i).
        table = (-spec.zipf_s * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
        base = np.arange(V, dtype=np.int32)
        per = 8
        starts = list(range(0, rows.shape[0], per))
        kids = ss["zipf"].spawn(len(starts))

        def add_bias(i):
            s0 = starts[i]
            s1 = min(rows.shape[0], s0 + per)
            ranks = np.random.default_rng(kids[i]).permuted(np.broadcast_to(base, (s1 - s0, V)), axis=1)
            rows[s0:s1] += table[ranks]

        list(_pool().map(add_bias, range(len(starts))))
    U = _normal(ss["noise"], (R, g, V), 1.0)
    std = _noise_std(spec)

    def add_target(i):
        U[i] *= std[i][:, None]
        U[i] += target[i, :g, :]

    list(_pool().map(add_target, range(R)))
    out["target"] = _store(target, spec.dtype)
    del target, rows
    out["U"] = _store(U, spec.dtype)
    del U
    if with_h:
        out["h"] = _store(_normal(ss["h"], (R, g, d), 1.0), spec.dtype)
    w_std = spec.w_std if spec.w_std is not None else float(1.0 / np.sqrt(d + r))
    out["w"] = _normal(ss["w"], (d + r,), w_std)
    out["b"] = np.float32(spec.b)
    out["raw_T"] = raw_step_time(spec, np.random.default_rng(ss["cost"]))
    out["req_ids"] = np.arange(R, dtype=np.uint32)
    return out
