"""Python binding of libdspark.so, the MI355X (gfx950) DSpark draft-head-and-verify chain.

Argument marshalling only: every step of the chain runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. The binding
raises if the library is missing -- there is no fallback path.

Calls (same names as the C ABI in include/dspark.h, without the prefix):
    prepack_w2, markov_draft, confidence, markov_draft_confidence, schedule_topb, pack_ragged,
    schedule_pack, verify, advance, observe, analytic_accept, sts_fit, cost_table_prepare,
    workspace_bytes, markov_logits
and ``Chain``, which holds preallocated buffers for repeated steps.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark.so")

F32, BF16 = 0, 1
VERIFY_STATIC, VERIFY_COMPACT, VERIFY_CAP_ACCEPT = 0, 1, 2
SCHED_ARGMAX, SCHED_GREEDY, SCHED_FIXED = 0, 1, 2
CALL_MARKOV_DRAFT, CALL_VERIFY, CALL_ANALYTIC_ACCEPT = 0, 1, 2

VERIFY_MODES = {"static": VERIFY_STATIC, "compact": VERIFY_COMPACT, "cap_accept": VERIFY_CAP_ACCEPT}
SCHED_MODES = {"argmax": SCHED_ARGMAX, "greedy": SCHED_GREEDY, "fixed": SCHED_FIXED}

_c = ctypes
_vp, _i, _u64, _sz, _f = _c.c_void_p, _c.c_int, _c.c_uint64, _c.c_size_t, _c.c_float

_SIGNATURES = {
    "dspark_status_string": (_c.c_char_p, [_i]),
    "dspark_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_workspace_init": (_i, [_vp, _sz, _vp]),
    "dspark_workspace_status_offset": (_sz, [_i, _i]),
    "dspark_set_draft_path": (_i, [_i]),
    "dspark_prepacked_w2_bytes": (_sz, [_i, _i, _i]),
    "dspark_prepack_w2": (_i, [_vp, _i, _i, _i, _vp, _sz, _vp]),
    "dspark_cost_table_prepare": (_i, [_vp, _i, _vp, _i, _i, _vp]),
    "dspark_markov_draft": (_i, [_vp, _vp, _vp, _vp, _u64, _u64, _vp, _vp, _i, _i, _i, _i, _i,
                                 _vp, _vp, _vp, _vp, _sz, _vp]),
    "dspark_markov_draft_noalloc": (_i, [_vp, _vp, _vp, _vp, _u64, _u64, _vp, _vp, _i, _i, _i, _i,
                                         _i, _vp, _vp, _vp, _vp]),
    "dspark_noalloc_scratch_bytes": (_sz, []),
    "dspark_probe_read": (_i, [_vp, _sz, _vp, _vp]),
    "dspark_probe_mfma": (_i, [_vp, _i, _i, _vp]),
    "dspark_probe_mfma_flops": (_c.c_double, [_i, _i]),
    "dspark_confidence": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _i, _i, _i, _i, _i, _i,
                               _vp, _vp, _vp, _vp]),
    "dspark_markov_draft_confidence": (_i, [_vp, _vp, _vp, _vp, _u64, _u64, _vp, _vp, _i, _i, _i,
                                            _i, _i, _vp, _vp, _f, _vp, _i, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _sz, _vp]),
    "dspark_schedule_topb": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "dspark_pack_ragged": (_i, [_vp, _vp, _vp, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                _vp]),
    "dspark_schedule_pack": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i,
                                  _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "dspark_verify": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _u64, _u64,
                           _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dspark_advance": (_i, [_vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _i, _vp]),
    "dspark_markov_shard_partials": (_i, [_vp, _c.c_longlong, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                          _vp, _sz, _vp]),
    "dspark_markov_shard_summary": (_i, [_vp, _sz, _i, _i, _vp, _vp]),
    "dspark_markov_shard_select": (_i, [_vp, _c.c_longlong, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i,
                                        _u64, _u64, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                        _vp, _i, _vp]),
    "dspark_sts_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "dspark_sts_fit": (_i, [_vp, _vp, _vp, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "dspark_observe_words": (_sz, [_i, _i, _i]),
    "dspark_observe": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "dspark_analytic_accept": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                    _vp, _vp, _sz, _vp]),
    "dspark_markov_logits": (_i, [_vp, _c.c_longlong, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "dspark_markov_partials": (_i, [_vp, _c.c_longlong, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz,
                                    _vp]),
    "dspark_markov_select": (_i, [_vp, _c.c_longlong, _vp, _vp, _vp, _i, _vp, _u64, _u64, _vp, _vp,
                                  _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _vp]),
}
EXPORTS = tuple(_SIGNATURES)

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdspark.so (build it with ``python -m draft_verify_sampling_markov_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m draft_verify_sampling_markov_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class DsparkError(RuntimeError):
    pass


def status_string(rc: int) -> str:
    return load_library().dspark_status_string(rc).decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise DsparkError(status_string(rc))


# ---------------------------------------------------------------------------
# tensor helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _dev(t, name: str, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _opt(t, name, dtype=None, shape=None):
    return None if t is None else _dev(t, name, dtype, shape)


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _empty(shape, dtype, device):
    return _torch().empty(shape, dtype=dtype, device=device)


# ---------------------------------------------------------------------------
# utilities
# ---------------------------------------------------------------------------

def workspace_bytes(call: int, R: int, gamma: int, V: int, r: int) -> int:
    return int(load_library().dspark_workspace_bytes(call, R, gamma, V, r))


DRAFT_AUTO, DRAFT_PER_SLOT, DRAFT_RESIDENT = 0, 1, 2


def set_draft_path(path: int) -> int:
    """Process-wide choice of draft kernels (DRAFT_AUTO: the library's choice;
    DRAFT_PER_SLOT: per-slot launches; DRAFT_RESIDENT: the resident-W2 block
    kernel where the shape allows it). Returns the previous choice."""
    rc = load_library().dspark_set_draft_path(int(path))
    _check(min(rc, 0))
    return rc


def draft_status(ws, R: int, V: int) -> int:
    """The error word of a draft workspace (synchronises): 1 if a resident
    draft's barrier wait ran out since the workspace was initialised."""
    off = int(load_library().dspark_workspace_status_offset(R, V))
    if off == 0 or off + 4 > ws.numel() * ws.element_size():
        raise ValueError("workspace too small for these sizes")
    return int(ws.view(-1)[off:off + 4].cpu().numpy().view(np.uint32)[0])


def workspace_init(ws, stream=None):
    """Put a freshly allocated workspace (uint8 device tensor) in its initial state."""
    _check(load_library().dspark_workspace_init(_dev(ws, "ws"), ws.numel() * ws.element_size(),
                                                _stream(stream)))
    return ws


def new_workspace(call: int, R: int, gamma: int, V: int, r: int, device, stream=None):
    """Allocate and initialise the workspace of `call` for these sizes."""
    torch = _torch()
    need = workspace_bytes(call, R, gamma, V, r)
    return workspace_init(_empty((max(need, 1),), torch.uint8, device), stream)


def prepacked_w2_bytes(r: int, V: int, dtype: int) -> int:
    return int(load_library().dspark_prepacked_w2_bytes(r, V, dtype))


def prepack_w2(W2, stream=None):
    """W2 [r, V] (float32 or bfloat16) -> pre-packed operand buffer (same dtype)."""
    torch = _torch()
    r, V = W2.shape
    dt = _dtype_code(W2)
    nbytes = prepacked_w2_bytes(r, V, dt)
    if nbytes == 0:
        raise DsparkError("unsupported W2 shape")
    out = torch.empty(nbytes // W2.element_size(), dtype=W2.dtype, device=W2.device)
    _check(load_library().dspark_prepack_w2(_dev(W2, "W2"), r, V, dt, out.data_ptr(), nbytes,
                                            _stream(stream)))
    return out


def cost_table_prepare(raw_step_time_s: Sequence[float], tiers: Sequence[int],
                       staircase: bool) -> np.ndarray:
    """Host call: raw step time T(M), M = 0..M_max -> sps_milli (uint32)."""
    raw = np.ascontiguousarray(raw_step_time_s, dtype=np.float64)
    tr = np.ascontiguousarray(tiers, dtype=np.int32)
    out = np.zeros(raw.shape[0], dtype=np.uint32)
    _check(load_library().dspark_cost_table_prepare(raw.ctypes.data, raw.shape[0] - 1,
                                                    tr.ctypes.data, tr.shape[0], int(bool(staircase)),
                                                    out.ctypes.data))
    return out


# ---------------------------------------------------------------------------
# hot calls
# ---------------------------------------------------------------------------

def markov_draft(U, W1, W2p, anchor, *, r: int, seed: int = 0, step: int = 0, step_dev=None,
                 req_ids=None, out=None, ws=None, stream=None):
    """U [R, gamma, V]; W1 [V, r]; W2p pre-packed; anchor [R] int32.
    step_dev: optional int64 [1] device tensor holding the step (overrides step).
    Returns (tokens int32 [R, gamma], p_draft f32, lse_draft f32)."""
    torch = _torch()
    R, gamma, V = U.shape
    dt = _dtype_code(U)
    dev = U.device
    if req_ids is None:
        req_ids = torch.arange(R, dtype=torch.int32, device=dev)
    if out is None:
        out = (_empty((R, gamma), torch.int32, dev), _empty((R, gamma), torch.float32, dev),
               _empty((R, gamma), torch.float32, dev))
    if ws is None:
        ws = new_workspace(CALL_MARKOV_DRAFT, R, gamma, V, r, dev, stream)
    tokens, p, lse = out
    _check(load_library().dspark_markov_draft(
        _dev(U, "U"), _dev(W1, "W1", U.dtype, (V, r)), _dev(W2p, "W2p", U.dtype),
        _dev(anchor, "anchor", torch.int32, (R,)), seed, step,
        _opt(step_dev, "step_dev", torch.int64, (1,)), _dev(req_ids, "req_ids", None, (R,)),
        R, gamma, V, r, dt, _dev(tokens, "tokens", torch.int32, (R, gamma)),
        _dev(p, "p_draft", torch.float32, (R, gamma)), _dev(lse, "lse_draft", torch.float32, (R, gamma)),
        _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))
    return tokens, p, lse


def markov_draft_noalloc(U, W1, W2p, anchor, *, r: int, seed: int = 0, step: int = 0,
                         step_dev=None, req_ids=None, out=None, stream=None):
    """markov_draft on the library's own device scratch array (no workspace,
    no allocation in the library). Returns (tokens, p_draft, lse_draft)."""
    torch = _torch()
    R, gamma, V = U.shape
    dev = U.device
    if req_ids is None:
        req_ids = torch.arange(R, dtype=torch.int32, device=dev)
    if out is None:
        out = (_empty((R, gamma), torch.int32, dev), _empty((R, gamma), torch.float32, dev),
               _empty((R, gamma), torch.float32, dev))
    tokens, p, lse = out
    _check(load_library().dspark_markov_draft_noalloc(
        _dev(U, "U"), _dev(W1, "W1", U.dtype, (V, r)), _dev(W2p, "W2p", U.dtype),
        _dev(anchor, "anchor", torch.int32, (R,)), seed, step,
        _opt(step_dev, "step_dev", torch.int64, (1,)), _dev(req_ids, "req_ids", None, (R,)),
        R, gamma, V, r, _dtype_code(U), _dev(tokens, "tokens", torch.int32, (R, gamma)),
        _dev(p, "p_draft", torch.float32, (R, gamma)), _dev(lse, "lse_draft", torch.float32, (R, gamma)),
        _stream(stream)))
    return tokens, p, lse


def probe_read(buf, sink, stream=None):
    """One streaming-read sweep over ``buf`` (dspark_probe_read); bytes read =
    buf.numel() * element size."""
    _check(load_library().dspark_probe_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                            _dev(sink, "sink"), _stream(stream)))


def probe_mfma(sink, *, grid: int, iters: int, stream=None) -> float:
    """One matrix-core loop launch (dspark_probe_mfma); returns its FLOP."""
    lib = load_library()
    _check(lib.dspark_probe_mfma(_dev(sink, "sink"), int(grid), int(iters), _stream(stream)))
    return float(lib.dspark_probe_mfma_flops(int(grid), int(iters)))


def markov_draft_confidence(U, W1, W2p, anchor, h, w, b: float, *, r: int, inv_temp=None,
                            seed: int = 0, step: int = 0, step_dev=None, req_ids=None, out=None,
                            conf_out=None, logit=None, ws=None, stream=None):
    """markov_draft and confidence in one call (each slot's GEMM launch also
    scores the slot). h [R, gamma, d]; w [d + r] f32. Returns (tokens, p_draft,
    lse_draft, conf, surv)."""
    torch = _torch()
    R, gamma, V = U.shape
    d = h.shape[2]
    dev = U.device
    if req_ids is None:
        req_ids = torch.arange(R, dtype=torch.int32, device=dev)
    if out is None:
        out = (_empty((R, gamma), torch.int32, dev), _empty((R, gamma), torch.float32, dev),
               _empty((R, gamma), torch.float32, dev))
    if conf_out is None:
        conf_out = (_empty((R, gamma), torch.float32, dev), _empty((R, gamma), torch.float32, dev))
    if ws is None:
        ws = new_workspace(CALL_MARKOV_DRAFT, R, gamma, V, r, dev, stream)
    tokens, p, lse = out
    conf, surv = conf_out
    _check(load_library().dspark_markov_draft_confidence(
        _dev(U, "U"), _dev(W1, "W1", U.dtype, (V, r)), _dev(W2p, "W2p", U.dtype),
        _dev(anchor, "anchor", torch.int32, (R,)), seed, step,
        _opt(step_dev, "step_dev", torch.int64, (1,)), _dev(req_ids, "req_ids", None, (R,)),
        R, gamma, V, r, _dtype_code(U), _dev(h, "h", U.dtype, (R, gamma, d)),
        _dev(w, "w", torch.float32, (d + r,)), float(b),
        _opt(inv_temp, "inv_temp", torch.float32, (gamma,)), d,
        _dev(tokens, "tokens", torch.int32, (R, gamma)),
        _dev(p, "p_draft", torch.float32, (R, gamma)), _dev(lse, "lse_draft", torch.float32, (R, gamma)),
        _dev(conf, "conf", torch.float32, (R, gamma)), _dev(surv, "surv", torch.float32, (R, gamma)),
        _opt(logit, "logit", torch.float32, (R, gamma)),
        _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))
    return tokens, p, lse, conf, surv


def confidence(h, W1, anchor, tokens, w, b: float, inv_temp=None, out=None, logit=None,
               stream=None):
    """h [R, gamma, d]; W1 [V, r]; w [d + r] f32. Returns (conf, surv) f32 [R, gamma];
    ``logit`` (f32 [R, gamma], optional) receives the pre-temperature logits."""
    torch = _torch()
    R, gamma, d = h.shape
    V, r = W1.shape
    dev = h.device
    if out is None:
        out = (_empty((R, gamma), torch.float32, dev), _empty((R, gamma), torch.float32, dev))
    conf, surv = out
    _check(load_library().dspark_confidence(
        _dev(h, "h"), _dev(W1, "W1", h.dtype), _dev(anchor, "anchor", torch.int32, (R,)),
        _dev(tokens, "tokens", torch.int32, (R, gamma)), _dev(w, "w", torch.float32, (d + r,)),
        float(b), _opt(inv_temp, "inv_temp", torch.float32, (gamma,)), R, gamma, d, V, r,
        _dtype_code(h), _dev(conf, "conf", torch.float32, (R, gamma)),
        _dev(surv, "surv", torch.float32, (R, gamma)), _opt(logit, "logit", torch.float32, (R, gamma)),
        _stream(stream)))
    return conf, surv


def schedule_topb(surv, sps_milli, *, B_cap: int, mode: int, K_fixed: int = 0, surv_budget=None,
                  out=None, stream=None):
    """surv [R, gamma] f32; sps_milli [M_max+1] (int32/uint32 device tensor).
    Returns (win_len int32 [R], K int32 [1])."""
    torch = _torch()
    R, gamma = surv.shape
    M_max = sps_milli.numel() - 1
    if out is None:
        out = (_empty((R,), torch.int32, surv.device), _empty((1,), torch.int32, surv.device))
    win, K = out
    _check(load_library().dspark_schedule_topb(
        _dev(surv, "surv", torch.float32), _opt(surv_budget, "surv_budget", torch.float32, (R, gamma)),
        _dev(sps_milli, "sps_milli"), M_max, R, gamma, int(B_cap), int(mode), int(K_fixed),
        _dev(win, "win_len", torch.int32, (R,)), _dev(K, "K_out", torch.int32, (1,)), _stream(stream)))
    return win, K


def schedule_pack(surv, sps_milli, anchor, tokens, tiers: Sequence[int], M_cap: int, *,
                  B_cap: int, mode: int, K_fixed: int = 0, surv_budget=None,
                  pack_windows: bool = True, sched_out=None, pack_out=None, stream=None):
    """schedule_topb then pack_ragged in one launch. pack_windows=False packs
    full blocks (as pack_ragged with win_len None). Returns ((win_len, K),
    pack dict)."""
    torch = _torch()
    R, gamma = surv.shape
    M_max = sps_milli.numel() - 1
    dev = surv.device
    if sched_out is None:
        sched_out = (_empty((R,), torch.int32, dev), _empty((1,), torch.int32, dev))
    if pack_out is None:
        pack_out = {"cu_seqlens": _empty((R + 1,), torch.int32, dev),
                    "packed_tokens": _empty((M_cap,), torch.int32, dev),
                    "packed_req": _empty((M_cap,), torch.int32, dev),
                    "packed_slot": _empty((M_cap,), torch.int32, dev),
                    "totals": _empty((2,), torch.int32, dev)}
    win, K = sched_out
    tr = np.ascontiguousarray(tiers, dtype=np.int32)
    _check(load_library().dspark_schedule_pack(
        _dev(surv, "surv", torch.float32), _opt(surv_budget, "surv_budget", torch.float32, (R, gamma)),
        _dev(sps_milli, "sps_milli"), M_max, R, gamma, int(B_cap), int(mode), int(K_fixed),
        _dev(win, "win_len", torch.int32, (R,)), _dev(K, "K_out", torch.int32, (1,)),
        _dev(anchor, "anchor", torch.int32, (R,)), _dev(tokens, "tokens", torch.int32, (R, gamma)),
        1 if pack_windows else 0, tr.ctypes.data, tr.shape[0], M_cap,
        _dev(pack_out["cu_seqlens"], "cu_seqlens", torch.int32, (R + 1,)),
        _dev(pack_out["packed_tokens"], "packed_tokens", torch.int32),
        _dev(pack_out["packed_req"], "packed_req", torch.int32),
        _dev(pack_out["packed_slot"], "packed_slot", torch.int32),
        _dev(pack_out["totals"], "totals", torch.int32, (2,)), _stream(stream)))
    return sched_out, pack_out


def pack_ragged(anchor, tokens, win_len, tiers: Sequence[int], M_cap: int, out=None, stream=None):
    """Returns dict of cu_seqlens [R+1], packed_tokens/req/slot [M_cap], totals [2] (int32)."""
    torch = _torch()
    R, gamma = tokens.shape
    dev = tokens.device
    if out is None:
        out = {"cu_seqlens": _empty((R + 1,), torch.int32, dev),
               "packed_tokens": _empty((M_cap,), torch.int32, dev),
               "packed_req": _empty((M_cap,), torch.int32, dev),
               "packed_slot": _empty((M_cap,), torch.int32, dev),
               "totals": _empty((2,), torch.int32, dev)}
    tr = np.ascontiguousarray(tiers, dtype=np.int32)
    _check(load_library().dspark_pack_ragged(
        _dev(anchor, "anchor", torch.int32, (R,)), _dev(tokens, "tokens", torch.int32),
        _opt(win_len, "win_len", torch.int32, (R,)), R, gamma, tr.ctypes.data, tr.shape[0], M_cap,
        _dev(out["cu_seqlens"], "cu_seqlens", torch.int32, (R + 1,)),
        _dev(out["packed_tokens"], "packed_tokens", torch.int32),
        _dev(out["packed_req"], "packed_req", torch.int32),
        _dev(out["packed_slot"], "packed_slot", torch.int32),
        _dev(out["totals"], "totals", torch.int32, (2,)), _stream(stream)))
    return out


def verify(target_packed, cu_seqlens, anchor, tokens, p_draft, lse_draft, U, W1, W2p, *, r: int,
           mode: int, win_len=None, seed: int = 0, step: int = 0, step_dev=None, req_ids=None,
           with_ceiling: bool = True, out=None, ws=None, stream=None):
    """Returns dict: accept_len [R], out_tokens [R, gamma+1], n_out [R], ceiling_len [R] or None."""
    torch = _torch()
    R, gamma, V = U.shape
    M_cap = target_packed.shape[0]
    dev = U.device
    if req_ids is None:
        req_ids = torch.arange(R, dtype=torch.int32, device=dev)
    if out is None:
        out = {"accept_len": _empty((R,), torch.int32, dev),
               "out_tokens": _empty((R, gamma + 1), torch.int32, dev),
               "n_out": _empty((R,), torch.int32, dev),
               "ceiling_len": _empty((R,), torch.int32, dev) if with_ceiling else None}
    if ws is None:
        ws = new_workspace(CALL_VERIFY, R, gamma, V, r, dev, stream)
    _check(load_library().dspark_verify(
        _dev(target_packed, "target_packed", U.dtype, (M_cap, V)), M_cap,
        _dev(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)), _dev(anchor, "anchor", torch.int32, (R,)),
        _dev(tokens, "tokens", torch.int32, (R, gamma)), _dev(p_draft, "p_draft", torch.float32, (R, gamma)),
        _dev(lse_draft, "lse_draft", torch.float32, (R, gamma)), _dev(U, "U"),
        _dev(W1, "W1", U.dtype, (V, r)), _dev(W2p, "W2p", U.dtype),
        _opt(win_len, "win_len", torch.int32, (R,)), int(mode), seed, step,
        _opt(step_dev, "step_dev", torch.int64, (1,)), _dev(req_ids, "req_ids", None, (R,)), R,
        gamma, V, r, _dtype_code(U),
        _dev(out["accept_len"], "accept_len", torch.int32, (R,)),
        _dev(out["out_tokens"], "out_tokens", torch.int32, (R, gamma + 1)),
        _dev(out["n_out"], "n_out", torch.int32, (R,)),
        _opt(out["ceiling_len"], "ceiling_len", torch.int32, (R,)),
        _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def markov_partials(U_k, ldU: int, W1, W2p, x_prev, xstride: int, *, R: int, V: int, r: int,
                    part, stream=None):
    """One slot's GEMM + per-tile softmax partials into ``part`` (uint8 buffer)."""
    _check(load_library().dspark_markov_partials(
        U_k.data_ptr(), int(ldU), _dev(W1, "W1", U_k.dtype, (V, r)), _dev(W2p, "W2p", U_k.dtype),
        x_prev.data_ptr(), int(xstride), R, V, r, _dtype_code(U_k), _dev(part, "part"),
        part.numel() * part.element_size(), _stream(stream)))


def markov_select(U_k, ldU: int, W1, W2p, x_prev, xstride: int, part, *, k: int, R: int, V: int,
                  r: int, seed: int, step: int, req_ids, tok_out, p_out, lse_out, ostride: int,
                  step_dev=None, stream=None):
    """One slot's draw from the partials of markov_partials (pointer-level outputs:
    tok_out/p_out/lse_out may be strided views' base pointers given as tensors)."""
    _check(load_library().dspark_markov_select(
        U_k.data_ptr(), int(ldU), _dev(W1, "W1", U_k.dtype, (V, r)), _dev(W2p, "W2p", U_k.dtype),
        x_prev.data_ptr(), int(xstride), _dev(part, "part"), seed, step,
        _opt(step_dev, "step_dev", _torch().int64, (1,)), req_ids.data_ptr(), int(k),
        R, V, r, _dtype_code(U_k), tok_out.data_ptr(), p_out.data_ptr(), lse_out.data_ptr(),
        int(ostride), _stream(stream)))


def markov_logits(U_k, ldU: int, W1, W2p, x_prev, *, R: int, V: int, r: int, stream=None):
    """Diagnostic: full Markov logits z [R, V] f32 of one slot."""
    torch = _torch()
    z = _empty((R, V), torch.float32, U_k.device)
    _check(load_library().dspark_markov_logits(
        U_k.data_ptr(), int(ldU), _dev(W1, "W1", U_k.dtype, (V, r)), _dev(W2p, "W2p", U_k.dtype),
        _dev(x_prev, "x_prev", torch.int32, (R,)), R, V, r, _dtype_code(U_k), z.data_ptr(),
        _stream(stream)))
    return z


def advance(anchor, accept_len, out_tokens, *, step_dev=None, surv_hist=None, surv=None,
            stream=None):
    """Carry a decode loop to its next step on the device: anchor <- the token
    committed last (out_tokens[r, accept_len[r]]), step_dev += 1, and the
    survival history surv_hist [n_hist, R, gamma] shifted by one level with
    surv entering at level 0."""
    torch = _torch()
    R, g1 = out_tokens.shape
    gamma = g1 - 1
    n_hist = 0 if surv_hist is None else surv_hist.shape[0]
    _check(load_library().dspark_advance(
        _dev(anchor, "anchor", torch.int32, (R,)), _dev(accept_len, "accept_len", torch.int32, (R,)),
        _dev(out_tokens, "out_tokens", torch.int32), R, gamma,
        _opt(step_dev, "step_dev", torch.int64, (1,)),
        _opt(surv_hist, "surv_hist", torch.float32, (n_hist, R, gamma)),
        _opt(surv, "surv", torch.float32, (R, gamma)), n_hist, _stream(stream)))


def markov_shard_partials(U_k, ldU: int, W1, W2p_g, x_prev, xstride: int, *, R: int, V_g: int,
                          V: int, r: int, part, stream=None):
    """Rank's GEMM pass over its V_g columns (dspark_markov_shard_partials)."""
    _check(load_library().dspark_markov_shard_partials(
        U_k.data_ptr(), int(ldU), _dev(W1, "W1", U_k.dtype, (V, r)), _dev(W2p_g, "W2p", U_k.dtype),
        x_prev.data_ptr(), int(xstride), R, int(V_g), V, r, _dtype_code(U_k), _dev(part, "part"),
        part.numel() * part.element_size(), _stream(stream)))


def markov_shard_summary(part, *, R: int, V_g: int, out, stream=None):
    """Rank's (max, sum of exp) per request from its partials workspace into
    ``out`` (float32 [R, 2] or a view of a [G, R, 2] buffer's row)."""
    _check(load_library().dspark_markov_shard_summary(
        _dev(part, "part"), part.numel() * part.element_size(), R, V_g, out.data_ptr(),
        _stream(stream)))


def markov_shard_select(U_k, ldU: int, W1, W2p_g, x_prev, xstride: int, part, summaries, *,
                        G: int, g: int, v0: int, k: int, R: int, V_g: int, V: int, r: int,
                        seed: int, step: int, req_ids, tok_out, p_out, lse_out, ostride: int = 1,
                        step_dev=None, stream=None):
    """Rank g's select for slot k (dspark_markov_shard_select); pointer-level
    outputs like markov_select."""
    torch = _torch()
    _check(load_library().dspark_markov_shard_select(
        U_k.data_ptr(), int(ldU), _dev(W1, "W1", U_k.dtype, (V, r)), _dev(W2p_g, "W2p", U_k.dtype),
        x_prev.data_ptr(), int(xstride), _dev(part, "part"),
        _dev(summaries, "summaries", torch.float32, (G, R, 2)), int(G), int(g), int(v0), seed, step,
        _opt(step_dev, "step_dev", torch.int64, (1,)), req_ids.data_ptr(), int(k), R, int(V_g), V, r,
        _dtype_code(U_k), tok_out.data_ptr(), p_out.data_ptr(), lse_out.data_ptr(), int(ostride),
        _stream(stream)))


def sts_fit(z, y, betas, *, n_bins: int = 16, mask=None, stream=None):
    """Per-position inverse temperatures (dspark_sts_fit). z, y: f32 [N, gamma];
    betas: f32 [n_grid] device tensor; mask: optional uint8/bool [N, gamma].
    Returns (inv_temp f32 [gamma], ece f32 [gamma, n_grid])."""
    torch = _torch()
    N, gamma = z.shape
    n_grid = betas.numel()
    nbytes = int(load_library().dspark_sts_workspace_bytes(N, gamma, n_grid, n_bins))
    if nbytes == 0:
        raise DsparkError("unsupported temperature-fit sizes")
    ws = _empty((nbytes,), torch.uint8, z.device)
    inv = _empty((gamma,), torch.float32, z.device)
    ece = _empty((gamma, n_grid), torch.float32, z.device)
    if mask is not None and mask.dtype == torch.bool:
        mask = mask.to(torch.uint8)
    _check(load_library().dspark_sts_fit(
        _dev(z, "z", torch.float32, (N, gamma)), _dev(y, "y", torch.float32, (N, gamma)),
        _opt(mask, "mask", torch.uint8, (N, gamma)), N, gamma, _dev(betas, "betas", torch.float32),
        n_grid, int(n_bins), inv.data_ptr(), ece.data_ptr(), ws.data_ptr(), nbytes, _stream(stream)))
    return inv, ece


def observe_words(R: int, gamma: int, n_bins: int) -> int:
    return int(load_library().dspark_observe_words(R, gamma, n_bins))


def new_observe_block(R: int, gamma: int, n_bins: int, device, stream=None):
    """A zeroed observability block (int64 device tensor of observe_words words)."""
    torch = _torch()
    n = observe_words(R, gamma, n_bins)
    if n == 0:
        raise DsparkError("unsupported observability block sizes")
    blk = _empty((n,), torch.int64, device)
    workspace_init(blk.view(torch.uint8), stream)
    return blk


def observe(conf, surv, win_len, accept_len, ceiling_len, cu_seqlens, stats, *, n_bins: int,
            stream=None):
    """Add one step to the observability block ``stats`` (dspark_observe)."""
    torch = _torch()
    R, gamma = conf.shape
    _check(load_library().dspark_observe(
        _dev(conf, "conf", torch.float32, (R, gamma)), _dev(surv, "surv", torch.float32, (R, gamma)),
        _dev(win_len, "win_len", torch.int32, (R,)), _dev(accept_len, "accept_len", torch.int32, (R,)),
        _dev(ceiling_len, "ceiling_len", torch.int32, (R,)),
        _dev(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)), R, gamma, int(n_bins),
        _dev(stats, "stats", torch.int64), stats.numel(), _stream(stream)))


def parse_observe(block, R: int, gamma: int, n_bins: int) -> Dict[str, object]:
    """Split a host copy of an observability block into its named counters
    (layout of dspark_observe) and derive ECE and utilisation from them."""
    b = np.asarray(block).view(np.uint64).astype(object)
    g1 = gamma + 1
    hist0, req0 = 8, 8 + 3 * g1
    bins0 = req0 + 3 * R
    out = {"steps": int(b[0]), "req_steps": int(b[1]), "committed": int(b[2]),
           "accepted": int(b[3]), "ceiling": int(b[4]), "window": int(b[5]),
           "verified": int(b[6]),
           "hist_window": b[hist0:hist0 + g1], "hist_accept": b[hist0 + g1:hist0 + 2 * g1],
           "hist_ceiling": b[hist0 + 2 * g1:hist0 + 3 * g1],
           "req_accepted": b[req0:req0 + R], "req_ceiling": b[req0 + R:req0 + 2 * R],
           "req_window": b[req0 + 2 * R:req0 + 3 * R],
           "bins": b[bins0:bins0 + 6 * gamma * n_bins].reshape(2, gamma, n_bins, 3)}

    def ece(cells):
        cnt = cells[..., 0].sum(axis=0)
        n = int(cnt.sum())
        if n == 0:
            return float("nan")
        ps, hits = cells[..., 1].sum(axis=0), cells[..., 2].sum(axis=0)
        return sum(abs(float(ps[i]) / 2.0 ** 32 - int(hits[i])) for i in range(n_bins)) / n

    out["ece_conditional"] = ece(out["bins"][0])
    out["ece_prefix"] = ece(out["bins"][1])
    out["ece_prefix_per_position"] = [ece(out["bins"][1, k][None]) for k in range(gamma)]
    out["utilisation"] = (out["accepted"] / out["ceiling"]) if out["ceiling"] else float("nan")
    return out


def analytic_accept(target_packed, cu_seqlens, anchor, tokens, lse_draft, U, W1, W2p, *, r: int,
                    out=None, ws=None, stream=None):
    """c*[R, gamma] f32 = 1 - 1/2 |p_d - p_t|_1 for every verified slot, NaN elsewhere."""
    torch = _torch()
    R, gamma, V = U.shape
    M_cap = target_packed.shape[0]
    dev = U.device
    if out is None:
        out = _empty((R, gamma), torch.float32, dev)
    if ws is None:
        ws = new_workspace(CALL_ANALYTIC_ACCEPT, R, gamma, V, r, dev, stream)
    _check(load_library().dspark_analytic_accept(
        _dev(target_packed, "target_packed", U.dtype, (M_cap, V)), M_cap,
        _dev(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)), _dev(anchor, "anchor", torch.int32, (R,)),
        _dev(tokens, "tokens", torch.int32, (R, gamma)),
        _dev(lse_draft, "lse_draft", torch.float32, (R, gamma)), _dev(U, "U"),
        _dev(W1, "W1", U.dtype, (V, r)), _dev(W2p, "W2p", U.dtype), R, gamma, V, r, _dtype_code(U),
        _dev(out, "cstar", torch.float32, (R, gamma)), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)))
    return out


from .chain import Chain  # noqa: E402
from .shard import ShardedDraft  # noqa: E402  (needs the functions above)

__all__ = [
    "load_library", "status_string", "DsparkError", "workspace_bytes", "workspace_init",
    "new_workspace", "prepacked_w2_bytes",
    "prepack_w2", "cost_table_prepare", "markov_draft", "confidence", "schedule_topb",
    "pack_ragged", "verify", "markov_logits", "markov_partials",
    "markov_select", "advance", "observe_words", "new_observe_block", "observe", "parse_observe",
    "analytic_accept", "sts_fit", "markov_shard_partials", "markov_shard_summary", "markov_shard_select", "ShardedDraft", "Chain",
    "EXPORTS", "F32", "BF16",
    "VERIFY_STATIC", "VERIFY_COMPACT", "VERIFY_CAP_ACCEPT", "SCHED_ARGMAX", "SCHED_GREEDY",
    "SCHED_FIXED", "VERIFY_MODES", "SCHED_MODES",
]
