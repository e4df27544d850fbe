"""bench.py's output contract.

CPU: more than one GPU is refused with a message and exit status 2, before
any GPU work. GPU: a short run prints one JSON line with every field the
measurement contract names (metric, value, unit, n_gpus, steps, warmup,
ms_per_step, higher_is_better, scaling, vs_baseline, dtype, data, config with
the workload, and the roofline object of the dominant kernel).
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_json_line_contract():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny",
                        "--mode", "static", "--steps", "3", "--warmup", "1", "--decode-steps", "2",
                        "--observe-calls", "1", "--no-cpu-baseline", "--samples", "5",
                        "--cold-samples", "2", "--profile-steps", "2",
                        "--other-configs", "tiny:compact"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "slots/s" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("tiny")
    rl = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rl, k
    assert rl["bound"] == "hbm" and rl["peak"] == 8000.0 and rl["unit"] == "GB/s"
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert min(d["graph_ms_per_step"], d["eager_ms_per_step"]) == pytest.approx(d["ms_per_step"],
                                                                               abs=1e-4)
    # algorithmic bytes count W2 once per block: per launch R V b + r V b / gamma + R r b
    R, g, V, r, b = 4, 7, 1024, 32, 4
    assert rl["algorithmic_bytes_per_launch"] == round((g * R * V * b + r * V * b + g * R * r * b) / g)
    for key in ("step_ms", "step_ms_cache_cold"):
        st = d[key]
        assert st["p10"] <= st["median"] <= st["p90"] and st["n"] > 0
    vr = d["verify_roofline"]
    assert vr["bound"] == "hbm" and vr["unit"] == "GB/s" and vr["peak"] == 8000.0
    assert abs(vr["frac"] - vr["achieved"] / vr["peak"]) < 1e-3
    # static: every packed row of the full blocks, then one target row per
    # request, the U rows of the residual requests and W2
    assert vr["verified_rows"] == R * (g + 1)
    assert vr["pass1_bytes"] == R * (g + 1) * V * b
    assert vr["pass2_bytes"] == (R + vr["residual_requests"]) * V * b + r * V * b
    assert vr["stage_us"] == pytest.approx(d["stages_ms"]["verify"] * 1e3, abs=0.1)
    assert vr["achieved"] == pytest.approx((vr["pass1_bytes"] + vr["pass2_bytes"])
                                           / (vr["stage_us"] * 1e-6) / 1e9, rel=2e-3, abs=0.06)
    assert "tiny:compact" in d["other_workloads"]
    assert d["draft_call"]["per_slot_ms"] > 0
    pk = d["peaks_measured"]
    # plausible for one MI355X: well above a tenth of the published peaks, not above them
    assert 800 < pk["hbm_read_GBs"] <= 8000 and 800 < pk["reread_77MB_GBs"] < 20000
    assert 250 < pk["mfma_bf16_TFLOPs"] <= 2600
    assert rl["frac_of_measured_peak"] == pytest.approx(rl["achieved"] / pk["hbm_read_GBs"], abs=1e-3)
