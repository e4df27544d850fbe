"""Build libdspark.so (gfx950) in-tree with hipcc.

Usage: python -m draft_verify_sampling_markov_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdspark.so")
SOURCES = ["abi.hip", "markov.hip", "resident.hip", "confidence.hip", "schedule.hip", "verify.hip", "decode.hip", "observe.hip",
           "calibrate.hip", "noalloc.hip", "probe.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # keep the compiler from emitting packed-fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-lane atomics stay single atomics: the optimizer's wave-combined
    # form reads the result back at once, which drains every load in flight
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if noise:
            sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc per source, in parallel), link them
    into one shared library; returns its path."""
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="dspark_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
                 os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
