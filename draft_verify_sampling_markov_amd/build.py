"""Build libdspark.so (gfx950) in-tree with hipcc.

Usage: python -m draft_verify_sampling_markov_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdspark.so")
SOURCES = ["abi.hip", "markov.hip", "confidence.hip", "schedule.hip", "verify.hip", "decode.hip", "observe.hip",
           "calibrate.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
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


def build(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
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
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
