"""Build libdspark.so (gfx950) in-tree with hipcc.

Usage: python -m draft_verify_sampling_markov_amd.build [-v] [--host-sanitize]

--host-sanitize builds libdspark_hostsan.so instead: the same library with
its host code (argument checks, sizes, the cost table) under AddressSanitizer
and UndefinedBehaviorSanitizer; the GPU code is built as usual. Load it into
a process started with clang's shared ASan runtime preloaded
(LD_PRELOAD=<rocm llvm>/lib/clang/<v>/lib/linux/libclang_rt.asan-x86_64.so,
ASAN_OPTIONS=detect_leaks=0) and pass its path to load_library().
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
LIB_HOSTSAN = os.path.join(PKG, "libdspark_hostsan.so")
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


# host-side sanitizers only: each -fsanitize= goes to the host pass
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan",
]


def build(verbose: bool = False, host_sanitize: bool = False, out: str = "") -> str:
    """Compile every HIP source (one hipcc per source, in parallel), link them
    into one shared library; returns its path (out, if given)."""
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    extra = HOST_SANITIZE_FLAGS if host_sanitize else []
    out = out or (LIB_HOSTSAN if host_sanitize else LIB)
    with tempfile.TemporaryDirectory(prefix="dspark_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c",
                 os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp],
             verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_sanitize="--host-sanitize" in sys.argv))
