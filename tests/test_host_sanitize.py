"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The test builds the library with its host pass under both sanitizers (the GPU
code unchanged) into a temporary directory. A child process with clang's
shared ASan runtime preloaded loads it, runs the C-ABI tests (argument checks,
workspace sizes, the cost table) and calls every size function on random and
extreme arguments; any sanitizer report aborts the child.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from draft_verify_sampling_markov_amd import build  # noqa: E402

FUZZ = r"""
import numpy as np
import os
import draft_verify_sampling_markov_amd as dv
lib = dv.load_library(os.environ["DSPARK_HOSTSAN_LIB"])
assert lib._name == os.environ["DSPARK_HOSTSAN_LIB"]
rng = np.random.default_rng(0)
vals = [-2**31, -1, 0, 1, 2, 7, 8, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257,
        2047, 2048, 4095, 4096, 4097, 151936, 1 << 20, 1 << 24, 1 << 28, 2**31 - 1]
for _ in range(5000):
    R, g, V, r = (int(rng.choice(vals)) for _ in range(4))
    lib.dspark_workspace_bytes(int(rng.integers(-1, 4)), R, g, V, r)
    lib.dspark_workspace_status_offset(R, V)
    lib.dspark_prepacked_w2_bytes(r, V, int(rng.integers(-1, 3)))
    lib.dspark_observe_words(R, g, r)
    lib.dspark_sts_workspace_bytes(R, g, V, r)
    lib.dspark_status_string(int(rng.integers(-50, 50)))
print("fuzz ok")
"""


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_code_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    lib = build.build(host_sanitize=True, out=str(tmp_path / "libdspark_hostsan.so"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               DSPARK_HOSTSAN_LIB=lib,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "hostsan_plugin",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert " passed" in r.stdout
    r = subprocess.run([sys.executable, "-c", FUZZ], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "fuzz ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
