"""Static checks on the gfx950 code objects inside libdspark.so (no GPU needed).

Three properties that cost microseconds per launch when they slip:
- no kernel enables the dispatch-packet pointer (the packet lives in host
  memory; the compiler reaches for it when it moves a small private array into
  LDS and needs the workgroup size to address it);
- the hot-path kernels use no scratch (private segment) memory;
- no kernel calls a device function (every helper is inlined).

The library is built here, so this reads our own build output. Each
translation unit contributes one offload bundle to the .hip_fatbin section.
The descriptor layout is the AMDHSA kernel descriptor: 64 bytes,
private_segment_fixed_size at byte 4, kernel_code_properties (u16) at byte 56
with bit 1 = ENABLE_SGPR_DISPATCH_PTR.
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

import draft_verify_sampling_markov_amd as dv

LLVM = "/opt/rocm/llvm/bin"
HOT = ("markov_partials_kernel", "markov_select_kernel", "residual_partials_kernel",
       "residual_select_kernel", "row_partials_kernel", "decide_kernel", "confidence_kernel",
       "schedule_kernel", "pack_kernel", "advance_kernel", "accept_jobs_kernel",
       "accept_partials_kernel", "accept_reduce_kernel", "observe_kernel",
       "markov_shard_summary_kernel", "markov_shard_select_kernel", "sts_curve_kernel",
       "sts_pick_kernel", "sts_advance_kernel", "schedule_pack_kernel")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _kernel_descriptors(co, readelf):
    data = open(co, "rb").read()
    syms = subprocess.run([readelf, "-s", "--wide", co], check=True, capture_output=True, text=True).stdout
    secs = subprocess.run([readelf, "-S", "--wide", co], check=True, capture_output=True, text=True).stdout
    sections = []  # (address, file offset, size), to map symbol addresses to bytes
    for line in secs.splitlines():
        m = re.match(r"\s*\[\s*\d+\]\s+\S+\s+\S+\s+([0-9a-f]+)\s+([0-9a-f]+)\s+([0-9a-f]+)", line)
        if m:
            sections.append((int(m.group(1), 16), int(m.group(2), 16), int(m.group(3), 16)))
    out = {}
    for line in syms.splitlines():
        f = line.split()
        if len(f) >= 8 and f[-1].endswith(".kd") and f[3] == "OBJECT":
            addr = int(f[1], 16)
            off = next((o + addr - a for a, o, sz in sections if a <= addr < a + sz), None)
            if off is None:
                continue
            kd = data[off:off + 64]
            out[f[-1][:-3]] = {"private": struct.unpack_from("<I", kd, 4)[0],
                               "props": struct.unpack_from("<H", kd, 56)[0]}
    return out


def _unbundle(d):
    """The gfx950 code object of every translation unit, written into d."""
    if not os.path.exists(dv.LIB_PATH):
        pytest.skip("libdspark.so not built")
    objcopy, bundler = _tool("llvm-objcopy"), _tool("clang-offload-bundler")
    if not (objcopy and bundler):
        pytest.skip("LLVM tools not available")
    fat = os.path.join(d, "fatbin")
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", dv.LIB_PATH,
                    os.path.join(d, "copy.so")], check=True, capture_output=True)
    blob = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), blob)]
    cos = []
    for n, st in enumerate(starts):
        end = starts[n + 1] if n + 1 < len(starts) else len(blob)
        part, co = os.path.join(d, f"b{n}"), os.path.join(d, f"b{n}.co")
        with open(part, "wb") as fh:
            fh.write(blob[st:end])
        subprocess.run([bundler, "--type=o", f"--targets={TARGET}", f"--input={part}",
                        f"--output={co}", "--unbundle"], check=True, capture_output=True)
        cos.append(co)
    return cos


def _descriptors():
    readelf = _tool("llvm-readelf")
    if not readelf:
        pytest.skip("LLVM tools not available")
    out = {}
    with tempfile.TemporaryDirectory() as d:
        for co in _unbundle(d):
            out.update(_kernel_descriptors(co, readelf))
    assert out, "no kernel descriptors found"
    return out


def test_every_translation_unit_is_inspected():
    names = " ".join(_descriptors())
    for h in HOT:
        assert h in names, h


def test_no_kernel_reads_the_dispatch_packet():
    bad = [k for k, v in _descriptors().items() if v["props"] & 0x2]
    assert not bad, f"kernels that enable the dispatch pointer: {bad}"


def test_vector_path_hot_kernels_use_no_scratch():
    # instantiations whose last template flag is false are the non-vector
    # fallbacks (unaligned rows, ranks not a multiple of 8); those may spill
    desc = _descriptors()
    bad = [k for k, v in desc.items()
           if v["private"] and any(h in k for h in HOT) and not re.search(r"Lb0EEEv", k)]
    assert not bad, f"hot kernels with scratch: {bad}"


def test_no_kernel_calls_a_device_function():
    # a device function that is not inlined becomes a call (s_swappc) with its
    # own stack frame: a single-workgroup kernel that called its sort pass
    # that way ran several times slower
    objdump = _tool("llvm-objdump")
    if not objdump:
        pytest.skip("llvm-objdump not available")
    with tempfile.TemporaryDirectory() as d:
        calls = 0
        for co in _unbundle(d):
            text = subprocess.run([objdump, "-d", co], check=True, capture_output=True,
                                  text=True).stdout
            calls += len(re.findall(r"\bs_swappc_b64\b", text))
    assert calls == 0, f"{calls} device-function calls in the code objects"
