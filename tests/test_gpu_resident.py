"""GPU parity of the resident-W2 draft kernel (dspark_set_draft_path
RESIDENT), through the C ABI.

The whole chain (draft + confidence, schedule, pack, verify) runs with the
draft as one launch that keeps W2 on chip for every slot, and every request
of every stage is compared with the oracle, teacher-forced as in
test_gpu_parity.py. The workspace's barrier error word must stay 0, and the
decode loop (graph-captured) must replay the eager loop bit for bit.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import log, run_and_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()          # raises if the HIP library is missing
    prev = dv.set_draft_path(dv.DRAFT_RESIDENT)
    yield dv
    dv.set_draft_path(prev)


def _status(dv, ch):
    return dv.draft_status(ch.ws_draft, ch.R, ch.V)


# eligible shapes (bfloat16, rank 256, V a multiple of 8): one and two
# staging phases, ragged request blocks, vocabularies smaller than the grid
@pytest.mark.parametrize("R,gamma,V", [(40, 4, 3000), (1, 1, 64), (37, 5, 1000), (200, 3, 2048),
                                       (256, 2, 4096), (129, 2, 16384)])
def test_small_resident_chain(dv, R, gamma, V):
    sp = synth.small_spec("resident", R=R, gamma=gamma, V=V, r=256, d=48, dtype="bf16", seed=R + V,
                          W_std=0.05)
    inp = synth.generate(sp)
    for vmode in ("static", "compact", "cap_accept"):
        res, ch = run_and_check(dv, sp, vmode, inp=inp, check_draft_conf=vmode == "static")
        assert _status(dv, ch) == 0


@pytest.mark.parametrize("name,vmode", [("qwen3", "static"), ("mixed", "cap_accept"),
                                        ("dsv4", "compact"), ("long", "compact")])
def test_full_size_resident_chain(dv, name, vmode):
    res, ch = run_and_check(dv, synth.CONFIGS[name], vmode)
    assert _status(dv, ch) == 0


def test_resident_decode_graph_replays(dv):
    # the resident launch inside a captured decode step: every replay equals
    # the eager loop, and each step is checked against the oracle
    from tests.test_gpu_decode import run_loop
    spec = synth.small_spec("resident_decode", R=24, gamma=4, V=4000, r=256, d=40, dtype="bf16",
                            seed=3, W_std=0.05, b=0.5)
    run_loop(dv, spec, "compact", 2, 5)


def test_resident_matches_per_slot_tokens(dv):
    # the two kernels merge partials in different orders, so only draws that
    # fall within rounding of a cumulative boundary may differ
    import torch
    sp = synth.small_spec("resident_cmp", R=64, gamma=5, V=8192, r=256, d=32, dtype="bf16", seed=8,
                          W_std=0.05)
    inp = synth.generate(sp)
    out = {}
    for path in (dv.DRAFT_RESIDENT, dv.DRAFT_PER_SLOT):
        dv.set_draft_path(path)
        res, ch = run_and_check(dv, sp, "static", inp=inp)
        out[path] = res
    dv.set_draft_path(dv.DRAFT_RESIDENT)
    a, b = out[dv.DRAFT_RESIDENT], out[dv.DRAFT_PER_SLOT]
    same = np.all(a["tokens"] == b["tokens"], axis=1)
    log(f"[resident] {same.sum()} of {sp.R} requests draft identical tokens on both kernels")
    assert same.sum() >= sp.R - 2
    np.testing.assert_allclose(a["conf"][same], b["conf"][same], rtol=0, atol=0)
