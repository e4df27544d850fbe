"""dspark_markov_draft_noalloc (the draft on the library's device scratch
array) against dspark_markov_draft (caller workspace), through the C ABI.

Two calls in a row, the second with a smaller input (the array keeps the first
call's partials where the second call's counters lie, so the call's own
clearing is what makes it correct); tokens, probabilities and log-sum-exps
must be bit-identical to the workspace call's. Also: both draft kernels,
replays of a captured graph, and the rejection of sizes beyond the array.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()
    return dv


def _both(dv, sp, seed=3, step=11):
    import torch
    inp = synth.generate(sp, with_h=False)
    dev, _ = upload({**inp, "h": np.zeros((1, 1, 1), dtype=inp["U"].dtype)}, sp)
    W2p = dv.prepack_w2(dev["W2"])
    ref = dv.markov_draft(dev["U"], dev["W1"], W2p, dev["anchor"], r=sp.r, seed=seed, step=step,
                          req_ids=dev["req_ids"])
    got = dv.markov_draft_noalloc(dev["U"], dev["W1"], W2p, dev["anchor"], r=sp.r, seed=seed,
                                  step=step, req_ids=dev["req_ids"])
    torch.cuda.synchronize()
    for a, b, name in zip(ref, got, ("tokens", "p_draft", "lse_draft")):
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), (sp.name, name)
    return dev, W2p


@pytest.mark.parametrize("path", ["per_slot", "resident"])
def test_noalloc_matches_workspace_call_large_then_small(dv, path):
    prev = dv.set_draft_path(dv.DRAFT_PER_SLOT if path == "per_slot" else dv.DRAFT_RESIDENT)
    try:
        big = synth.small_spec("noalloc_big", R=200, gamma=4, V=65536, r=256, d=8, dtype="bf16",
                               seed=1, W_std=0.05)
        small = synth.small_spec("noalloc_small", R=20, gamma=5, V=3000, r=64, d=8, dtype="bf16",
                                 seed=2)
        _both(dv, big)
        _both(dv, small)
        _both(dv, big)
        log(f"[noalloc] {path}: matches the workspace call (large, small, large)")
    finally:
        dv.set_draft_path(prev)


def test_noalloc_graph_replays(dv):
    import torch
    sp = synth.small_spec("noalloc_graph", R=33, gamma=3, V=4000, r=32, d=8, dtype="bf16", seed=4)
    dev, W2p = _both(dv, sp)
    R, g = sp.R, sp.gamma
    out = (torch.empty((R, g), dtype=torch.int32, device="cuda"),
           torch.empty((R, g), dtype=torch.float32, device="cuda"),
           torch.empty((R, g), dtype=torch.float32, device="cuda"))
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        dv.markov_draft_noalloc(dev["U"], dev["W1"], W2p, dev["anchor"], r=sp.r, seed=5,
                                step_dev=step, req_ids=dev["req_ids"], out=out)
    for s in range(3):
        step.fill_(s)
        gr.replay()
        torch.cuda.synchronize()
        ref = dv.markov_draft(dev["U"], dev["W1"], W2p, dev["anchor"], r=sp.r, seed=5, step=s,
                              req_ids=dev["req_ids"])
        torch.cuda.synchronize()
        for a, b in zip(ref, out):
            assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), s


def test_noalloc_rejects_sizes_beyond_the_array(dv):
    lib = dv.load_library()
    assert lib.dspark_noalloc_scratch_bytes() == 8 << 20
    need = dv.workspace_bytes(dv.CALL_MARKOV_DRAFT, 2048, 1, 151936, 256)
    assert need > lib.dspark_noalloc_scratch_bytes()
    # host-side check: nothing is launched, so the pointers are never read
    rc = lib.dspark_markov_draft_noalloc(1, 1, 1, 1, 0, 0, None, 1, 2048, 1, 151936, 256,
                                         dv.BF16, 1, 1, 1, None)
    assert rc == -5   # DSPARK_EWORKSPACE
