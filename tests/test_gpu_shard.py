"""GPU parity of the vocabulary-sharded draft (per-rank calls
dspark_markov_partials / dspark_markov_shard_summary /
dspark_markov_shard_select, G ranks issued on one device), through the C ABI.

The sharded draw is the single-device draw, so the oracle check is the
draft's own (teacher-forced per slot, same tolerances); in addition exactly
one rank owns every draw, and the sharded tokens match the unsharded draft
except at excused near-ties.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import log, upload, check_draft, sample_requests, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()
    return dv


def run_sharded(dv, spec, G, sample=None, seed=4, step=17):
    import torch
    label = f"{spec.name}/G{G}"
    log(f"[shard] {label}: R={spec.R} gamma={spec.gamma} V={spec.V} r={spec.r} dtype={spec.dtype}")
    inp = synth.generate(spec)
    dev, _ = upload(inp, spec)
    sd = dv.ShardedDraft(dev["U"], dev["W1"], dev["W2"], G)
    owners = []
    tok, p, lse = sd.draft(dev["anchor"], seed=seed, step=step, req_ids=dev["req_ids"],
                           owners=owners)
    ref = dv.markov_draft(dev["U"], dev["W1"], dv.prepack_w2(dev["W2"]), dev["anchor"], r=spec.r,
                          seed=seed, step=step, req_ids=dev["req_ids"])
    torch.cuda.synchronize()
    res = {"tokens": tok.cpu().numpy(), "p_draft": p.cpu().numpy(), "lse_draft": lse.cpu().numpy()}
    reqs = np.arange(spec.R) if sample is None else sample_requests(spec.R, sample)
    flips = check_draft(res, inp, seed, step, reqs, label)
    # exactly one owner per draw, and its id is the combined token
    for k, own in enumerate(owners):
        o = own.cpu().numpy()
        assert np.all((o >= 0).sum(axis=0) == 1), (label, k)
        assert np.array_equal(o.max(axis=0), res["tokens"][:, k]), (label, k)
        b = np.asarray(sd.bounds)
        rank = np.argmax(o >= 0, axis=0)
        assert np.all((b[rank] <= res["tokens"][:, k]) & (res["tokens"][:, k] < b[rank + 1])), label
    # against the unsharded draft: identical up to excused near-ties (the
    # first differing slot changes every later slot's condition, so compare
    # each request up to its first difference)
    ut = ref[0].cpu().numpy()
    diffs = 0
    for r in range(spec.R):
        d = np.nonzero(ut[r] != res["tokens"][r])[0]
        upto = d[0] if len(d) else spec.gamma
        diffs += len(d) > 0
        np.testing.assert_allclose(res["lse_draft"][r, :upto], ref[2].cpu().numpy()[r, :upto],
                                   rtol=0, atol=TOL)
        np.testing.assert_allclose(res["p_draft"][r, :upto], ref[1].cpu().numpy()[r, :upto],
                                   rtol=0, atol=TOL)
    assert diffs <= max(2, spec.R // 20), (label, diffs)
    log(f"[shard] {label}: ok; excused flips {flips}; requests differing from the unsharded draft "
        f"{diffs}")


SMALL = dict(R=20, gamma=5, V=3000, r=64, d=96, seed=41)


@pytest.mark.parametrize("G,dtype", [(2, "bf16"), (3, "bf16"), (8, "bf16"), (8, "f32"),
                                     (1, "bf16")])
def test_small_sharded_draft(dv, G, dtype):
    run_sharded(dv, synth.small_spec(f"shard_{dtype}", dtype=dtype, **SMALL), G)


def test_ragged_rank_vocab_and_shards(dv):
    spec = synth.small_spec("shard_ragged", R=33, gamma=4, V=2950, r=100, d=40, dtype="bf16",
                            seed=12)
    run_sharded(dv, spec, 5)


@pytest.mark.parametrize("name", ["qwen3", "dsv4"])
def test_full_size_eight_way(dv, name):
    run_sharded(dv, synth.CONFIGS[name], 8)
