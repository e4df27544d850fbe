"""C-ABI checks that need no GPU: the library loads, exports every function
include/dspark.h declares, rejects bad arguments on the host before touching
the device, and its host cost-table utility matches the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


def _lib():
    import draft_verify_sampling_markov_amd as dv
    if not os.path.exists(dv.LIB_PATH):
        pytest.skip("libdspark.so not built (run __graft_entry__.build())")
    return dv, dv.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    dv, lib = _lib()
    names = _declared()
    assert len(names) == 32
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(dv.EXPORTS) == names


def test_draft_path_switch_and_status_offset():
    dv, lib = _lib()
    prev = lib.dspark_set_draft_path(dv.DRAFT_PER_SLOT)
    assert prev == dv.DRAFT_AUTO
    assert lib.dspark_set_draft_path(7) == -1            # unknown value: DSPARK_EINVAL
    assert lib.dspark_set_draft_path(dv.DRAFT_RESIDENT) == dv.DRAFT_PER_SLOT
    assert lib.dspark_set_draft_path(dv.DRAFT_AUTO) == dv.DRAFT_RESIDENT
    R, V = 64, 151936
    off = lib.dspark_workspace_status_offset(R, V)
    ws = dv.workspace_bytes(dv.CALL_MARKOV_DRAFT, R, 7, V, 256)
    assert 0 < off and off % 256 == 0 and off + 4 <= ws
    assert lib.dspark_workspace_status_offset(0, V) == 0


def test_status_strings():
    dv, lib = _lib()
    for rc in range(0, -7, -1):
        s = dv.status_string(rc)
        assert s.startswith("DSPARK")
    assert "unknown" in dv.status_string(-99)


def test_workspace_sizes():
    dv, lib = _lib()
    R, g, V, r = 64, 7, 151936, 256
    n_t = -(-V // 64)
    assert dv.workspace_bytes(dv.CALL_MARKOV_DRAFT, R, g, V, r) >= n_t * R * 8
    assert dv.workspace_bytes(dv.CALL_VERIFY, R, g, V, r) > R * (g + 1) * 8
    assert dv.workspace_bytes(dv.CALL_VERIFY, 4096, 1, V, r) == 0   # R(g+1) > 4096
    assert dv.workspace_bytes(99, R, g, V, r) == 0
    assert dv.prepacked_w2_bytes(256, V, dv.BF16) == n_t * 8 * 4 * 64 * 8 * 2
    assert dv.prepacked_w2_bytes(300, V, dv.BF16) == 0
    assert dv.prepacked_w2_bytes(200, V, dv.F32) == 0


def test_host_validation_rejects_before_launch():
    dv, lib = _lib()
    EINVAL, EDTYPE, ETIER, ESIZE, EWS = -1, -2, -3, -4, -5
    p = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation first
    # markov_draft: bad dtype, bad sizes, null pointers, missing workspace
    assert lib.dspark_markov_draft(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 5, p, p, p, p, 1 << 30, None) == EDTYPE
    assert lib.dspark_markov_draft(p, p, p, p, 0, 0, None, p, 4, 17, 1024, 32, 0, p, p, p, p, 1 << 30, None) == ESIZE
    assert lib.dspark_markov_draft(p, p, p, p, 0, 0, None, p, 600, 7, 1024, 32, 0, p, p, p, p, 1 << 30, None) == ESIZE
    assert lib.dspark_markov_draft(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 129, 0, p, p, p, p, 1 << 30, None) == ESIZE
    assert lib.dspark_workspace_init(None, 256, None) == EINVAL
    assert lib.dspark_markov_draft(None, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, p, p, 1 << 30, None) == EINVAL
    assert lib.dspark_markov_draft(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, p, p, 8, None) == EWS
    assert lib.dspark_markov_draft(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, p, None, 1 << 30, None) == EWS
    # confidence
    assert lib.dspark_confidence(p, p, p, p, p, 0.0, None, 4, 7, 0, 1024, 32, 0, p, p, None, None) == ESIZE
    assert lib.dspark_confidence(p, None, p, p, p, 0.0, None, 4, 7, 64, 1024, 32, 0, p, p, None, None) == EINVAL
    # draft + confidence in one call: the checks of both
    dc = lib.dspark_markov_draft_confidence
    assert dc(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 5, p, p, 0.0, None, 64, p, p, p, p, p, None, p, 1 << 30, None) == EDTYPE
    assert dc(p, p, p, p, 0, 0, None, p, 4, 17, 1024, 32, 0, p, p, 0.0, None, 64, p, p, p, p, p, None, p, 1 << 30, None) == ESIZE
    assert dc(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, 0.0, None, 0, p, p, p, p, p, None, p, 1 << 30, None) == ESIZE
    assert dc(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, None, p, 0.0, None, 64, p, p, p, p, p, None, p, 1 << 30, None) == EINVAL
    assert dc(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, 0.0, None, 64, p, p, p, p, None, None, p, 1 << 30, None) == EINVAL
    assert dc(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, 0.0, None, 64, p, p, p, p, p, None, p, 8, None) == EWS
    # no-allocation draft: the draft's checks, then the array's size, before any device call
    na = lib.dspark_markov_draft_noalloc
    assert na(p, p, p, p, 0, 0, None, p, 4, 7, 1024, 32, 5, p, p, p, None) == EDTYPE
    assert na(p, p, p, p, 0, 0, None, p, 4, 17, 1024, 32, 0, p, p, p, None) == ESIZE
    assert na(p, p, p, p, 0, 0, None, None, 4, 7, 1024, 32, 0, p, p, p, None) == EINVAL
    assert na(p, p, p, p, 0, 0, None, p, 2048, 1, 151936, 256, 1, p, p, p, None) == EWS  # bf16
    # peak probes
    assert lib.dspark_probe_read(None, 1024, p, None) == EINVAL
    assert lib.dspark_probe_read(p, 1000, p, None) == ESIZE
    assert lib.dspark_probe_read(ctypes.c_void_p(24), 1024, p, None) == ESIZE
    assert lib.dspark_probe_mfma(None, 8, 8, None) == EINVAL
    assert lib.dspark_probe_mfma(p, 0, 8, None) == ESIZE
    assert lib.dspark_probe_mfma(p, 8, 0, None) == ESIZE
    assert lib.dspark_probe_mfma_flops(256, 512) == 256 * 4 * 512 * 8 * 16384
    # schedule + pack in one launch: the checks of both
    sp = lib.dspark_schedule_pack
    tiers = (ctypes.c_int32 * 2)(16, 32)
    bad_tiers = (ctypes.c_int32 * 2)(32, 16)
    assert sp(p, None, p, 32, 4, 7, 12, 3, 0, p, p, p, p, 1, tiers, 2, 32, p, p, p, p, p, None) == EINVAL
    assert sp(p, None, p, 32, 4, 7, 12, 0, 0, p, p, None, p, 1, tiers, 2, 32, p, p, p, p, p, None) == EINVAL
    assert sp(p, None, p, 32, 4, 7, 12, 0, 0, p, p, p, p, 1, tiers, 2, 31, p, p, p, p, p, None) == ESIZE
    assert sp(p, None, p, 3, 4, 7, 12, 0, 0, p, p, p, p, 1, tiers, 2, 32, p, p, p, p, p, None) == ESIZE
    assert sp(p, None, p, 32, 4, 7, 12, 0, 0, p, p, p, p, 1, bad_tiers, 2, 32, p, p, p, p, p, None) == ETIER
    # schedule
    assert lib.dspark_schedule_topb(p, None, p, 32, 4, 7, 12, 3, 0, p, p, None) == EINVAL
    assert lib.dspark_schedule_topb(p, None, p, 3, 4, 7, 12, 0, 0, p, p, None) == ESIZE
    assert lib.dspark_schedule_topb(None, None, p, 32, 4, 7, 12, 0, 0, p, p, None) == EINVAL
    # pack: tiers
    tiers = (ctypes.c_int32 * 3)(16, 8, 32)
    assert lib.dspark_pack_ragged(p, p, None, 4, 7, tiers, 3, 32, p, p, p, p, p, None) == ETIER
    tiers = (ctypes.c_int32 * 3)(8, 16, 32)
    assert lib.dspark_pack_ragged(p, p, None, 4, 7, tiers, 0, 32, p, p, p, p, p, None) == ETIER
    assert lib.dspark_pack_ragged(p, p, None, 4, 7, tiers, 3, 31, p, p, p, p, p, None) == ESIZE
    # verify
    args = [p, 32, p, p, p, p, p, p, p, p, None, 2, 0, 0, None, p, 4, 7, 1024, 32, 0, p, p, p, None, p, 1 << 30, None]
    assert lib.dspark_verify(*args) == EINVAL          # cap-accept needs win_len
    args[11] = 7
    assert lib.dspark_verify(*args) == EINVAL          # bad mode
    args[11] = 0
    args[1] = 31
    assert lib.dspark_verify(*args) == ESIZE           # M_cap < R (gamma + 1)
    args[1] = 32
    args[-2] = 16
    assert lib.dspark_verify(*args) == EWS
    # advance: sizes, history depth, missing buffers
    assert lib.dspark_advance(p, p, p, 0, 7, None, None, None, 0, None) == ESIZE
    assert lib.dspark_advance(p, p, p, 4, 17, None, None, None, 0, None) == ESIZE
    assert lib.dspark_advance(p, p, p, 4, 7, None, p, p, 9, None) == ESIZE
    assert lib.dspark_advance(p, None, p, 4, 7, None, None, None, 0, None) == EINVAL
    assert lib.dspark_advance(p, p, p, 4, 7, None, None, p, 2, None) == EINVAL
    # observe: sizes, bins, missing buffers, short block
    assert lib.dspark_observe_words(4, 7, 0) == 0 and lib.dspark_observe_words(4, 7, 33) == 0
    assert lib.dspark_observe_words(4, 17, 8) == 0
    assert lib.dspark_observe_words(4, 7, 8) == 8 + 3 * 8 + 3 * 4 + 2 * 7 * 8 * 3
    assert lib.dspark_observe(p, p, p, p, p, p, 4, 7, 0, p, 1 << 20, None) == ESIZE
    assert lib.dspark_observe(p, p, p, p, None, p, 4, 7, 8, p, 1 << 20, None) == EINVAL
    assert lib.dspark_observe(p, p, p, p, p, p, 4, 7, 8, p, 10, None) == EWS
    # analytic acceptance: sizes, pointers, workspace
    acc = [p, 32, p, p, p, p, p, p, p, 4, 7, 1024, 32, 0, p, p, 1 << 30, None]
    assert lib.dspark_analytic_accept(*acc[:9], 4, 7, 1024, 32, 7, *acc[14:]) == EDTYPE
    acc2 = list(acc); acc2[1] = 31
    assert lib.dspark_analytic_accept(*acc2) == ESIZE
    acc2 = list(acc); acc2[14] = None
    assert lib.dspark_analytic_accept(*acc2) == EINVAL
    acc2 = list(acc); acc2[16] = 64
    assert lib.dspark_analytic_accept(*acc2) == EWS
    assert dv.workspace_bytes(dv.CALL_ANALYTIC_ACCEPT, 64, 7, 151936, 256) > 512 * 2374 * 4
    # sharded draft: sizes, rank range, shard range, workspace
    assert lib.dspark_markov_shard_partials(p, 1024, p, p, p, 1, 4, 2000, 1024, 32, 0, p, 1 << 30, None) == ESIZE
    assert lib.dspark_markov_shard_partials(p, 1024, None, p, p, 1, 4, 512, 1024, 32, 0, p, 1 << 30, None) == EINVAL
    assert lib.dspark_markov_shard_partials(p, 1024, p, p, p, 1, 4, 512, 1024, 32, 0, p, 64, None) == EWS
    assert lib.dspark_markov_shard_summary(p, 1 << 30, 0, 100, p, None) == ESIZE
    assert lib.dspark_markov_shard_summary(None, 1 << 30, 4, 100, p, None) == EINVAL
    assert lib.dspark_markov_shard_summary(p, 16, 4, 100, p, None) == EWS
    sel = [p, 1024, p, p, p, 1, p, p, 2, 0, 0, 0, 0, None, p, 1, 4, 512, 1024, 32, 0, p, p, p, 1, None]
    bad = list(sel); bad[9] = 2                      # g >= G
    assert lib.dspark_markov_shard_select(*bad) == ESIZE
    bad = list(sel); bad[10] = 600                   # v0 + V_g > V
    assert lib.dspark_markov_shard_select(*bad) == ESIZE
    bad = list(sel); bad[7] = None                   # summaries
    assert lib.dspark_markov_shard_select(*bad) == EINVAL
    bad = list(sel); bad[20] = 9                     # dtype
    assert lib.dspark_markov_shard_select(*bad) == EDTYPE
    # temperature fit: sizes, pointers, workspace
    assert lib.dspark_sts_workspace_bytes(100, 7, 0, 16) == 0
    assert lib.dspark_sts_workspace_bytes(100, 7, 16, 33) == 0
    assert lib.dspark_sts_workspace_bytes(100, 7, 16, 16) >= 100 * 4 + 16 * 16 * 3 * 8
    assert lib.dspark_sts_fit(p, p, None, 100, 17, p, 16, 16, p, p, p, 1 << 20, None) == ESIZE
    assert lib.dspark_sts_fit(p, None, None, 100, 7, p, 16, 16, p, p, p, 1 << 20, None) == EINVAL
    assert lib.dspark_sts_fit(p, p, None, 100, 7, p, 16, 16, p, p, p, 64, None) == EWS
    # prepack
    assert lib.dspark_prepack_w2(p, 32, 1024, 1, p, 10, None) == EWS
    assert lib.dspark_prepack_w2(p, 32, 1024, 3, p, 1 << 30, None) == EDTYPE


@pytest.mark.parametrize("name", ["tiny", "qwen3", "dsv4", "mixed", "long"])
def test_cost_table_matches_oracle(name):
    dv, lib = _lib()
    sp = synth.CONFIGS[name]
    raw = synth.raw_step_time(sp)
    got = dv.cost_table_prepare(raw, sp.tiers, sp.staircase)
    ref = oracle.cost_table_prepare(raw, sp.tiers, sp.staircase)
    assert got.tolist() == ref
    assert got.shape[0] == sp.M_max + 1


@pytest.mark.parametrize("seed", range(6))
def test_cost_table_random_curves_match_oracle(seed):
    """Noisy, non-monotone curves with NaN, negative and infinite entries, and
    tier lists that reach past M_max, in both table shapes."""
    dv, lib = _lib()
    rng = np.random.default_rng(seed)
    M_max = int(rng.integers(0, 300))
    raw = rng.uniform(-1e-3, 5e-3, M_max + 1)
    for bad in (np.nan, np.inf, -np.inf, 0.0):
        raw[rng.integers(0, M_max + 1, 3)] = bad
    n = int(rng.integers(1, 33))
    tiers = np.unique(rng.integers(1, 2 * M_max + 3, n)).tolist()
    for staircase in (False, True):
        got = dv.cost_table_prepare(raw.tolist(), tiers, staircase)
        ref = oracle.cost_table_prepare(raw.tolist(), tiers, staircase)
        assert got.tolist() == ref, (seed, staircase)


def test_cost_table_rejects_bad_tiers():
    dv, lib = _lib()
    with pytest.raises(dv.DsparkError):
        dv.cost_table_prepare([1.0, 2.0, 3.0], [2, 1], True)
    with pytest.raises(dv.DsparkError):
        dv.cost_table_prepare([1.0, 2.0, 3.0], [], True)
