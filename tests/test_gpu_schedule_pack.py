"""dspark_schedule_pack against dspark_schedule_topb followed by
dspark_pack_ragged, through the C ABI.

The fused launch runs the same scheduler and pack code in one workgroup, with
the windows passed through shared memory, so every output must be identical:
windows, K, cu_seqlens, packed tokens / requests / slots and the totals. The
oracle parity of the fused call is covered by the chain parity tests, whose
steps use it. Cases: the three scheduler modes, a stale budget array, full
blocks (pack_windows off) and scheduled windows, an empty budget, the row
limit R (gamma + 1) = 4096, and a total that exceeds every tier. The
full-block pack (no window array) must also equal the scanned pack of
windows that are all gamma. A seeded randomised test checks the scheduler
call itself against the oracle over 120 cases (ties, flat rows, NaN and
out-of-range survivals, zero cost-table entries, all three modes).
"""
import numpy as np
import pytest

from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dv():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_markov_amd as dv
    dv.load_library()
    return dv


def _case(dv, R, gamma, V, B, mode, K_fixed, stale, windows, tiers, seed):
    import torch
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.3, 1.0, (R, gamma)).astype(np.float32)
    surv = torch.from_numpy(np.cumprod(c, axis=1)).cuda()
    budget = torch.from_numpy(np.cumprod(rng.uniform(0.3, 1.0, (R, gamma)), axis=1)
                              .astype(np.float32)).cuda() if stale else None
    M_max = R * (gamma + 1)
    raw = 1e-3 + 4e-6 * np.arange(M_max + 1, dtype=np.float64)
    sps = torch.from_numpy(dv.cost_table_prepare(raw, tiers, True).astype(np.int32)).cuda()
    anchor = torch.from_numpy(rng.integers(0, V, R).astype(np.int32)).cuda()
    tokens = torch.from_numpy(rng.integers(0, V, (R, gamma)).astype(np.int32)).cuda()
    M_cap = M_max
    win_a, K_a = dv.schedule_topb(surv, sps, B_cap=B, mode=mode, K_fixed=K_fixed, surv_budget=budget)
    pack_a = dv.pack_ragged(anchor, tokens, win_a if windows else None, tiers, M_cap)
    (win_b, K_b), pack_b = dv.schedule_pack(surv, sps, anchor, tokens, tiers, M_cap, B_cap=B,
                                            mode=mode, K_fixed=K_fixed, surv_budget=budget,
                                            pack_windows=windows)
    torch.cuda.synchronize()
    assert np.array_equal(win_a.cpu().numpy(), win_b.cpu().numpy())
    assert int(K_a.item()) == int(K_b.item())
    for k in pack_a:
        assert np.array_equal(pack_a[k].cpu().numpy(), pack_b[k].cpu().numpy()), k
    return int(K_b.item()), pack_b["totals"].cpu().numpy()


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("windows", [True, False])
def test_fused_equals_two_calls(dv, mode, windows):
    tiers = [8, 16, 32, 64, 128, 256, 512]
    for R, gamma, B, stale, seed in [(64, 7, 448, False, 1), (64, 7, 100, True, 2),
                                     (13, 16, 50, False, 3), (1, 1, 1, False, 4),
                                     (64, 7, 0, False, 5)]:
        K, tot = _case(dv, R, gamma, 1000, B, mode, 37, stale, windows, tiers, seed)
        log(f"[sched+pack] mode={mode} windows={windows} R={R} gamma={gamma} B={B}: K={K} "
            f"totals={tot.tolist()}")


def test_row_limit_and_tier_overflow(dv):
    # R (gamma + 1) = 4096 packed rows; tiers that stop below the full block
    K, tot = _case(dv, 256, 15, 5000, 3840, 0, 0, False, True, [512, 1024, 2048, 4096], 7)
    assert tot[0] <= 4096
    K, tot = _case(dv, 256, 15, 5000, 3840, 0, 0, False, False, [512, 1024, 2048], 8)
    assert tot.tolist() == [4096, -1]


@pytest.mark.parametrize("R,gamma,extra", [(1, 1, 0), (64, 7, 0), (13, 16, 37), (256, 15, 0),
                                           (2048, 1, 5)])
def test_full_block_pack_equals_scanned_pack(dv, R, gamma, extra):
    # win_len NULL takes the index-arithmetic path; an explicit array of gamma
    # windows takes the scan-and-search path: every output must agree
    import torch
    rng = np.random.default_rng(R * 31 + gamma)
    V = 5000
    anchor = torch.from_numpy(rng.integers(0, V, R).astype(np.int32)).cuda()
    tokens = torch.from_numpy(rng.integers(0, V, (R, gamma)).astype(np.int32)).cuda()
    full = torch.full((R,), gamma, dtype=torch.int32, device="cuda")
    M_cap = R * (gamma + 1) + extra
    tiers = [8, 64, 512, 4096]
    a = dv.pack_ragged(anchor, tokens, None, tiers, M_cap)
    b = dv.pack_ragged(anchor, tokens, full, tiers, M_cap)
    torch.cuda.synchronize()
    for k in a:
        assert np.array_equal(a[k].cpu().numpy(), b[k].cpu().numpy()), k
    assert a["totals"].cpu().numpy().tolist()[0] == R * (gamma + 1)
    log(f"[pack] full blocks R={R} gamma={gamma} M_cap={M_cap}: index path == scanned path")


def _random_survivals(rng, kind, R, gamma):
    """Survival arrays of six kinds: products of random confidences, four
    distinct levels (many ties), one value everywhere, zeros and ones, values
    out of [0, 1] with NaNs, and values a few quantisation steps (2^-20) apart."""
    if kind == 0:
        return np.cumprod(rng.uniform(0.05, 1.0, (R, gamma)), axis=1).astype(np.float32)
    if kind == 1:
        lv = np.array([1.0, 0.75, 0.5, 0.25], np.float32)
        return np.sort(lv[rng.integers(0, 4, (R, gamma))], axis=1)[:, ::-1].copy()
    if kind == 2:
        return np.full((R, gamma), np.float32(rng.uniform(0, 1)), np.float32)
    if kind == 3:
        return np.sort(rng.choice(np.array([0.0, 1.0], np.float32), (R, gamma)), axis=1)[:, ::-1].copy()
    if kind == 4:
        a = rng.uniform(-0.5, 1.5, (R, gamma)).astype(np.float32)
        a[rng.random((R, gamma)) < 0.05] = np.nan
        return a
    return (rng.uniform(0.2, 0.9) + rng.integers(-3, 4, (R, gamma)) * 2.0 ** -20).astype(np.float32)


def test_randomised_scheduler_against_oracle(dv):
    """120 seeded random cases of the scheduler call against the oracle: request
    counts up to 512 and gamma up to 16 (keys up to the 4096-row limit), the
    three modes, random budgets, stale budget arrays, cost tables with zero
    entries, and the survival kinds above (ties at every radix digit, flat
    rows, NaN and out-of-range values)."""
    import torch
    import oracle
    rng = np.random.default_rng(2024)
    for case in range(120):
        while True:
            gamma = int(rng.integers(1, 17))
            R = int(rng.integers(1, 513))
            if R * (gamma + 1) <= 4096:
                break
        kind = case % 6
        surv = _random_survivals(rng, kind, R, gamma)
        M_max = min(4096, R * (gamma + 1) + int(rng.integers(0, 64)))
        m = np.arange(M_max + 1)
        sps = np.maximum(1, 1e6 / (1.0 + 0.002 * m + rng.uniform(0, 0.01, M_max + 1))).astype(np.uint32)
        if case % 7 == 0:
            sps[rng.integers(0, M_max + 1, 5)] = 0
        B_cap = int(rng.integers(0, R * gamma + 6))
        mode = int(rng.integers(0, 3))
        K_fixed = int(rng.integers(0, R * gamma + 3))
        budget = (np.clip(surv * rng.uniform(0.5, 1.2), 0, 1).astype(np.float32)
                  if case % 5 == 0 else None)
        ref = oracle.schedule_topb(surv, [int(x) for x in sps], B_cap, mode, K_fixed, budget)
        win, K = dv.schedule_topb(
            torch.from_numpy(surv).cuda(), torch.from_numpy(sps.view(np.int32)).cuda(), B_cap=B_cap,
            mode=mode, K_fixed=K_fixed,
            surv_budget=None if budget is None else torch.from_numpy(budget).cuda())
        torch.cuda.synchronize()
        label = f"case {case}: kind {kind} R {R} gamma {gamma} mode {mode} B {B_cap}"
        assert win.cpu().numpy().tolist() == list(ref["win_len"]), label
        assert int(K.cpu()[0]) == ref["K"], label
    log("[schedule] 120 random cases equal the oracle")
