"""dspark_markov_draft_confidence against dspark_markov_draft followed by
dspark_confidence, through the C ABI.

The fused call runs the confidence head inside each slot's GEMM launch (its
prologue) with the same wave code as the confidence kernel, so every output
must agree bit for bit with the two separate calls: tokens, draft
probabilities and log-normalisers, confidences, survivals and logits. The oracle parity of the
fused call is covered by the chain parity tests, whose steps use it.
Shapes: a single request and slot, ragged request counts and vocabularies,
bfloat16 and float32, hidden sizes and ranks that are not multiples of the
vector width (scalar dot products), inverse temperatures on and off; both
placements of the head (in the GEMM prologue when few of the GEMM's
workgroups carry a request, e.g. 64 requests over a 151936 vocabulary; a launch
of its own after the draft otherwise, e.g. 256 requests). A last test checks
the confidence call against the oracle at hidden sizes past one round of
the dot product's loads.
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


# (R, gamma, V, r, d, dtype, temperatures)
SHAPES = [(1, 1, 65, 32, 16, "bf16", False), (7, 5, 3000, 64, 96, "bf16", True),
          (33, 4, 2950, 96, 100, "bf16", True), (20, 6, 1000, 36, 48, "f32", False),
          (64, 7, 151936, 256, 2560, "bf16", True), (5, 16, 517, 100, 37, "f32", True),
          (40, 3, 151936, 64, 200, "f32", True), (256, 2, 129280, 256, 512, "bf16", False)]


@pytest.mark.parametrize("R,gamma,V,r,d,dtype,temps", SHAPES)
def test_fused_equals_two_calls(dv, R, gamma, V, r, d, dtype, temps):
    import torch
    log(f"[draft+conf] R={R} gamma={gamma} V={V} r={r} d={d} {dtype} temps={temps}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(R * 7919 + V)
    U = (torch.randn((R, gamma, V), generator=g) * 2.0).to(tdt).cuda()
    W1 = (torch.randn((V, r), generator=g) * 0.3).to(tdt).cuda()
    W2 = (torch.randn((r, V), generator=g) * 0.3).to(tdt).cuda()
    h = torch.randn((R, gamma, d), generator=g).to(tdt).cuda()
    w = (torch.randn((d + r,), generator=g) * 0.05).cuda()
    anchor = torch.randint(0, V, (R,), generator=g, dtype=torch.int32).cuda()
    inv = (torch.rand((gamma,), generator=g) * 2 + 0.25).cuda() if temps else None
    W2p = dv.prepack_w2(W2)
    b = 0.7
    # two calls
    tok, p, lse = dv.markov_draft(U, W1, W2p, anchor, r=r, seed=5, step=9)
    logit_a = torch.empty((R, gamma), dtype=torch.float32, device="cuda")
    conf_a, surv_a = dv.confidence(h, W1, anchor, tok, w, b, inv_temp=inv, logit=logit_a)
    # one call
    logit_b = torch.empty((R, gamma), dtype=torch.float32, device="cuda")
    out = dv.markov_draft_confidence(U, W1, W2p, anchor, h, w, b, r=r, inv_temp=inv, seed=5,
                                     step=9, logit=logit_b)
    torch.cuda.synchronize()
    ref = [t.cpu().numpy() for t in (tok, p, lse, conf_a, surv_a, logit_a)]
    got = [t.cpu().numpy() for t in (*out, logit_b)]
    for name, a, c in zip(("tokens", "p_draft", "lse_draft", "conf", "surv", "logit"), ref, got):
        assert np.array_equal(a.view(np.uint32), c.view(np.uint32)), name
    assert np.all(np.diff(got[4], axis=1) <= 0)       # survival never grows along a request
    log(f"[draft+conf] R={R} gamma={gamma} V={V}: bit-identical")


# hidden sizes past one round of the dot product's loads (512 16-byte chunks
# per wave): 520 (two chunk groups), 8200 (three rounds, the last with one
# chunk), a float32 row of 4100, and 8201 (not a multiple of the vector
# width: the scalar path)
@pytest.mark.parametrize("d,dtype", [(520, "bf16"), (8200, "bf16"), (4100, "f32"), (8201, "bf16")])
def test_confidence_long_hidden_rows_against_oracle(dv, d, dtype):
    import torch
    import oracle
    R, gamma, V, r = 6, 3, 700, 72
    log(f"[conf long d] R={R} gamma={gamma} d={d} {dtype}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(d)
    h = torch.randn((R, gamma, d), generator=g).to(tdt)
    W1 = (torch.randn((V, r), generator=g) * 0.3).to(tdt)
    w = torch.randn((d + r,), generator=g) * 0.05
    anchor = torch.randint(0, V, (R,), generator=g, dtype=torch.int32)
    tokens = torch.randint(0, V, (R, gamma), generator=g, dtype=torch.int32)
    b = -0.3
    logit = torch.empty((R, gamma), dtype=torch.float32, device="cuda")
    conf, surv = dv.confidence(h.cuda(), W1.cuda(), anchor.cuda(), tokens.cuda(), w.cuda(), b,
                               logit=logit)
    torch.cuda.synchronize()
    ref = oracle.confidence(h.float().numpy(), W1.float().numpy(), anchor.numpy(), tokens.numpy(),
                            w.numpy(), b)
    # fp32 sums of d + r products of size ~0.05 against the float64 oracle
    np.testing.assert_allclose(logit.cpu().numpy(), ref["logit"], rtol=0, atol=2e-4)
    np.testing.assert_allclose(conf.cpu().numpy(), ref["conf"], rtol=0, atol=5e-5)
    np.testing.assert_allclose(surv.cpu().numpy(), ref["surv"], rtol=0, atol=5e-5)
