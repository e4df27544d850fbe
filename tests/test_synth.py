"""Synthetic input recipes: shapes, determinism, bf16 rounding."""
import numpy as np

import synth


def test_bf16_rounding_matches_bit_definition():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0, -2.0, 1.00390625, 1.01171875, 3.0e-39], dtype=np.float32)])
    assert np.array_equal(synth.to_bf16_bits(x), synth._to_bf16_bits_np(x))
    # ties go to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert synth.to_bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80
    assert synth.to_bf16_bits(np.array([1.01171875], np.float32))[0] == 0x3F82
    assert np.array_equal(synth.bf16_bits_to_f32(synth.to_bf16_bits(x[:5])),
                          synth.bf16_bits_to_f32(synth.to_bf16_bits(x[:5])))


def test_generate_shapes_and_determinism():
    sp = synth.small_spec(R=5, gamma=3, V=300, r=8, d=12, dtype="bf16")
    a, b = synth.generate(sp), synth.generate(sp)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["U"].shape == (5, 3, 300) and a["U"].dtype == np.uint16
    assert a["target"].shape == (5, 4, 300)
    assert a["W1"].shape == (300, 8) and a["W2"].shape == (8, 300)
    assert a["h"].shape == (5, 3, 12) and a["w"].shape == (20,)
    assert a["raw_T"].shape == (sp.M_max + 1,)
    assert a["anchor"].min() >= 0 and a["anchor"].max() < 300


def test_named_workloads_match_their_shapes():
    c = synth.CONFIGS
    assert (c["qwen3"].R, c["qwen3"].gamma, c["qwen3"].V, c["qwen3"].r, c["qwen3"].d) == (64, 7, 151936, 256, 2560)
    assert (c["dsv4"].R, c["dsv4"].gamma, c["dsv4"].V) == (256, 5, 129280)
    assert c["dsv4"].tiers[-1] == c["dsv4"].M_max == 1536
    assert (c["long"].R, c["long"].gamma) == (128, 15)
    assert c["long"].budgets == (128, 256, 512, 1024, 1920)
    assert c["tiny"].dtype == "f32" and c["tiny"].budgets == (12,)


def test_draft_noise_follows_the_recipe():
    sp = synth.small_spec(R=6, gamma=4, V=20000, r=8, d=4, dtype="f32",
                          noise=("class", (0.3, 0.8, 1.5)), zipf_s=None)
    inp = synth.generate(sp)
    diff = inp["U"] - inp["target"][:, :4, :]
    for r in range(6):
        assert abs(diff[r].std() - (0.3, 0.8, 1.5)[r % 3]) < 0.02
