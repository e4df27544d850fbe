"""Pins of the oracle's ragged pack: hand-computed cu_seqlens and the pages'
worked examples (tests/golden/pack_tier_examples.json)."""
import json
import os

import numpy as np

from oracle.pack import pack_ragged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_tier_examples.json")


def test_hand_example():
    anchor = [10, 20, 30]
    tokens = np.array([[11, 12, 13], [21, 22, 23], [31, 32, 33]])
    out = pack_ragged(anchor, tokens, [2, 0, 3], tiers=[4, 8, 12], M_cap=12)
    assert out["cu_seqlens"] == [0, 3, 4, 8]
    assert out["M"] == 8 and out["M_pad"] == 8
    assert out["packed_tokens"] == [10, 11, 12, 20, 30, 31, 32, 33, 0, 0, 0, 0]
    assert out["packed_req"] == [0, 0, 0, 1, 2, 2, 2, 2, -1, -1, -1, -1]
    assert out["packed_slot"] == [0, 1, 2, 0, 0, 1, 2, 3, -1, -1, -1, -1]


def test_static_is_full_block_and_overflow_flag():
    anchor = [1, 2]
    tokens = np.array([[3, 4], [5, 6]])
    out = pack_ragged(anchor, tokens, None, tiers=[4], M_cap=6)
    assert out["cu_seqlens"] == [0, 3, 6] and out["M"] == 6 and out["M_pad"] == -1


def test_golden_tier_rounding():
    with open(GOLDEN) as f:
        g = json.load(f)
    for case in g["tier_rounding"]:
        M = case["M"]
        # R requests with windows summing to M - R
        R = 1
        tokens = np.zeros((R, M - R), dtype=np.int64)
        out = pack_ragged([0] * R, tokens, [M - R], case["tiers"], M_cap=M)
        assert out["M"] == M and out["M_pad"] == case["M_pad"]
    for case in g["max_capture"]:
        gamma, R = case["num_speculative_tokens"], case["max_num_seq"]
        out = pack_ragged([0] * R, np.zeros((R, gamma), dtype=np.int64), None,
                          [case["capture"]], M_cap=case["capture"])
        assert out["M"] == case["capture"] == out["M_pad"]
