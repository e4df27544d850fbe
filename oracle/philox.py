"""Philox4x64-10 counter-based generator, written from its published definition
(Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
SC'11): a 4-word (64-bit) counter, a 2-word key, ten rounds of the Philox
S-box (two 64x64 -> 128-bit multiplies whose high halves are xored into the
other words with the round key), and a Weyl increment of the key between rounds.

The method samples its drafts left to right and verifies them by rejection
sampling (DSpark digest, "Architecture (drafter)"; the stream is keyed by
(seed, request, position)). Counter layout used here:

    counter = (k, req_id, step, 0)      k = slot 1..gamma+1 within the block
    key     = (seed, 0)

and the four 64-bit output words serve four purposes at slot k:

    word 0  draft sample          word 1  accept test
    word 2  residual resample     word 3  bonus sample

A 64-bit word x maps to the uniform u = (x >> 40) * 2**-24 in [0, 1 - 2**-24],
exact in float32 (our own mapping, not a vendor one).

Pure-Python integers: slow and obviously correct.
"""
from __future__ import annotations

from typing import Iterable, Sequence, Tuple

import numpy as np

MASK64 = (1 << 64) - 1

# Multipliers and Weyl key increments of Philox4x64 (SC'11 paper).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15   # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B   # sqrt(3) - 1

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_RESIDUAL = 2
PURPOSE_BONUS = 3


def _mulhilo(a: int, b: int) -> Tuple[int, int]:
    p = a * b
    return (p >> 64) & MASK64, p & MASK64


def philox4x64_10(counter: Sequence[int], key: Sequence[int]) -> Tuple[int, int, int, int]:
    """One Philox4x64-10 block: returns four 64-bit words for (counter, key)."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform24(word: int) -> float:
    """Top 24 bits of a 64-bit word as a float in [0, 1 - 2**-24]."""
    return float(int(word) >> 40) * (2.0 ** -24)


def uniforms(seed: int, step: int, req_id: int, k: int) -> Tuple[float, float, float, float]:
    """The four uniforms (draft, accept, residual, bonus) of slot k of a request."""
    words = philox4x64_10((k, req_id, step, 0), (seed, 0))
    return tuple(uniform24(w) for w in words)  # type: ignore[return-value]


def uniform(seed: int, step: int, req_id: int, k: int, purpose: int) -> float:
    return uniforms(seed, step, req_id, k)[purpose]
