"""Pins of the oracle's Philox4x64-10 against numpy's independent implementation
of the same published generator, plus range and uniformity checks."""
import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4x64_10, uniform24, uniforms

M64 = (1 << 64) - 1


def _numpy_block(counter, key):
    # numpy's Philox increments its 256-bit counter before producing a block,
    # so start it one below the wanted counter (with borrow across words).
    c = [int(x) & M64 for x in counter]
    v = c[0] | (c[1] << 64) | (c[2] << 128) | (c[3] << 192)
    v = (v - 1) % (1 << 256)
    prev = [(v >> (64 * i)) & M64 for i in range(4)]
    g = np.random.Philox(counter=np.array(prev, dtype=np.uint64),
                         key=np.array([int(k) & M64 for k in key], dtype=np.uint64))
    return [int(x) for x in g.random_raw(4)]


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((7, 3, 0, 0), (0, 0)),
    ((1, 2, 3, 4), (123456789, 987654321)),
    ((0, 7, 9, 1 << 63), (M64, 5)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((15, 255, 1 << 40, 0), (0xDEADBEEF, 0)),
]


@pytest.mark.parametrize("counter,key", CASES)
def test_matches_numpy_philox(counter, key):
    assert list(philox4x64_10(counter, key)) == _numpy_block(counter, key)


def test_matches_numpy_philox_random_counters():
    rng = np.random.default_rng(5)
    for _ in range(200):
        counter = [int(x) for x in rng.integers(0, 1 << 63, size=4, dtype=np.int64)]
        key = [int(x) for x in rng.integers(0, 1 << 63, size=2, dtype=np.int64)]
        assert list(philox4x64_10(counter, key)) == _numpy_block(counter, key)


def test_uniform24_range_and_exactness():
    assert uniform24(0) == 0.0
    assert uniform24(M64) == 1.0 - 2.0 ** -24
    assert uniform24(1 << 63) == 0.5
    for w in (12345678901234567, M64 - 99, 1 << 40):
        u = uniform24(w)
        assert float(np.float32(u)) == u          # exact in float32
        assert 0.0 <= u < 1.0


def test_uniforms_are_uniform_and_distinct_by_purpose():
    n = 4000
    us = np.array([uniforms(0, 0, rid, 1) for rid in range(n)])
    for p in range(4):
        assert stats.kstest(us[:, p], "uniform").pvalue > 1e-3
    # the four purposes are different streams
    assert np.corrcoef(us.T)[np.triu_indices(4, 1)].max() < 0.1
    # distinct slots, steps and seeds give different blocks
    assert uniforms(0, 0, 3, 1) != uniforms(0, 0, 3, 2)
    assert uniforms(0, 0, 3, 1) != uniforms(0, 1, 3, 1)
    assert uniforms(0, 0, 3, 1) != uniforms(1, 0, 3, 1)
