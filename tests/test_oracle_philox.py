"""Pins of the oracle's Philox4x64-10 against numpy's independent implementation."""
import numpy as np
import pytest

from oracle.philox import philox4x64_10, uniforms

MASK = (1 << 64) - 1


def _numpy_block(counter, key):
    # numpy's Philox increments its 256-bit counter before producing a block, so the
    # block for counter c is the first output of a generator started at c - 1.
    v = sum(int(x) << (64 * i) for i, x in enumerate(counter))
    v = (v - 1) % (1 << 256)
    start = np.array([(v >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=start, key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


def test_philox_matches_numpy_random_counters():
    rng = np.random.default_rng(1234)
    for _ in range(300):
        ctr = tuple(int(x) for x in rng.integers(0, 2**64, size=4, dtype=np.uint64))
        key = tuple(int(x) for x in rng.integers(0, 2**64, size=2, dtype=np.uint64))
        assert philox4x64_10(ctr, key) == _numpy_block(ctr, key)


@pytest.mark.parametrize("ctr,key", [((0, 0, 0, 0), (0, 0)),
                                     ((MASK, MASK, MASK, MASK), (MASK, MASK)),
                                     ((3, 17, 0, 0), (0, 0)),
                                     ((8, 255, 7, 0), (42, 0))])
def test_philox_edge_counters(ctr, key):
    assert philox4x64_10(ctr, key) == _numpy_block(ctr, key)


def test_uniforms_layout_and_range():
    seen = set()
    for seed in (0, 1, 2**40 + 3):
        for b in range(5):
            for j in range(9):
                for off in (0, 1, 77):
                    ua, us = uniforms(seed, b, j, off)
                    w = philox4x64_10((j, b, off, 0), (seed, 0))
                    assert ua == (w[0] >> 40) / 2**24 and us == (w[1] >> 40) / 2**24
                    for u in (ua, us):
                        assert 0.0 <= u <= 1.0 - 2**-24
                        assert (u * 2**24).is_integer()
                        assert np.float32(u) == u
                    seen.add((ua, us))
    assert len(seen) == 3 * 5 * 9 * 3  # distinct counters give distinct draws


def test_uniforms_are_uniform():
    from scipy import stats
    us = np.array([uniforms(7, b, j, 0)[0] for b in range(400) for j in range(10)])
    assert stats.kstest(us, "uniform").pvalue > 1e-3
