"""Pins of the oracle's Philox4x64-10 against numpy.random.Philox (same generator).

numpy's bit generator advances its 256-bit counter before producing a block,
so the first four raw words for state counter c are the Philox block at c+1
(word 0 incremented, carrying into word 1, ...).
"""
import numpy as np
import pytest

from oracle.philox import philox4x64_10, uniform24, uniform53

MASK = (1 << 64) - 1


def _inc(ctr):
    c = list(ctr)
    for i in range(4):
        c[i] = (c[i] + 1) & MASK
        if c[i] != 0:
            break
    return tuple(c)


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 7, 11, 13), (123, 456)),
    ((MASK, 3, 0, 9), (2**63 + 5, 77)),
    ((MASK, MASK, 1, 0), (1, MASK)),
    ((31, 16, 1, 2**40), (20261202, 0)),
]


@pytest.mark.parametrize("ctr,key", CASES)
def test_against_numpy_philox(ctr, key):
    bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    w = [int(x) for x in bg.random_raw(8)]
    assert tuple(w[:4]) == philox4x64_10(_inc(ctr), key)
    assert tuple(w[4:]) == philox4x64_10(_inc(_inc(ctr)), key)


def test_random_counters_against_numpy():
    rng = np.random.default_rng(7)
    for _ in range(50):
        ctr = tuple(int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.uint64))
        key = tuple(int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.uint64))
        bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
        assert tuple(int(x) for x in bg.random_raw(4)) == philox4x64_10(_inc(ctr), key)


def test_uniform_bit_extraction():
    assert uniform24(0) == 0.0
    assert uniform24(MASK) == 1.0 - 2.0 ** -24
    assert uniform24(1 << 40) == 2.0 ** -24
    assert uniform24((1 << 40) - 1) == 0.0
    assert uniform53(MASK) == 1.0 - 2.0 ** -53
    assert uniform53(1 << 11) == 2.0 ** -53
    # exact dyadics: multiplying back gives the integer
    w = 0xDEADBEEFCAFEF00D
    assert uniform24(w) * 2**24 == (w >> 40)
    assert uniform53(w) * 2**53 == (w >> 11)
