"""Pins for the oracle's Philox4x64-10 against NumPy's independent implementation
(numpy.random.Philox), run here as a known-answer source."""

import numpy as np
import pytest

from oracle.philox import MASK64, philox4x64_10, uniforms_for_node


def _numpy_block(counter, key):
    # numpy's Philox increments its 256-bit counter before producing a block, so
    # start it one below the counter we want.
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & MASK64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array([int(k) for k in key], dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


def test_zero_counter_zero_key_block():
    got = philox4x64_10((0, 0, 0, 0), (0, 0))
    assert list(got) == _numpy_block((0, 0, 0, 0), (0, 0))


@pytest.mark.parametrize("counter,key", [
    ((1, 0, 0, 0), (0, 0)),
    ((0, 1, 0, 0), (7, 0)),
    ((5, 3, 9, 0), (123456789, 0)),
    ((MASK64, MASK64, MASK64, MASK64), (MASK64, MASK64)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_matches_numpy(counter, key):
    assert list(philox4x64_10(counter, key)) == _numpy_block(counter, key)


def test_random_counters_match_numpy():
    rng = np.random.default_rng(0)
    for _ in range(50):
        counter = [int(x) for x in rng.integers(0, 2 ** 63, size=4, dtype=np.int64)]
        key = [int(x) for x in rng.integers(0, 2 ** 63, size=2, dtype=np.int64)]
        assert list(philox4x64_10(counter, key)) == _numpy_block(counter, key)


def test_node_uniforms_are_24_bit_and_distinct():
    seen = set()
    for b in range(3):
        for i in range(40):
            ua, us = uniforms_for_node(17, 5, b, i)
            for u in (ua, us):
                assert 0.0 <= u < 1.0
                assert (u * 2 ** 24) == int(u * 2 ** 24)
                assert np.float32(u) == u
            seen.add((ua, us))
    assert len(seen) == 120
    # the counter layout puts the node in word 0, the request in word 1, the offset in word 2
    w = philox4x64_10((4, 2, 5, 0), (17, 0))
    assert uniforms_for_node(17, 5, 2, 4) == ((w[0] >> 40) * 2.0 ** -24, (w[1] >> 40) * 2.0 ** -24)
