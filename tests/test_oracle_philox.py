"""Pins for the oracle's Philox-4x32-10 and its uniform conversions."""
import os

import numpy as np
import pytest
from scipy import stats

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_known_answer_vectors(ctr, key, expect):
    out = philox.philox4x32_10(*ctr, *key)
    assert [int(x) for x in out] == expect


def test_vectorised_matches_scalar():
    c0 = np.arange(1000, dtype=np.uint64) * 7919
    out = philox.philox4x32_10(c0, 5, 0xDEADBEEF, 2, 0x12345678, 0x9ABCDEF0)
    for i in (0, 1, 517, 999):
        s = philox.philox4x32_10(int(c0[i]), 5, 0xDEADBEEF, 2, 0x12345678, 0x9ABCDEF0)
        assert [int(o[i]) for o in out] == [int(x) for x in s]


def test_accept_uniform_on_24bit_grid():
    us = [philox.accept_uniform(0xABCDEF0123456789, rid, j)
          for rid in range(50) for j in range(1, 18)]
    for u in us:
        assert 0.0 <= u < 1.0
        assert float(np.float32(u)) == u          # exact in binary32
        assert (u * 2 ** 24) == int(u * 2 ** 24)  # on the 2^-24 grid


def test_gumbel_uniform_open_interval_and_exact():
    u = philox.gumbel_uniforms(42, 7, 3, philox.STREAM_DRAFT, 10007)
    assert u.shape == (10007,)
    assert np.all(u > 0) and np.all(u < 1)
    assert np.all(u.astype(np.float32).astype(np.float64) == u)
    k = u * 2 ** 24
    assert np.all(k == np.floor(k)) and np.all(k % 2 == 1)   # odd multiples of 2^-24


def test_word_to_vocab_mapping():
    # vocab entry v uses word (v & 3) of counter (v >> 2, j, req, stream)
    seed, rid, j, st = 0x1122334455667788, 99, 4, 2
    u = philox.gumbel_uniforms(seed, rid, j, st, 64)
    k0, k1 = philox.split_seed(seed)
    for v in (0, 1, 2, 3, 4, 37, 63):
        w = philox.philox4x32_10(v >> 2, j, rid, st, k0, k1)[v & 3]
        assert u[v] == ((int(w) >> 9) * 2 + 1) * 2.0 ** -24


def test_uniformity_chi_square():
    u = philox.gumbel_uniforms(2024, 1, 1, 0, 400000)
    counts = np.histogram(u, bins=256, range=(0, 1))[0]
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4


def test_streams_and_positions_differ():
    a = philox.gumbel_uniforms(5, 1, 1, 0, 64)
    b = philox.gumbel_uniforms(5, 1, 1, 2, 64)
    c = philox.gumbel_uniforms(5, 1, 2, 0, 64)
    d = philox.gumbel_uniforms(5, 2, 1, 0, 64)
    for x in (b, c, d):
        assert np.mean(a == x) < 0.05
