"""Pins for the oracle's Philox-4x32-10 and its uniform conversions.

The generator is pinned against an independent implementation: AMD's rocRAND
Philox-4x32-10 (its header implementation compiled as a host program from
``philox_rocrand_ref.cpp``), bit for bit, on counters that exercise every
word, carries near 2^32 and the all-zero / all-one extremes.  (rocRAND
reaches counter word 1 through a 64-bit count of outputs, so word 1 stays
below 2^30 there; the step's counters use small positions in that word.)
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is needed to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_rocrand_ref")
    r = subprocess.run([hipcc, "-O1", os.path.join(HERE, "philox_rocrand_ref.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr

    def run(rows):
        txt = "".join(f"{s} {a} {b} {c} {d}\n" for s, a, b, c, d in rows)
        out = subprocess.run([exe], input=txt, capture_output=True, text=True, check=True)
        return [[int(x) for x in line.split()] for line in out.stdout.splitlines()]
    return run


def test_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(7)
    M = 0xFFFFFFFF
    C1 = (1 << 30) - 1       # rocRAND's 64-bit output offset reaches c1 < 2^30
    rows = [(0, 0, 0, 0, 0), ((1 << 64) - 1, M, C1, M, M), (0x1122334455667788, 5, 7, 9, 11),
            (42, M, 0, 0, 0), (42, M, C1, 0, 0), (42, 0, 0, M, M)]
    for _ in range(300):
        rows.append((int(rng.integers(0, 1 << 63)) * 2 + int(rng.integers(0, 2)),
                     int(rng.integers(0, 1 << 32)), int(rng.integers(0, 1 << 30)),
                     int(rng.integers(0, 1 << 32)), int(rng.integers(0, 1 << 32))))
    ref = rocrand_ref(rows)
    assert len(ref) == len(rows)
    for (seed, c0, c1, c2, c3), want in zip(rows, ref):
        k0, k1 = philox.split_seed(seed)
        got = [int(x) for x in philox.philox4x32_10(c0, c1, c2, c3, k0, k1)]
        assert got == want, (seed, c0, c1, c2, c3)


def test_matches_rocrand_vectorised_vocab_rows(rocrand_ref):
    # the exact counters one Gumbel draw over a small vocab consumes
    seed, rid, j = 0xDEADBEEFCAFEF00D, 123456789, 17
    k0, k1 = philox.split_seed(seed)
    groups = np.arange(64, dtype=np.uint64)
    words = np.stack(philox.philox4x32_10(groups, j, rid, philox.STREAM_SAMPLE, k0, k1), 1)
    ref = rocrand_ref([(seed, g, j, rid, philox.STREAM_SAMPLE) for g in range(64)])
    assert words.tolist() == ref


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
