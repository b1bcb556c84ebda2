"""Philox-4x32-10 counter-based generator and the step's uniform draws.

Test infrastructure (see ``oracle/__init__``): never imported by the product.

The generator is Philox-4x32 with 10 rounds as defined by Salmon, Moraes,
Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), sec. 4:
each round multiplies counter words 0 and 2 by the two Philox multipliers,
keeps both halves of each 64-bit product, and mixes them with words 1 and 3
and the round key; the key is advanced by the two Weyl constants between
rounds.

The pages say only that draft and correction tokens are *sampled*
("LongSpark", sec. 2.1, eqs. (1)-(2) and (4)).  The convention below fixes
which uniform each decision consumes, so that two independent
implementations make the same draws:

* key      = (seed mod 2^32, seed >> 32)
* counter  = (v >> 2, j, req_id, stream); output word ``v & 3`` serves vocab
  entry ``v``.  ``j`` is the 1-based draft position (``K_b + 1`` for the
  bonus row), ``req_id`` a per-request 32-bit id, ``stream`` 0 for drafting,
  1 for the acceptance test, 2 for the correction / bonus token.
* acceptance uniform: word 0 of counter (0, j, req_id, 1), ``u = (x >> 8) *
  2^-24`` in [0, 1).
* Gumbel uniform: ``u = (2 * (x >> 9) + 1) * 2^-24`` in (0, 1), so that
  ``-log(-log u)`` is finite.
Both conversions are exact in binary32 and binary64.
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

STREAM_DRAFT = 0
STREAM_ACCEPT = 1
STREAM_SAMPLE = 2


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised Philox-4x32-10.  Counter words are arrays (or ints) of
    values < 2^32; the key is two 32-bit ints.  Returns four uint32 arrays."""
    m = np.uint64(MASK32)
    x0 = np.asarray(c0, dtype=np.uint64) & m
    x1 = np.asarray(c1, dtype=np.uint64) & m
    x2 = np.asarray(c2, dtype=np.uint64) & m
    x3 = np.asarray(c3, dtype=np.uint64) & m
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    ka, kb = int(k0) & MASK32, int(k1) & MASK32
    for rnd in range(10):
        if rnd:
            ka = (ka + PHILOX_W0) & MASK32
            kb = (kb + PHILOX_W1) & MASK32
        p0 = np.uint64(PHILOX_M0) * x0          # exact: both factors < 2^32
        p1 = np.uint64(PHILOX_M1) * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(ka), lo1,
                          hi0 ^ x3 ^ np.uint64(kb), lo0)
    return tuple(x.astype(np.uint32) for x in (x0, x1, x2, x3))


def split_seed(seed: int):
    seed = int(seed) & ((1 << 64) - 1)
    return seed & MASK32, seed >> 32


def accept_uniform(seed: int, req_id: int, j: int) -> float:
    """The acceptance uniform for draft position ``j`` of request ``req_id``."""
    k0, k1 = split_seed(seed)
    x = philox4x32_10(0, j, req_id, STREAM_ACCEPT, k0, k1)[0]
    return float(int(x) >> 8) * 2.0 ** -24


def gumbel_uniforms(seed: int, req_id: int, j: int, stream: int,
                    vocab: int) -> np.ndarray:
    """Uniforms in (0, 1) for vocab entries 0..vocab-1 (float64)."""
    k0, k1 = split_seed(seed)
    groups = np.arange((vocab + 3) // 4, dtype=np.uint64)
    words = philox4x32_10(groups, j, req_id, stream, k0, k1)
    x = np.stack(words, axis=1).reshape(-1)[:vocab].astype(np.uint64)
    return ((x >> np.uint64(9)) * 2 + 1).astype(np.float64) * 2.0 ** -24
