"""Pins for the oracle's number handling and for eq. (5)'s survival products.

* ``bf16_bits_to_f64`` (the decode every attention, LM-head and scheduler pin
  goes through) against torch's own bfloat16 -> float64 conversion over all
  65,536 bit patterns;
* ``f32_to_bf16_bits`` (round to nearest, ties to even) against torch's
  float32 -> bfloat16 conversion on random values, exact halfway cases of
  both parities, values just off halfway, and the overflow to infinity;
* ``distribute_budget``'s S^ against a per-request ``np.cumprod`` and a
  two-request example worked by hand from "ForeSpark", sec. 4.4, eq. (5)
  (``tests/golden/forespark_eq5_budget.json``).

Each pin is also run against planted mistakes (a decode that drops the sign or shifts wrongly, a
truncating encode, an exclusive running product) to show that it would catch
them; the mistakes live only in this file.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import schedule as osch
from oracle.attention import bf16_bits_to_f64, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "forespark_eq5_budget.json")
ALL_BITS = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _torch_decode(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def _torch_encode(x):
    return (torch.from_numpy(np.asarray(x, np.float32).copy()).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def _decode_matches(fn):
    with np.errstate(invalid="ignore"):   # the NaN patterns
        got = np.asarray(fn(ALL_BITS), np.float64)
    ref = _torch_decode(ALL_BITS)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    # signed zeros must keep their sign as well
    same &= np.signbit(got) == np.signbit(ref)
    return bool(same.all())


def _encode_cases():
    rng = np.random.default_rng(1234)
    vals = [rng.normal(0, s, 20000).astype(np.float32) for s in (1e-3, 1.0, 3.0, 1e4)]
    hi = rng.integers(0, 0x7F7F, 4000, dtype=np.uint32)
    hi[0::2] &= ~np.uint32(1)          # even upper halves
    hi[1::2] |= np.uint32(1)           # odd upper halves
    sign = (rng.integers(0, 2, hi.size, dtype=np.uint32) << 31)
    halfway = ((hi << 16) | 0x8000 | sign).astype(np.uint32)
    below = ((hi << 16) | 0x7FFF | sign).astype(np.uint32)
    above = ((hi << 16) | 0x8001 | sign).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x00008000, 0x00018000, 0x7F7FFFFF,
                        0xFF7FFFFF, 0x7F7F8000, 0x3F808000, 0x3F818000, 0x00000001],
                       np.uint32)
    bits = np.concatenate([halfway, below, above, special])
    vals.append(bits.view(np.float32))
    return np.concatenate(vals)


def _encode_matches(fn):
    x = _encode_cases()
    return bool(np.array_equal(np.asarray(fn(x), np.uint16), _torch_encode(x)))


def test_bf16_decode_equals_torch_on_every_pattern():
    assert _decode_matches(bf16_bits_to_f64)


def test_bf16_decode_pin_catches_sign_and_shift_mistakes():
    def drops_sign(bits):   # masks the sign bit away
        u = (np.asarray(bits, np.uint16).astype(np.uint32) & 0x7FFF) << 16
        return u.view(np.float32).astype(np.float64)
    assert not _decode_matches(drops_sign)

    def short_shift(bits):  # the pattern lands one bit too low
        u = np.asarray(bits, np.uint16).astype(np.uint32) << 15
        return u.view(np.float32).astype(np.float64)
    assert not _decode_matches(short_shift)

    def no_shift(bits):     # reads the pattern as the low half of a float
        return np.asarray(bits, np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)
    assert not _decode_matches(no_shift)


def test_bf16_encode_equals_torch_round_to_nearest_even():
    assert _encode_matches(f32_to_bf16_bits)


def test_bf16_encode_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (bf16 has 7 fraction bits)
    assert f32_to_bf16_bits(np.float32(1.0 + 2.0 ** -8))[()] == 0x3F80
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert f32_to_bf16_bits(np.float32(1.0 + 3 * 2.0 ** -8))[()] == 0x3F82


def test_bf16_encode_pin_catches_wrong_rounding():
    def truncate(x):
        return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert not _encode_matches(truncate)

    def ties_away(x):
        u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
        return ((u + 0x8000) >> 16).astype(np.uint16)
    assert not _encode_matches(ties_away)


def _golden():
    g = json.load(open(GOLDEN))
    return g, np.array(g["q_off"]), np.array(g["p"], np.float64)


def test_survival_worked_example_eq5():
    g, q_off, p = _golden()
    for B, want in g["verify_len_by_budget"].items():
        S, b = osch.distribute_budget(p, q_off, int(B))
        assert np.array_equal(S, np.array(g["survival"])), "S^ must be exact here"
        assert b.tolist() == want, (B, b.tolist(), want)


@pytest.mark.parametrize("seed", range(4))
def test_survival_is_the_inclusive_running_product(seed):
    rng = np.random.default_rng(seed)
    d = rng.integers(0, 17, 9)
    q_off = np.concatenate([[0], np.cumsum(d)])
    p = rng.uniform(0.01, 1.0, q_off[-1])
    S, _ = osch.distribute_budget(p, q_off, 10)
    for i in range(len(d)):
        seg = slice(q_off[i], q_off[i + 1])
        np.testing.assert_allclose(S[seg], np.cumprod(p[seg]), rtol=1e-15, atol=0)


def test_survival_pin_catches_exclusive_product():
    g, q_off, p = _golden()

    def exclusive(p, q_off, B):
        S = np.empty(len(p))
        for i in range(len(q_off) - 1):
            seg = p[q_off[i]:q_off[i + 1]]
            S[q_off[i]:q_off[i + 1]] = np.concatenate([[1.0], np.cumprod(seg)[:-1]])
        return S
    assert not np.array_equal(exclusive(p, q_off, 3), np.array(g["survival"]))
    # and the budget split that an exclusive product would give differs too
    order = sorted(range(len(p)), key=lambda m: -exclusive(p, q_off, 3)[m])[:3]
    b = [sum(1 for m in order if q_off[i] <= m < q_off[i + 1]) for i in range(2)]
    assert b != g["verify_len_by_budget"]["3"]
