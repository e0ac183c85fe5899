"""Pins of the oracle's bfloat16 rounding.

The decode rounds k_val, v and q_val to the bank dtype and stores rows and
readings in it (page "sparse_delta_memory/decode.py", docstring of
sdm_decode_step and the casts in _sdm_decode_kernel); the reading taken is
round-to-nearest, ties to even. The float32 path is checked against torch's
own float32 -> bfloat16 conversion (a library routine with that rounding), the
double path against an exact rational nearest-value search.
"""

import ctypes
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import f32_to_bf16_bits_torch


def _edge_floats():
    bits = [0x00000000, 0x80000000, 0x3f800000, 0x3f808000, 0x3f818000, 0x3f807fff, 0x3f808001,
            0x7f7fffff, 0x7f7f7fff, 0x7f7f8000, 0xff7f8000, 0x00000001, 0x00008000, 0x00018000,
            0x007fffff, 0x00800000, 0x7f800000, 0xff800000, 0x3effffff, 0xbf808000, 0x477fe000]
    return np.array(bits, dtype=np.uint32).view(np.float32)


def _oracle_bits(xs):
    return np.array([oracle.float_to_bf16(float(x)) for x in xs], dtype=np.uint16)


def test_float_to_bf16_matches_torch_on_edges():
    xs = _edge_floats()
    assert np.array_equal(_oracle_bits(xs), f32_to_bf16_bits_torch(xs))


def test_float_to_bf16_matches_torch_on_random_bits():
    rng = np.random.default_rng(30)
    u = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    xs = u.view(np.float32)
    xs = xs[np.isfinite(xs)]
    assert np.array_equal(_oracle_bits(xs), f32_to_bf16_bits_torch(xs))
    # near-ties: low 16 bits around 0x8000
    base = rng.integers(0, 2 ** 16, 5000, dtype=np.uint64).astype(np.uint32) << 16
    low = rng.choice(np.array([0x7fff, 0x8000, 0x8001], np.uint32), 5000)
    xs = ((base & 0x7f7f0000) | low).view(np.float32)
    assert np.array_equal(_oracle_bits(xs), f32_to_bf16_bits_torch(xs))


def test_nan_stays_nan():
    for b in (0x7fc00000, 0x7f800001, 0xffc00001):
        x = np.array([b], np.uint32).view(np.float32)[0]
        r = oracle.float_to_bf16(float(x))
        assert (r & 0x7f80) == 0x7f80 and (r & 0x007f) != 0


def _bf16_value(bits: int) -> Fraction:
    x = np.array([bits << 16], np.uint32).view(np.float32)[0]
    return Fraction(float(x))


def _nearest_bf16_exact(x: float) -> int:
    """Nearest bfloat16 by exhaustive neighbour comparison in exact rationals."""
    fx = Fraction(x)
    if x == 0:
        return 0x8000 if np.signbit(x) else 0
    sign = 0x8000 if x < 0 else 0
    a = abs(fx)
    # start from the truncation of the float32 nearest to x and look at neighbours
    t = int(np.array([abs(np.float32(x))], np.float32).view(np.uint32)[0]) >> 16
    best = None
    for cand in range(max(0, t - 2), min(0x7f80, t + 3) + 1):
        v = Fraction(float("inf")) if cand == 0x7f80 else _bf16_value(cand)
        if cand == 0x7f80:
            # overflow threshold: max finite + half an ulp rounds to infinity (ties to even)
            lim = _bf16_value(0x7f7f) + (_bf16_value(0x7f7f) - _bf16_value(0x7f7e)) / 2
            if a >= lim:
                return sign | 0x7f80
            continue
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and cand % 2 == 0):
            best = (d, cand)
    return sign | best[1]


def test_double_to_bf16_is_one_rounding():
    rng = np.random.default_rng(31)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)))
    # doubles exactly halfway between bfloat16 values, and just off them
    for b in rng.integers(1, 0x7f7f, 500):
        lo, hi = _bf16_value(int(b)), _bf16_value(int(b) + 1)
        mid = float((lo + hi) / 2)
        xs += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    for x in xs:
        assert oracle.double_to_bf16(x) == _nearest_bf16_exact(x), x


def test_double_rounding_differs_from_two_step():
    """A double just above a bfloat16 tie, whose float32 rounding lands on the tie:
    one rounding goes up, two roundings go to even (down)."""
    lo = _bf16_value(0x3f80)  # 1.0
    hi = _bf16_value(0x3f81)
    x = float((lo + hi) / 2) + 2.0 ** -40
    assert oracle.double_to_bf16(x) == 0x3f81
    assert oracle.float_to_bf16(float(np.float32(x))) == 0x3f80


@pytest.mark.parametrize("b", [0, 1, 0x3f80, 0x7f7f, 0x8001, 0xc2f7])
def test_widening_is_exact(b):
    assert oracle.bf16_to_float(b) == float(np.array([b << 16], np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("bits", [0x7f800001, 0xff800001, 0x7f80ffff, 0x7fa00000])
def test_nan_with_low_payload_stays_nan_in_the_decode(bits):
    """A float32 NaN whose payload lies only in the low 16 bits (or a signalling NaN)
    truncates to the bits of an infinity; the rounding must still give a NaN (the
    reading "NaN stays NaN"). Passed as raw float32 bits through the decode on a
    bfloat16 bank, where v is rounded to the bank dtype: the written row and the
    reading of it are NaNs, not infinities. (A Python float would quiet the NaN on
    its way in, which is why this goes through an array.)"""
    bank = np.array([[0x3f80]], np.uint16)  # one slot, hd 1: 1.0
    v = np.array([[bits]], np.uint32).view(np.float32)
    readings = oracle.decode_step(bank, np.array([[0]]), np.array([[1.0]], np.float32), v,
                                  np.array([[1.0]], np.float32), np.array([[0.0]], np.float32), np.array([[0]]),
                                  np.array([[1.0]], np.float32))
    for b in (int(bank[0, 0]), int(readings[0, 0])):
        assert (b & 0x7f80) == 0x7f80 and (b & 0x007f) != 0, hex(b)


def test_array_conversion_is_the_scalar_one():
    """The oracle's array form converts every element as the scalar form does (edge bit
    patterns, NaN payloads and random bits), and as torch does on the non-NaN ones."""
    rng = np.random.default_rng(7)
    edge = np.array([0, 0x80000000, 1, 0x7fff, 0x8000, 0x8001, 0x18000, 0x3f808000, 0x3f818000, 0x7f7f8000,
                     0x7f7fffff, 0x7f800000, 0xff800000, 0x7f800001, 0x7fc00000, 0xffffffff, 0x807fffff],
                     dtype=np.uint32)
    bits = np.concatenate([edge, rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)])
    got = oracle.float_to_bf16_array(bits.view(np.float32))
    lib = oracle._load()
    want = np.array([lib.oracle_float_to_bf16(ctypes.c_float.from_buffer_copy(int(b).to_bytes(4, "little")))
                     for b in bits], dtype=np.uint16)
    assert np.array_equal(got, want)
    ok = (bits & 0x7fffffff) <= 0x7f800000
    t = torch.from_numpy(bits[ok].view(np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[ok], t)
