"""Pins for the oracle's storage-type conversions (binary16 and bfloat16 <-> double).

The decoders are checked exhaustively against numpy's own binary16 decoder and against the
bfloat16 definition as the upper half of a binary32 pattern.  The encoders are checked for
round-to-nearest-even against numpy (binary16) and against brute-force neighbour search.
"""
import numpy as np
import pytest

from oracle import oracle as orc


def test_f16_decode_every_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_every_pattern_is_upper_half_of_binary32():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([orc.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _f16_cases(rng):
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = np.sort(finite[np.isfinite(finite)].astype(np.float64))
    finite = np.unique(finite)
    mids = (finite[:-1] + finite[1:]) / 2.0               # exact ties in double
    rand = np.concatenate([rng.standard_normal(4000) * s for s in (1e-7, 1e-5, 1e-2, 1.0, 1e3, 6e4)])
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 2.0 ** -24,
                     2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, np.inf, -np.inf])
    return np.concatenate([mids, rand, edge])


def test_f64_to_f16_round_nearest_even_matches_numpy():
    vals = _f16_cases(np.random.default_rng(1))
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f64_to_f16_bits(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _bf16_value(b):
    return float((np.uint32(b) << np.uint32(16)).view(np.float32))


@pytest.mark.parametrize("seed", [0, 1])
def test_f64_to_bf16_is_nearest_with_ties_to_even(seed):
    rng = np.random.default_rng(seed)
    vals = np.concatenate([rng.standard_normal(3000) * s for s in (1e-39, 1e-3, 1.0, 1e30)])
    # exact midpoints between neighbouring bfloat16 values
    b = rng.integers(0, 0x7F7F, 2000, dtype=np.uint32)
    mids = np.array([(_bf16_value(x) + _bf16_value(x + 1)) / 2.0 for x in b])
    vals = np.concatenate([vals, mids, -mids])
    for v in vals:
        got = orc.f64_to_bf16_bits(float(v))
        g = _bf16_value(got)
        # neighbours of the result in the bfloat16 grid (same sign)
        mag = got & 0x7FFF
        for nb in (mag - 1, mag + 1):
            if 0 <= nb < 0x7F80:
                n = _bf16_value(nb | (got & 0x8000))
                assert abs(v - g) <= abs(v - n), (v, got)
                if abs(v - g) == abs(v - n):
                    assert (got & 1) == 0, (v, got)        # tie goes to the even pattern


def test_f64_to_bf16_overflow_and_signed_zero():
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127                   # halfway to 2^128
    assert orc.f64_to_bf16_bits(big) == 0x7F80
    assert orc.f64_to_bf16_bits(np.nextafter(big, 0)) == 0x7F7F
    assert orc.f64_to_bf16_bits(-0.0) == 0x8000
    assert orc.f64_to_bf16_bits(2.0 ** -133) == 0x0001
    assert orc.f64_to_bf16_bits(2.0 ** -134) == 0x0000     # tie with zero goes to even (zero)
