"""Pins for the oracle's storage decoding and bf16 rounding (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.numerics import decode, round_to_bf16, round_to_storage
from workloads.synth import bf16_bits_to_f32, f32_to_bf16_bits

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _is_nan_bits(b):
    b = b.astype(np.int64)
    return ((b >> 7) & 0xFF == 0xFF) & (b & 0x7F != 0)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_decode_matches_float32_reinterpretation_exhaustively():
    # bf16 is the top half of a float32: an independent library route to the same value.
    ref = bf16_bits_to_f32(ALL).astype(np.float64)
    got = decode(ALL, "bf16")
    nan = _is_nan_bits(ALL)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_known_values():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0001: 2.0 ** -133,
             0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x7F80: np.inf,
             0xFF80: -np.inf}
    for bits, v in cases.items():
        assert decode(np.array([bits], np.uint16), "bf16")[0] == v
    z = decode(np.array([0x8000], np.uint16), "bf16")[0]
    assert z == 0 and np.signbit(z)


def test_round_trip_is_identity_for_every_bf16_pattern():
    nan = _is_nan_bits(ALL)
    back = round_to_bf16(decode(ALL, "bf16"))
    assert np.array_equal(back[~nan], ALL[~nan])
    assert _is_nan_bits(back[nan]).all()


@pytest.mark.parametrize("v,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),          # tie between 0x3F80 and 0x3F81 -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),      # tie between 0x3F81 and 0x3F82 -> even
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie
    (2.0 ** -134, 0x0000),              # subnormal tie -> even (zero)
    (3 * 2.0 ** -134, 0x0002),          # subnormal tie -> even
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie at the top rounds to infinity
    (2.0 ** 128, 0x7F80),
    (-0.0, 0x8000),
    (0.0, 0x0000),
    (1e-50, 0x0000),
])
def test_round_to_bf16_hand_cases(v, bits):
    assert int(round_to_bf16(np.array([v]))[0]) == bits


def _exact_rne_bf16(v: float) -> int:
    """Brute-force RNE: find the two neighbouring bf16 values with exact rationals."""
    if v == 0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    # enumerate all finite positive bf16 values by binary search over bit patterns
    pos = np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f32(pos).astype(np.float64)
    i = int(np.searchsorted(vals, float(a), side="right")) - 1
    lo_b, lo = int(pos[i]), Fraction(float(vals[i]))
    if lo == a:
        return sign | lo_b
    hi_b = lo_b + 1
    hi = Fraction(float(vals[i + 1])) if hi_b <= 0x7F7F else Fraction(2) ** 128
    if a - lo < hi - a:
        return sign | lo_b
    if a - lo > hi - a:
        return sign | (hi_b if hi_b <= 0x7F7F else 0x7F80)
    pick = lo_b if lo_b % 2 == 0 else hi_b
    return sign | (pick if pick <= 0x7F7F else 0x7F80)


def test_round_to_bf16_matches_exact_brute_force():
    rng = np.random.default_rng(7)
    mags = np.concatenate([
        rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, 300),
        rng.standard_normal(50) * 2.0 ** -130,
    ])
    for v in mags:
        assert int(round_to_bf16(np.array([v]))[0]) == _exact_rne_bf16(float(v)), v


def test_round_to_bf16_agrees_with_input_generator_rounding():
    # Two independent implementations (quantum counting vs bit arithmetic).
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(200000) * 3).astype(np.float32)
    f = np.concatenate([f, np.float32([1.00390625, 1.01171875, -1.00390625])])
    assert np.array_equal(round_to_bf16(f.astype(np.float64)), f32_to_bf16_bits(f))


def test_round_to_storage_f32_is_ieee_cast():
    v = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    r = round_to_storage(v, "f32")
    assert r.dtype == np.float32
    assert r[0] == np.float32(1.0) and r[1] == np.float32(1.0 + 2.0 ** -22)
