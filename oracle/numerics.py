"""Exact storage-dtype decoding and bf16 round-to-nearest-even (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Storage conventions: ``f32`` tensors are ``numpy.float32`` arrays; ``bf16``
tensors are ``numpy.uint16`` arrays of bf16 bit patterns (1 sign bit, 8
exponent bits with bias 127, 7 fraction bits).

The pages fix no precision.  The storage dtype and its rounding rule are a
reading: bf16 values are produced by IEEE round-to-nearest, ties-to-even.
Decoding is written from the field definition (sign, exponent, fraction) with
``numpy.ldexp``, which is exact; it is pinned against the float32 bit
reinterpretation in the tests.
"""

from __future__ import annotations

import numpy as np


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every element of a storage tensor."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    bits = np.asarray(a, dtype=np.uint16).astype(np.int64)
    sign = np.where((bits >> 15) & 1, -1.0, 1.0)
    e = (bits >> 7) & 0xFF
    frac = (bits & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + frac / 128.0, (e - 127).astype(np.int64))
    subnormal = sign * np.ldexp(frac / 128.0, -126)
    out = np.where(e == 0, subnormal, normal)
    special = np.where(frac == 0, sign * np.inf, np.nan)
    return np.where(e == 0xFF, special, out)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 bit patterns, to nearest with ties to even.

    Each magnitude is written as an integer number of bf16 quanta (2^(E-7) for
    a normal number with exponent E, 2^-133 below the normal range); that count
    is rounded with ``numpy.rint`` (ties to even) and re-encoded.  Magnitudes
    that round to 2^128 or beyond become infinity; NaN becomes the quiet NaN
    0x7FC0 with the input's sign.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    neg = np.signbit(v)
    nan = np.isnan(v)
    finite = np.isfinite(v) & (a > 0)
    safe = np.where(finite, a, 1.0)
    _, e = np.frexp(safe)                     # safe = f * 2**e, 0.5 <= f < 1
    E = e.astype(np.int64) - 1                # safe = 1.xxx * 2**E
    qexp = np.maximum(E, -126) - 7            # exponent of one bf16 quantum
    n = np.rint(np.ldexp(safe, -qexp))        # exact scaling, then RNE to integer
    r = np.ldexp(n, qexp)                     # rounded magnitude (exact)
    # encode the rounded magnitude
    sub = r < 2.0 ** -126
    sub_bits = np.ldexp(r, 133)               # integer 0..127 in the subnormal range
    rr = np.where(sub | (r == 0), 1.0, r)
    fr, ex = np.frexp(rr)
    Er = ex.astype(np.int64) - 1
    mant = (fr * 2.0 - 1.0) * 128.0           # integer 0..127
    norm_bits = (Er + 127) * 128 + mant
    bits = np.where(sub, sub_bits, norm_bits)
    bits = np.where(Er + 127 >= 255, 0x7F80, bits)  # overflow to infinity
    bits = np.where(finite, bits, 0)
    bits = np.where(np.isinf(v), 0x7F80, bits)
    bits = bits.astype(np.int64) | np.where(neg, 0x8000, 0)
    bits = np.where(nan, 0x7FC0 | np.where(neg, 0x8000, 0), bits)
    return bits.astype(np.uint16)


def round_to_storage(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype (RNE for both dtypes)."""
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_zero(shape, dtype: str) -> np.ndarray:
    """A tensor of +0 in the storage dtype."""
    return np.zeros(shape, dtype=np.float32 if dtype == "f32" else np.uint16)


def storage_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Signed integer view of the storage bit patterns (int32 for f32, int16 for bf16)."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)
    if dtype == "bf16":
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)
    raise ValueError(f"unknown dtype {dtype!r}")
