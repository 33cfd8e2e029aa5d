"""Seeded input generators (host side, numpy only).

Recipe (the same for every consumer):

* ``rng = numpy.random.Generator(numpy.random.PCG64(seed))``.
* Draw float64 standard normals in the order x [T,d], W_g [F,d], W_u [F,d],
  W_d [F,d].  W_g and W_u are scaled by 1/sqrt(d) and W_d by 1/sqrt(F), i.e.
  variance 1/fan_in.  (W_u is stored as W_u^T rows, i.e. [F][d]; W_d is stored
  as [F][d], one contiguous d-row per hidden unit.)
* Cast to float32 (numpy, round-to-nearest-even); for bf16 storage round the
  float32 value to bf16 with round-to-nearest-even on the bit pattern.
* Per-token gate bias ``beta_t = -Phi^{-1}(1 - rho_t)`` stored as float32.
  With x ~ N(0,1) and var(W_g) = 1/d the gate pre-activation has unit
  variance, so the realised fraction of active (positive) gate units is about
  rho_t.

Storage conventions: an ``f32`` tensor is a ``numpy.float32`` array, a
``bf16`` tensor is a ``numpy.uint16`` array holding the bf16 bit patterns.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from statistics import NormalDist
from typing import Callable, Optional, Sequence, Union

import numpy as np

DTYPES = ("f32", "bf16")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Works on the IEEE bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits.  NaNs become a quiet NaN with the same sign.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = np.where(nan, ((bits >> 16) | 0x40).astype(np.uint16), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float values to the storage representation of ``dtype``."""
    f32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f32
    if dtype == "bf16":
        return f32_to_bf16_bits(f32)
    raise ValueError(f"unknown dtype {dtype!r}")


def gate_bias_for_density(rho: float) -> float:
    """Gate bias that makes a unit-variance Gaussian positive with probability rho."""
    if not 0.0 < rho < 1.0:
        raise ValueError("density must be in (0, 1)")
    return -NormalDist().inv_cdf(1.0 - rho)


@dataclass
class FfnInputs:
    dtype: str
    x: np.ndarray        # [T, d]   storage dtype
    w_gate: np.ndarray   # [F, d]   storage dtype (W_g^T, nn.Linear weight layout)
    w_up: np.ndarray     # [F, d]   storage dtype (W_u^T)
    w_down: np.ndarray   # [F, d]   storage dtype (W_d, one row per hidden unit)
    gate_bias: Optional[np.ndarray]  # [T] float32, or None
    seed: int

    @property
    def shape(self):
        T, d = self.x.shape
        return T, d, self.w_gate.shape[0]


BiasSpec = Union[None, float, Sequence[float], np.ndarray, Callable[[np.ndarray], np.ndarray]]


def _bias_vector(T: int, spec: BiasSpec) -> Optional[np.ndarray]:
    if spec is None:
        return None
    if callable(spec):
        b = np.asarray(spec(np.arange(T)), dtype=np.float64)
    elif np.isscalar(spec):
        b = np.full(T, float(spec))
    else:
        b = np.asarray(spec, dtype=np.float64)
    if b.shape != (T,):
        raise ValueError("gate bias must have one value per token")
    return b.astype(np.float32)


def ffn_inputs(T: int, d: int, F: int, dtype: str, seed: int = 0,
               gate_bias: BiasSpec = None) -> FfnInputs:
    """Seeded x, W_g, W_u, W_d (and gate bias) for one FFN layer."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_storage(rng.standard_normal((T, d)), dtype)
    wg = to_storage(rng.standard_normal((F, d)) * (1.0 / math.sqrt(d)), dtype)
    wu = to_storage(rng.standard_normal((F, d)) * (1.0 / math.sqrt(d)), dtype)
    wd = to_storage(rng.standard_normal((F, d)) * (1.0 / math.sqrt(F)), dtype)
    return FfnInputs(dtype, x, wg, wu, wd, _bias_vector(T, gate_bias), seed)


def pre_activations(T: int, F: int, dtype: str, seed: int = 0, density: float = 0.01,
                    hot_rows: Sequence[int] = (), hot_density: float = 0.2,
                    specials: bool = False) -> np.ndarray:
    """A standalone gate pre-activation tensor [T, F] in the storage dtype.

    Values are N(beta, 1) with beta set for ``density``; rows in ``hot_rows``
    use ``hot_density`` instead.  With ``specials`` a sprinkling of +-0,
    +-denormals, +-inf and NaNs (both signs) is written over random positions.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    beta = np.full((T, 1), gate_bias_for_density(density))
    hot = np.asarray(list(hot_rows), dtype=np.int64)
    if hot.size:
        beta[hot] = gate_bias_for_density(hot_density)
    v = rng.standard_normal((T, F)) + beta
    s = to_storage(v, dtype)
    if specials and T * F > 0:
        n = max(1, (T * F) // 50)
        pos = rng.integers(0, T * F, size=n)
        kind = rng.integers(0, 8, size=n)
        flat = s.reshape(-1)
        if dtype == "bf16":
            table = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1],
                             dtype=np.uint16)
            flat[pos] = table[kind]
        else:
            bits = flat.view(np.uint32)
            table = np.array([0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x7F800000,
                              0xFF800000, 0x7FC00000, 0xFFC00001], dtype=np.uint32)
            bits[pos] = table[kind]
    return s


def grad_output(T: int, d: int, dtype: str, seed: int = 0) -> np.ndarray:
    """A seeded upstream gradient dy [T, d] (standard normals) in the storage dtype.

    Drawn from its own stream (seed sequence [seed, 2]) so that it never
    repeats the draws of ``ffn_inputs`` for the same seed.
    """
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    return to_storage(rng.standard_normal((T, d)), dtype)
