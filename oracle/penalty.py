"""The L1 activation penalty and its gradient, from TwELL (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages' training recipe adds an L1 penalty on the ReLU activations of the
feed-forward layers to the loss (gist.science "Sparser, Faster, Lighter
Transformer Language Models", Resumen Técnico §2.B, training-strategy paragraph, and §4,
coefficient 2e-5; edge.aivizor.me news post, first paragraph).  The pages do
not say how the sum is normalised.  Readings taken here:

* The penalty of an activation matrix h = ReLU(pre) is lam * ||h||_1 with
  ||h||_1 = sum over all entries of |h| (here every entry is >= 0); any
  per-token or per-unit normalisation is folded into lam by the caller.
* Its gradient with respect to h is lam at every active entry (h > 0) and 0
  elsewhere (at h = 0 the subgradient 0 is taken; ReLU passes no gradient
  there anyway), rounded to the storage dtype.  In TwELL form it has the
  TwELL matrix's own pattern: lam in every used slot, 0 in the padding, and
  lam at the active entries of the dense backup rows.
"""

from __future__ import annotations

import math

import numpy as np

from .numerics import decode, round_to_storage, storage_zero
from .twell import Packed, active, unpack


def l1_norm(h: np.ndarray, dtype: str) -> float:
    """sum |h| over every entry, exactly rounded to float64 (math.fsum)."""
    return math.fsum(np.abs(decode(h, dtype)).reshape(-1).tolist())


def l1_norm_twell(p: Packed) -> float:
    """||h||_1 of the activation matrix a TwELL matrix describes."""
    return l1_norm(unpack(p), p.dtype)


def l1_grad(h: np.ndarray, dtype: str, lam: float) -> np.ndarray:
    """d(lam * ||h||_1)/dh in the storage dtype: lam where h is active, else +0."""
    g = round_to_storage(np.array([lam], np.float64), dtype)[0]
    return np.where(active(h, dtype), g, storage_zero((), dtype)).astype(h.dtype)


def l1_grad_twell(p: Packed, lam: float):
    """The same gradient in TwELL form: (values [T, n_t, cap], dense rows [n_ovf, F])."""
    g = round_to_storage(np.array([lam], np.float64), p.dtype)[0]
    used = np.arange(p.cap)[None, None, :] < np.minimum(p.cnt.astype(np.int64), p.cap)[:, :, None]
    val = np.where(used, g, storage_zero((), p.dtype)).astype(p.val.dtype)
    dense = l1_grad(p.dense, p.dtype, lam) if p.n_ovf else storage_zero((0, p.shape[1]), p.dtype)
    return val, dense
