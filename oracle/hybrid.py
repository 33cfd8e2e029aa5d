"""The hybrid training format: compact ELL rows plus a dense backup (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Format (gist.science "Sparser, Faster, Lighter Transformer Language Models",
Resumen Técnico §2.A, hybrid format for training; q2bstudio post on TwELL,
third paragraph).  Training activations are far from uniformly sparse, so the
pages store the rows with few non-zeros in a compact ELL matrix and send the
rows with many non-zeros to a dense backup matrix; the conversion from TwELL
is one of the training kernels (same summary, §2.B).

The pages give no width and no field layout.  The readings taken here (also
declared in ``include/twell.h``):

* The ELL part has a fixed width E (slots per row), chosen by the caller.
* cnt[t] = number of active entries of row t (the true count; active as in
  TwELL: IEEE v > 0 decided on the bits).
* Row t is an ELL row iff cnt[t] <= E.  Its slots s < cnt[t] hold the s-th
  active entry in ascending column order: the value bits and the column
  index.  Every other slot holds +0 and column 0.
* Rows with cnt[t] > E are dense rows: listed in ascending order, each kept
  whole (ReLU'd) in the dense backup; their ELL slots are all padding.
* Converted from a TwELL matrix, the result is the hybrid of the activation
  matrix the TwELL matrix describes (``twell.unpack``), whatever the TwELL
  tile width and capacity were.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import storage_zero
from .twell import Packed, active, relu_storage, unpack


@dataclass
class Hybrid:
    dtype: str
    width: int
    cnt: np.ndarray         # [T] int32, true number of active entries per row
    val: np.ndarray         # [T, width] storage dtype
    col: np.ndarray         # [T, width] int32 column index
    dense_rows: np.ndarray  # [n_dense] int32, ascending rows with cnt > width
    dense: np.ndarray       # [n_dense, F] storage dtype, ReLU'd rows

    @property
    def n_dense(self) -> int:
        return int(self.dense_rows.shape[0])


def _check(h: np.ndarray, dtype: str, width: int):
    if h.ndim != 2:
        raise ValueError("activations must be [T, F]")
    if width < 1:
        raise ValueError("the ELL width must be at least 1")
    want = np.float32 if dtype == "f32" else np.uint16
    if h.dtype != want:
        raise ValueError(f"{dtype} storage must be {np.dtype(want).name}")
    return h.shape


def hybrid_loop(h: np.ndarray, dtype: str, width: int) -> Hybrid:
    """The hybrid of an activation matrix in storage dtype, written as plain loops."""
    T, F = _check(h, dtype, width)
    act = active(h, dtype)
    cnt = np.zeros(T, dtype=np.int32)
    val = storage_zero((T, width), dtype)
    col = np.zeros((T, width), dtype=np.int32)
    dense_list = []
    for t in range(T):
        cols = [j for j in range(F) if act[t, j]]
        cnt[t] = len(cols)
        if len(cols) > width:
            dense_list.append(t)
            continue
        for s, j in enumerate(cols):
            val[t, s] = h[t, j]
            col[t, s] = j
    dense_rows = np.array(dense_list, dtype=np.int32)
    dense = storage_zero((len(dense_list), F), dtype)
    for r, t in enumerate(dense_list):
        for j in range(F):
            if act[t, j]:
                dense[r, j] = h[t, j]
    return Hybrid(dtype, width, cnt, val, col, dense_rows, dense)


def hybrid(h: np.ndarray, dtype: str, width: int) -> Hybrid:
    """Vectorised: same result as ``hybrid_loop`` for any input."""
    T, F = _check(h, dtype, width)
    act = active(h, dtype)
    cnt = act.sum(axis=1).astype(np.int32)
    ell = cnt <= width
    rank = np.cumsum(act, axis=1) - 1
    t_i, j_i = np.nonzero(act & ell[:, None])
    val = storage_zero((T, width), dtype)
    col = np.zeros((T, width), dtype=np.int32)
    val[t_i, rank[t_i, j_i]] = h[t_i, j_i]
    col[t_i, rank[t_i, j_i]] = j_i
    dense_rows = np.nonzero(~ell)[0].astype(np.int32)
    dense = relu_storage(h[dense_rows], dtype) if dense_rows.size else storage_zero((0, F), dtype)
    return Hybrid(dtype, width, cnt, val, col, dense_rows, dense)


def from_twell(p: Packed, width: int) -> Hybrid:
    """The conversion TwELL -> hybrid: the hybrid of the matrix ``p`` describes."""
    return hybrid(unpack(p), p.dtype, width)


def unhybrid(hy: Hybrid, F: int) -> np.ndarray:
    """Dense [T, F] storage tensor described by a hybrid matrix."""
    T = hy.cnt.shape[0]
    out = storage_zero((T, F), hy.dtype)
    for t in range(T):
        if hy.cnt[t] <= hy.width:
            n = int(hy.cnt[t])
            out[t, hy.col[t, :n]] = hy.val[t, :n]
    if hy.n_dense:
        out[hy.dense_rows] = hy.dense
    return out
