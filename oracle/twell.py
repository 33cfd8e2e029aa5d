"""TwELL (tile-wise ELLPACK) packing, unpacking and the sparse FFN path (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Format (gist.science "Sparser, Faster, Lighter Transformer Language Models",
Resumen Técnico §2.A; estadored.mx news item on the same paper, paragraph on
TwELL; q2bstudio post on TwELL, third paragraph).  The hidden dimension F of a
token-major activation matrix is cut into contiguous column tiles of width W;
for every (token row t, tile k) the format keeps the number of non-zeros, the
non-zero values and their column index inside the tile, up to a fixed
capacity C per tile.  Rows in which some tile holds more than C non-zeros
overflow and are kept whole in a dense backup matrix.

The pages give no field layout.  The readings taken here (also declared in
``include/twell.h``):

* active(v) is IEEE ``v > 0`` decided on the bit pattern: +denormals and +inf
  are active; +-0, negatives and every NaN are not.
* cnt[t, k]  = number of active columns in tile k of row t, not capped.
* val[t, k, s], idx[t, k, s] for s < min(cnt, C): the s-th active column of the
  tile in ascending column order, its value bits and its column offset in the
  tile.  Unused slots hold +0 and index 0.
* A row overflows iff some tile has cnt > C (cnt == C still fits).  Overflow
  rows are listed in ascending order; their TwELL slots still hold the first
  min(cnt, C) entries; ``dense`` holds ReLU(row) for them in the same order.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import decode, storage_bits, storage_zero

_ACTIVE_MAX = {"f32": 0x7F800000, "bf16": 0x7F80}


@dataclass
class Packed:
    dtype: str
    tile: int
    cap: int
    cnt: np.ndarray       # [T, nt] uint16, true (uncapped) count per tile
    val: np.ndarray       # [T, nt, cap] storage dtype
    idx: np.ndarray       # [T, nt, cap] uint8, column offset inside the tile
    ovf_rows: np.ndarray  # [n_ovf] int32, ascending
    dense: np.ndarray     # [n_ovf, F] storage dtype, ReLU'd overflow rows

    @property
    def n_ovf(self) -> int:
        return int(self.ovf_rows.shape[0])

    @property
    def shape(self):
        T, nt = self.cnt.shape
        return T, nt * self.tile


def active(pre: np.ndarray, dtype: str) -> np.ndarray:
    """Elementwise IEEE ``pre > 0`` decided on the storage bits."""
    b = storage_bits(pre, dtype)
    return (b > 0) & (b <= _ACTIVE_MAX[dtype])


def relu_storage(pre: np.ndarray, dtype: str) -> np.ndarray:
    """ReLU in the storage dtype: active values kept bit for bit, everything else +0."""
    pre = np.asarray(pre)
    return np.where(active(pre, dtype), pre, storage_zero((), dtype)).astype(pre.dtype)


def _check(pre: np.ndarray, dtype: str, tile: int, cap: int):
    if pre.ndim != 2:
        raise ValueError("pre-activations must be [T, F]")
    T, F = pre.shape
    if tile <= 0 or F % tile != 0:
        raise ValueError("F must be a multiple of the tile width")
    if tile > 256:
        raise ValueError("tile width must fit a uint8 column offset")
    if not 1 <= cap <= tile:
        raise ValueError("capacity must be in [1, tile]")
    want = np.float32 if dtype == "f32" else np.uint16
    if pre.dtype != want:
        raise ValueError(f"{dtype} storage must be {np.dtype(want).name}")
    return T, F, F // tile


def pack_loop(pre: np.ndarray, dtype: str, tile: int, cap: int) -> Packed:
    """Reference packer written as plain loops (small inputs only)."""
    T, F, nt = _check(pre, dtype, tile, cap)
    act = active(pre, dtype)
    cnt = np.zeros((T, nt), dtype=np.uint16)
    val = storage_zero((T, nt, cap), dtype)
    idx = np.zeros((T, nt, cap), dtype=np.uint8)
    ovf = []
    for t in range(T):
        row_overflows = False
        for k in range(nt):
            n = 0
            for c in range(tile):
                j = k * tile + c
                if act[t, j]:
                    if n < cap:
                        val[t, k, n] = pre[t, j]
                        idx[t, k, n] = c
                    n += 1
            cnt[t, k] = n
            if n > cap:
                row_overflows = True
        if row_overflows:
            ovf.append(t)
    ovf_rows = np.array(ovf, dtype=np.int32)
    dense = storage_zero((len(ovf), F), dtype)
    for r, t in enumerate(ovf):
        for j in range(F):
            if act[t, j]:
                dense[r, j] = pre[t, j]
    return Packed(dtype, tile, cap, cnt, val, idx, ovf_rows, dense)


def pack(pre: np.ndarray, dtype: str, tile: int, cap: int) -> Packed:
    """Vectorised packer: same result as ``pack_loop`` for any input."""
    T, F, nt = _check(pre, dtype, tile, cap)
    pre3 = pre.reshape(T, nt, tile)
    act = active(pre3, dtype)
    cnt = act.sum(axis=2, dtype=np.int64)
    # rank of each active column among the active columns of its tile
    rank = np.cumsum(act, axis=2, dtype=np.int32) - 1
    keep = act & (rank < cap)
    t_i, k_i, c_i = np.nonzero(keep)
    s_i = rank[t_i, k_i, c_i]
    val = storage_zero((T, nt, cap), dtype)
    idx = np.zeros((T, nt, cap), dtype=np.uint8)
    val[t_i, k_i, s_i] = pre3[t_i, k_i, c_i]
    idx[t_i, k_i, s_i] = c_i.astype(np.uint8)
    ovf_rows = np.nonzero((cnt > cap).any(axis=1))[0].astype(np.int32)
    dense = relu_storage(pre[ovf_rows], dtype) if ovf_rows.size else storage_zero((0, F), dtype)
    return Packed(dtype, tile, cap, cnt.astype(np.uint16), val, idx, ovf_rows, dense)


def unpack(p: Packed) -> np.ndarray:
    """Dense [T, F] storage tensor described by a TwELL matrix (+ dense backup rows)."""
    T, F = p.shape
    nt = F // p.tile
    out = storage_zero((T, nt, p.tile), p.dtype)
    n = np.minimum(p.cnt.astype(np.int64), p.cap)
    slot = np.arange(p.cap)[None, None, :]
    used = slot < n[:, :, None]
    t_i, k_i, s_i = np.nonzero(used)
    out[t_i, k_i, p.idx[t_i, k_i, s_i].astype(np.int64)] = p.val[t_i, k_i, s_i]
    out = out.reshape(T, F)
    if p.n_ovf:
        out[p.ovf_rows] = p.dense
    return out


def tile_major(p: Packed):
    """The records of ``p`` in the tile-major layout of ``include/twell.h``
    (``twell_layout``): the record of (row t, tile k) -- count and cap slots --
    moves from position t * nt + k to k * T + t, so that a tile's records are
    contiguous over the tokens (the hidden-tile-major walk of the fused
    inference kernel, gist.science Resumen Técnico §2.B).  A change of order
    only: every record is kept whole.  Returns (cnt [nt, T], val [nt, T, cap],
    idx [nt, T, cap])."""
    return (np.ascontiguousarray(p.cnt.transpose(1, 0)), np.ascontiguousarray(p.val.transpose(1, 0, 2)),
            np.ascontiguousarray(p.idx.transpose(1, 0, 2)))


def sparse_ffn(p: Packed, x: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """y from the packed gate activations, one active entry at a time (float64).

    For every row: gather the active hidden units from the TwELL slots (or from
    the dense backup row when the row overflowed), form u = x_t . W_u^T[j] for
    those units only, and sum h * u * W_d[j].  This is the sparse route of the
    gist.science summary, Resumen Técnico §2.B, written without any blocking.
    """
    T, F = p.shape
    X = decode(x, p.dtype)
    WU = decode(w_up, p.dtype)
    WD = decode(w_down, p.dtype)
    y = np.zeros((T, X.shape[1]), dtype=np.float64)
    ovf_pos = {int(t): r for r, t in enumerate(p.ovf_rows)}
    for t in range(T):
        if t in ovf_pos:
            hrow = decode(p.dense[ovf_pos[t]], p.dtype)
            js = np.nonzero(hrow)[0]
            hs = hrow[js]
        else:
            js_l, hs_l = [], []
            for k in range(F // p.tile):
                for s in range(min(int(p.cnt[t, k]), p.cap)):
                    js_l.append(k * p.tile + int(p.idx[t, k, s]))
                    hs_l.append(p.val[t, k, s])
            js = np.array(js_l, dtype=np.int64)
            hs = decode(np.array(hs_l, dtype=p.val.dtype), p.dtype)
        if js.size == 0:
            continue
        u = WU[js] @ X[t]
        y[t] = (hs * u) @ WD[js]
    return y
