"""Pins for the oracle's hybrid training format (ELL rows + dense backup) and its
conversion from TwELL (CPU only)."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.hybrid import from_twell, hybrid, hybrid_loop, unhybrid
from oracle.numerics import round_to_bf16
from oracle.twell import active, pack, relu_storage
from workloads.synth import to_storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits_f32(rows):
    return np.array([[int(b, 16) for b in r] for r in rows], dtype=np.uint64).astype(np.uint32).view(np.float32)


def _same(a, b):
    assert a.dtype == b.dtype and a.shape == b.shape
    assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def _hy_equal(a, b):
    for f in ("cnt", "val", "col", "dense_rows", "dense"):
        _same(getattr(a, f), getattr(b, f))


@pytest.mark.parametrize("conv", [hybrid, hybrid_loop])
def test_hand_worked_example(conv):
    with open(os.path.join(GOLDEN, "hybrid_example.json")) as f:
        g = json.load(f)
    h = _bits_f32(g["f32_bits"])
    hy = conv(h, "f32", g["width"])
    assert hy.cnt.tolist() == g["cnt"]
    _same(hy.val, _bits_f32(g["val_bits"]))
    assert hy.col.tolist() == g["col"]
    assert hy.dense_rows.tolist() == g["dense_rows"]
    _same(hy.dense, _bits_f32(g["dense_bits"]))


def test_width_boundary_and_empty_rows():
    # a row with exactly `width` actives is an ELL row; one more makes it dense
    h = to_storage(np.array([[1, 2, -1, -1], [1, 2, 3, -1], [-1, -1, -1, -1]], np.float64), "bf16")
    hy = hybrid(h, "bf16", 2)
    assert hy.cnt.tolist() == [2, 3, 0]
    assert hy.dense_rows.tolist() == [1]
    assert hy.col[0].tolist() == [0, 1] and hy.col[2].tolist() == [0, 0]
    assert not hy.val[1].any()  # a dense row keeps no ELL entries


_special = st.sampled_from([0.0, -0.0, 1e-45, -1e-45, float("inf"), float("-inf"), float("nan"), 1.0, -1.0])


@st.composite
def _case(draw):
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    T = draw(st.integers(0, 7))
    F = draw(st.sampled_from([1, 3, 8, 16, 24]))
    width = draw(st.integers(1, 10))
    seed = draw(st.integers(0, 2 ** 31))
    dens = draw(st.sampled_from([0.0, 0.1, 0.4, 1.0]))
    rng = np.random.default_rng(seed)
    v = np.abs(rng.standard_normal((T, F))) + 1e-3
    v = np.where(rng.random((T, F)) < dens, v, -v)
    if draw(st.booleans()) and T * F:
        k = max(1, T * F // 4)
        pos = rng.integers(0, T * F, size=k)
        v.reshape(-1)[pos] = [draw(_special) for _ in range(k)]
    return dtype, width, to_storage(v, dtype)


@settings(max_examples=300, deadline=None)
@given(_case())
def test_vectorised_equals_loops(case):
    dtype, width, h = case
    _hy_equal(hybrid(h, dtype, width), hybrid_loop(h, dtype, width))


@settings(max_examples=300, deadline=None)
@given(_case())
def test_invariants(case):
    dtype, width, h = case
    hy = hybrid(h, dtype, width)
    T, F = h.shape
    relu = relu_storage(h, dtype)
    _same(unhybrid(hy, F), relu)                     # the format loses nothing
    act = active(h, dtype)
    assert hy.cnt.tolist() == act.sum(axis=1).tolist()
    assert hy.dense_rows.tolist() == np.nonzero(hy.cnt > width)[0].tolist()
    for t in range(T):
        n = int(hy.cnt[t]) if hy.cnt[t] <= width else 0
        cols = hy.col[t, :n]
        assert np.all(np.diff(cols) > 0) and np.all((0 <= cols) & (cols < F))
        assert act[t, cols].all()
        _same(hy.val[t, :n], h[t, cols])
        assert not hy.col[t, n:].any() and not hy.val[t, n:].view(np.uint8).any()
    _same(hy.dense, relu[hy.dense_rows])


@settings(max_examples=200, deadline=None)
@given(_case(), st.sampled_from([(1, 1), (4, 1), (4, 2), (8, 3), (8, 8)]))
def test_from_twell_is_the_hybrid_of_the_activations(case, fmt):
    # whatever the TwELL tile and capacity (rows overflowing TwELL included),
    # converting TwELL gives the hybrid of ReLU(pre)
    dtype, width, pre = case
    tile, cap = fmt
    T, F = pre.shape
    if F % tile:
        pre = np.ascontiguousarray(pre[:, : F - F % tile])
    if pre.shape[1] == 0:
        return
    _hy_equal(from_twell(pack(pre, dtype, tile, cap), width), hybrid(relu_storage(pre, dtype), dtype, width))


def test_bf16_values_are_carried_bit_for_bit():
    v = np.array([[0.1, -0.2, 0.3, 1e-40]], np.float64)   # 1e-40 is a bf16 denormal
    h = round_to_bf16(v)
    hy = hybrid(h, "bf16", 4)
    assert hy.cnt.tolist() == [3]
    _same(hy.val[0, :3], h[0, [0, 2, 3]])
