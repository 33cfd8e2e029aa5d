"""Pins for the oracle TwELL packer/unpacker and the sparse FFN route (CPU only)."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.ffn import ffn, ffn_from_h, rel_l2
from oracle.numerics import decode, round_to_storage
from oracle.twell import active, pack, pack_loop, relu_storage, sparse_ffn, tile_major, unpack
from workloads.synth import ffn_inputs, pre_activations, to_storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _storage(values, dtype):
    arr = np.array([[(-0.0 if v == "-0" else v) for v in row] for row in values], np.float64)
    return to_storage(arr, dtype)


def _assert_same(a, b):
    assert a.dtype == b.dtype and a.shape == b.shape
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def _assert_packed_equal(p, q):
    for f in ("cnt", "val", "idx", "ovf_rows", "dense"):
        _assert_same(getattr(p, f), getattr(q, f))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("packer", [pack, pack_loop])
def test_hand_worked_example(dtype, packer):
    g = _load("twell_pack_example.json")
    pre = _storage(g["pre"], dtype)
    p = packer(pre, dtype, g["tile"], g["cap"])
    assert p.cnt.tolist() == g["cnt"]
    _assert_same(p.val, _storage(np.array(g["val"]).reshape(2, -1), dtype).reshape(p.val.shape))
    assert p.idx.tolist() == g["idx"]
    assert p.ovf_rows.tolist() == g["ovf_rows"]
    _assert_same(p.dense, _storage(g["dense"], dtype))
    assert int(p.cnt.sum()) == g["nnz"]
    # the -0.0 of row 0 must come back as +0 in the dense row
    assert not np.signbit(decode(p.dense, dtype)).any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_special_values(dtype):
    g = _load("twell_special_values.json")
    bits = np.array([[int(b, 16) for b in g[f"{dtype}_bits"]]], dtype=np.uint64)
    pre = bits.astype(np.uint32).view(np.float32) if dtype == "f32" else bits.astype(np.uint16)
    assert np.nonzero(active(pre, dtype)[0])[0].tolist() == g["active_cols"]
    p = pack(pre, dtype, g["tile"], g["cap"])
    assert p.cnt.tolist() == g["cnt"]
    assert p.idx[0, 0, :2].tolist() == g["active_cols"]
    _assert_packed_equal(p, pack_loop(pre, dtype, g["tile"], g["cap"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_capacity_edge(dtype):
    # tile 8, cap 3: a tile with exactly 3 actives fits, 4 actives overflow the row.
    row_fit = [1, -1, 2, -1, 3, -1, -1, -1]
    row_ovf = [1, 2, -1, 3, 4, -1, -1, -1]
    pre = to_storage(np.array([row_fit, row_ovf, row_fit], np.float64), dtype)
    p = pack(pre, dtype, 8, 3)
    assert p.cnt[:, 0].tolist() == [3, 4, 3]
    assert p.ovf_rows.tolist() == [1]
    assert p.idx[1, 0].tolist() == [0, 1, 3]   # first three of the overflowing tile kept
    assert p.idx[0, 0].tolist() == [0, 2, 4]


_special_f32 = st.sampled_from([0.0, -0.0, 1e-45, -1e-45, float("inf"), float("-inf"),
                                float("nan"), 1.0, -1.0, 0.5])


@st.composite
def _pre_case(draw):
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    tile = draw(st.sampled_from([1, 2, 4, 8, 16, 32]))
    nt = draw(st.integers(1, 4))
    T = draw(st.integers(0, 6))
    cap = draw(st.integers(1, tile))
    seed = draw(st.integers(0, 2 ** 31))
    dens = draw(st.sampled_from([0.0, 0.05, 0.3, 0.7, 1.0]))
    rng = np.random.default_rng(seed)
    v = np.abs(rng.standard_normal((T, nt * tile))) + 1e-3
    v = np.where(rng.random((T, nt * tile)) < dens, v, -v)
    if draw(st.booleans()) and T * nt * tile:
        k = max(1, T * nt * tile // 5)
        specials = np.array([draw(_special_f32) for _ in range(k)])
        pos = rng.integers(0, T * nt * tile, size=k)
        v.reshape(-1)[pos] = specials
    return dtype, tile, cap, to_storage(v, dtype)


@settings(max_examples=300, deadline=None)
@given(_pre_case())
def test_vectorised_packer_equals_loop_packer(case):
    dtype, tile, cap, pre = case
    _assert_packed_equal(pack(pre, dtype, tile, cap), pack_loop(pre, dtype, tile, cap))


@settings(max_examples=300, deadline=None)
@given(_pre_case())
def test_invariants(case):
    dtype, tile, cap, pre = case
    p = pack(pre, dtype, tile, cap)
    relu = relu_storage(pre, dtype)
    # unpack(pack(H)) == ReLU(H) bit for bit
    _assert_same(unpack(p), relu)
    # counts sum to the non-zeros of ReLU(H)
    nz = active(pre, dtype)
    assert int(p.cnt.astype(np.int64).sum()) == int(nz.sum())
    T, F = pre.shape
    n = np.minimum(p.cnt.astype(np.int64), cap)
    for t in range(T):
        for k in range(F // tile):
            ids = p.idx[t, k, :n[t, k]].astype(np.int64)
            assert np.all(np.diff(ids) > 0) and np.all(ids < tile)
            # every kept slot is active and holds that column's bits
            assert active(pre[t, k * tile + ids], dtype).all()
            _assert_same(p.val[t, k, :n[t, k]], pre[t, k * tile + ids])
            # padding is +0 / 0
            assert not p.idx[t, k, n[t, k]:].any()
            assert not p.val[t, k, n[t, k]:].view(np.uint8).any()
    ovf = (p.cnt.astype(np.int64) > cap).any(axis=1)
    assert p.ovf_rows.tolist() == np.nonzero(ovf)[0].tolist()
    _assert_same(p.dense, relu[p.ovf_rows])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hot", [(), (0, 3)])
def test_sparse_route_equals_dense_route(dtype, hot):
    # Exactness of skipping zeros: entry-by-entry sparse FFN == dense FFN on the same h.
    T, d, F, tile, cap = 6, 16, 64, 16, 3
    inp = ffn_inputs(T, d, F, dtype, seed=11)
    pre = pre_activations(T, F, dtype, seed=12, density=0.08, hot_rows=hot, hot_density=0.6)
    p = pack(pre, dtype, tile, cap)
    if hot:
        assert set(hot) <= set(p.ovf_rows.tolist())
    y_sparse = sparse_ffn(p, inp.x, inp.w_up, inp.w_down)
    h = decode(relu_storage(pre, dtype), dtype)
    y_dense = ffn_from_h(h, inp.x, inp.w_up, inp.w_down, dtype)
    assert rel_l2(y_sparse, y_dense) <= 1e-12


def test_sparse_route_from_gate_matches_dense_ffn():
    # Gate computed in float64, rounded to the storage dtype, packed, run sparsely:
    # agrees with the dense float64 FFN up to the bf16 rounding of h.
    T, d, F = 16, 64, 256
    inp = ffn_inputs(T, d, F, "bf16", seed=5, gate_bias=-1.0)
    from oracle.ffn import gate_pre
    pre_s = round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, "bf16"), "bf16")
    p = pack(pre_s, "bf16", 64, 16)
    y = sparse_ffn(p, inp.x, inp.w_up, inp.w_down)
    y64 = ffn(inp.x, inp.w_gate, inp.w_up, inp.w_down, inp.gate_bias, "bf16")
    assert rel_l2(y, y64) <= 4 * 2.0 ** -9


def test_pack_rejects_bad_shapes():
    pre = to_storage(np.zeros((2, 10)), "f32")
    with pytest.raises(ValueError):
        pack(pre, "f32", 4, 2)
    with pytest.raises(ValueError):
        pack(to_storage(np.zeros((2, 8)), "f32"), "f32", 4, 5)
    with pytest.raises(ValueError):
        pack(to_storage(np.zeros((2, 8)), "f32"), "bf16", 4, 2)


@settings(max_examples=200, deadline=None)
@given(_pre_case())
def test_tile_major_records_rebuild_relu(case):
    """Tile-major layout (include/twell.h, twell_layout): the record of (row t,
    tile k) sits at flat position k * T + t.  Walking the flat arrays by that
    definition alone, one record at a time, must rebuild ReLU(H) bit for bit
    (overflow rows from the dense backup), independently of ``unpack``."""
    dtype, tile, cap, pre = case
    p = pack(pre, dtype, tile, cap)
    T, F = pre.shape
    nt = F // tile
    cnt_t, val_t, idx_t = tile_major(p)
    assert cnt_t.shape == (nt, T) and val_t.shape == (nt, T, cap) and idx_t.shape == (nt, T, cap)
    c, v, i = cnt_t.reshape(-1), val_t.reshape(-1, cap), idx_t.reshape(-1, cap)
    h = np.zeros_like(pre)
    h[...] = relu_storage(np.zeros_like(pre), dtype)  # +0 of the storage dtype
    overflow = np.zeros(T, dtype=bool)
    for t in range(T):
        for k in range(nt):
            r = k * T + t
            overflow[t] |= int(c[r]) > cap
            for s_ in range(min(int(c[r]), cap)):
                h[t, k * tile + int(i[r, s_])] = v[r, s_]
    for r_, t in enumerate(p.ovf_rows):
        h[t] = p.dense[r_]
    assert overflow.tolist() == [t in set(p.ovf_rows.tolist()) for t in range(T)]
    _assert_same(h, relu_storage(pre, dtype))


def test_tile_major_hand_example():
    """The golden example's counts in tile-major order, written out by hand:
    rows 0 and 1 of tile 0, then rows 0 and 1 of tile 1, ..."""
    g = _load("twell_pack_example.json")
    pre = _storage(g["pre"], "f32")
    p = pack(pre, "f32", g["tile"], g["cap"])
    cnt_t, _, idx_t = tile_major(p)
    T = len(g["cnt"])
    assert cnt_t.reshape(-1).tolist() == [g["cnt"][t][k] for k in range(len(g["cnt"][0])) for t in range(T)]
    assert idx_t.reshape(-1, g["cap"]).tolist() == [g["idx"][t][k] for k in range(len(g["idx"][0])) for t in range(T)]
