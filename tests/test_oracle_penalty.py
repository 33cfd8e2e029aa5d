"""Pins for the oracle's L1 activation penalty and its gradient (CPU only)."""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.numerics import decode
from oracle.penalty import l1_grad, l1_grad_twell, l1_norm, l1_norm_twell
from oracle.twell import Packed, active, pack, relu_storage, unpack
from workloads.synth import pre_activations, to_storage


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_l1_norm_hand_values(dtype):
    h = to_storage(np.array([[0.5, 0.0, 2.0], [0.0, 0.25, 0.0]], np.float64), dtype)
    assert l1_norm(h, dtype) == 2.75
    assert l1_norm(h[:0], dtype) == 0.0
    inf = to_storage(np.array([[1.0, np.inf]], np.float64), dtype)
    assert l1_norm(inf, dtype) == math.inf


def test_l1_norm_is_exactly_rounded():
    # 1 + many tiny terms: a naive float64 loop would lose them
    h = np.array([[1.0] + [2.0 ** -60] * 1024], np.float32)
    assert l1_norm(h, "f32") == 1.0 + 1024 * 2.0 ** -60


@settings(max_examples=100, deadline=None)
@given(st.sampled_from(["f32", "bf16"]), st.integers(0, 2 ** 31), st.sampled_from([(4, 1), (8, 2), (16, 16)]))
def test_twell_norm_equals_norm_of_relu(dtype, seed, fmt):
    tile, cap = fmt
    pre = pre_activations(9, 4 * tile, dtype, seed=seed, density=0.2, hot_rows=(1, 5), hot_density=0.7)
    p = pack(pre, dtype, tile, cap)
    assert l1_norm_twell(p) == l1_norm(relu_storage(pre, dtype), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradient_matches_finite_differences(dtype):
    # d(lam ||h||_1)/dh_j = lam for active j (h_j > 0), in float64 on the decoded values
    lam = 2e-5
    pre = pre_activations(4, 32, dtype, seed=3, density=0.3)
    h = relu_storage(pre, dtype)
    g = decode(l1_grad(h, dtype, lam), dtype)
    H = decode(h, dtype)
    eps = 1e-3
    for t, j in zip(*np.nonzero(active(h, dtype))):
        Hp = H.copy()
        Hp[t, j] += eps
        fd = lam * (np.abs(Hp).sum() - np.abs(H).sum()) / eps
        assert abs(fd - lam) <= 1e-9 and abs(g[t, j] - lam) <= lam * 2.0 ** -8
    assert not g[~active(h, dtype)].any()


@settings(max_examples=100, deadline=None)
@given(st.sampled_from(["f32", "bf16"]), st.integers(0, 2 ** 31), st.sampled_from([(4, 1), (8, 2), (16, 16)]))
def test_twell_gradient_has_the_twell_pattern(dtype, seed, fmt):
    tile, cap = fmt
    lam = 2e-5
    pre = pre_activations(7, 3 * tile, dtype, seed=seed, density=0.25, hot_rows=(2,), hot_density=0.8,
                          specials=True)
    p = pack(pre, dtype, tile, cap)
    gv, gd = l1_grad_twell(p, lam)
    # unpacking the gradient with the matrix's own pattern gives the dense gradient
    gp = Packed(p.dtype, p.tile, p.cap, p.cnt, gv, p.idx, p.ovf_rows, gd)
    want = l1_grad(relu_storage(pre, dtype), dtype, lam)
    assert np.array_equal(unpack(gp).view(np.uint8), want.view(np.uint8))
    # padding slots are +0
    used = np.arange(cap)[None, None, :] < np.minimum(p.cnt.astype(np.int64), cap)[:, :, None]
    assert not gv[~used].view(np.uint8).any()
