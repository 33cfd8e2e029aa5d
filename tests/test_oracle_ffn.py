"""Pins for the float64 dense ReGLU FFN oracle (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.ffn import ffn, gate_pre, rel_l2, row_rel_l2
from workloads.synth import bf16_bits_to_f32, ffn_inputs, to_storage


def _exact_values(a, dtype):
    """Exact rationals of stored values, via the float32 route (independent of the oracle)."""
    f = bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)
    return [[Fraction(float(v)) for v in row] for row in np.atleast_2d(f)]


def _exact_ffn(inp):
    """Brute force in exact rational arithmetic, straight from the definition."""
    dt = inp.dtype
    X, G, U, D = (_exact_values(a, dt) for a in (inp.x, inp.w_gate, inp.w_up, inp.w_down))
    T, d, F = len(X), len(X[0]), len(G)
    beta = [Fraction(0)] * T if inp.gate_bias is None else \
        [Fraction(float(b)) for b in np.asarray(inp.gate_bias, np.float32)]
    Y = []
    for t in range(T):
        y = [Fraction(0)] * d
        for j in range(F):
            pre = sum(X[t][k] * G[j][k] for k in range(d)) + beta[t]
            if pre <= 0:
                continue
            up = sum(X[t][k] * U[j][k] for k in range(d))
            for c in range(d):
                y[c] += pre * up * D[j][c]
        Y.append(y)
    return Y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,d,F,seed", [(1, 2, 3, 0), (2, 8, 16, 1), (3, 5, 7, 2), (3, 8, 16, 3)])
def test_ffn_matches_exact_rational_brute_force(dtype, T, d, F, seed):
    rng = np.random.default_rng(100 + seed)
    bias = (rng.standard_normal(T) * 0.5).astype(np.float32)
    inp = ffn_inputs(T, d, F, dtype, seed=seed, gate_bias=bias)
    y = ffn(inp.x, inp.w_gate, inp.w_up, inp.w_down, inp.gate_bias, dtype)
    Y = _exact_ffn(inp)
    scale = max(1e-300, max(abs(float(v)) for row in Y for v in row))
    for t in range(T):
        for c in range(d):
            assert abs(y[t, c] - float(Y[t][c])) <= 1e-12 * scale


def test_identity_weights_closed_form():
    # d = F = 4, W_g = W_u = W_d = I, no bias: y = ReLU(x) * x.
    x = to_storage(np.array([[1.0, -2.0, 3.0, 0.5]]), "f32")
    eye = to_storage(np.eye(4), "f32")
    y = ffn(x, eye, eye, eye, None, "f32")
    assert np.array_equal(y, np.array([[1.0, 0.0, 9.0, 0.25]]))


def test_single_active_unit_is_rank_one_hand_worked():
    # x = [1, 2]; gate rows [1,0], [0,-1], [-1,-1] give pre = [1, -2, -3]:
    # only unit 0 fires with h = 1; u_0 = 3*1 + 1*2 = 5; W_d[0] = [2, -1]
    # so y = 1 * 5 * [2, -1] = [10, -5].  Units 1, 2 have large up/down rows that must not leak.
    x = to_storage(np.array([[1.0, 2.0]]), "bf16")
    wg = to_storage(np.array([[1.0, 0.0], [0.0, -1.0], [-1.0, -1.0]]), "bf16")
    wu = to_storage(np.array([[3.0, 1.0], [64.0, 64.0], [-32.0, 8.0]]), "bf16")
    wd = to_storage(np.array([[2.0, -1.0], [100.0, 100.0], [7.0, -7.0]]), "bf16")
    y = ffn(x, wg, wu, wd, None, "bf16")
    assert np.array_equal(y, np.array([[10.0, -5.0]]))


def test_relu_is_on_the_gate_only_and_bias_is_per_token():
    # Token 0: bias +1 -> pre = 1*1 + 1 = 2 > 0, u = -3 (negative up value passes through):
    #          y0 = 2 * (-3) * [1, 1] = [-6, -6].
    # Token 1: bias -5 -> pre = 1 - 5 = -4 -> inactive, y1 = 0 even though u = -3.
    x = to_storage(np.array([[1.0], [1.0]]), "f32")
    wg = to_storage(np.array([[1.0]]), "f32")
    wu = to_storage(np.array([[-3.0]]), "f32")
    wd = to_storage(np.array([[1.0, 1.0]]), "f32")
    y = ffn(x, wg, wu, wd, np.array([1.0, -5.0], np.float32), "f32")
    assert np.array_equal(y, np.array([[-6.0, -6.0], [0.0, 0.0]]))
    assert np.array_equal(gate_pre(x, wg, np.array([1.0, -5.0], np.float32), "f32"),
                          np.array([[2.0], [-4.0]]))


def test_transposed_operands_are_distinguished():
    # Non-square, asymmetric weights: token x = [1, 0, 0] selects column 0 of every
    # weight row.  gate rows: [1,5,5],[ -1,5,5] -> pre = [1, -1]; up rows: [2,9,9],[9,9,9]
    # -> u_0 = 2; down rows: [[1,2,3]] ... y = 1*2*[1,2,3] = [2,4,6].
    x = to_storage(np.array([[1.0, 0.0, 0.0]]), "f32")
    wg = to_storage(np.array([[1.0, 5.0, 5.0], [-1.0, 5.0, 5.0]]), "f32")
    wu = to_storage(np.array([[2.0, 9.0, 9.0], [9.0, 9.0, 9.0]]), "f32")
    wd = to_storage(np.array([[1.0, 2.0, 3.0], [50.0, 50.0, 50.0]]), "f32")
    assert np.array_equal(ffn(x, wg, wu, wd, None, "f32"), np.array([[2.0, 4.0, 6.0]]))


def test_all_inactive_gives_exact_zero():
    inp = ffn_inputs(5, 16, 32, "bf16", seed=4, gate_bias=-1e30)
    y = ffn(inp.x, inp.w_gate, inp.w_up, inp.w_down, inp.gate_bias, "bf16")
    assert not y.any()


def test_zero_gate_is_inactive():
    # pre exactly 0 -> ReLU gives 0 (no contribution) whatever u and W_d are.
    x = to_storage(np.array([[1.0, -1.0]]), "f32")
    wg = to_storage(np.array([[1.0, 1.0]]), "f32")
    wu = to_storage(np.array([[5.0, 0.0]]), "f32")
    wd = to_storage(np.array([[3.0, 3.0]]), "f32")
    assert not ffn(x, wg, wu, wd, None, "f32").any()


def test_rel_l2_helpers():
    a = np.array([[3.0, 4.0], [0.0, 0.0]])
    b = np.array([[3.0, 4.0 + 0.5], [0.0, 0.0]])
    assert rel_l2(b, a) == pytest.approx(0.1)
    r = row_rel_l2(b, a)
    assert r[0] == pytest.approx(0.1) and r[1] == 0.0
    assert rel_l2(np.zeros(3), np.zeros(3)) == 0.0
    assert rel_l2(np.ones(3), np.zeros(3)) == float("inf")
