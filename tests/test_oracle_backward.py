"""Pins for the oracle's FFN backward pass (CPU only).

The oracle's gradients are checked against two derivations that share nothing
with its formulas: torch's automatic differentiation of the forward layer
(float64, on the CPU), and central finite differences of the loss.  Closed
forms cover the L1 term alone and the all-inactive case.
"""

import numpy as np
import pytest
import torch

from oracle.backward import ffn_backward, ffn_backward_hybrid, grads64
from oracle.ffn import gate_pre, rel_l2
from oracle.hybrid import hybrid
from oracle.numerics import decode, round_to_storage
from oracle.twell import relu_storage
from workloads.synth import ffn_inputs, gate_bias_for_density, grad_output

KEYS = ("dx", "dw_gate", "dw_up", "dw_down")


def _case(T, d, F, dtype, seed, rho):
    inp = ffn_inputs(T, d, F, dtype, seed=seed, gate_bias=gate_bias_for_density(rho))
    pre = gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype)
    h = relu_storage(round_to_storage(pre, dtype), dtype)  # the stored activations
    dy = grad_output(T, d, dtype, seed=seed)
    return inp, h, dy


def _autograd(inp, h, dy, lam):
    """torch autograd of <dy, y> + lam * sum(h), the stored h passed straight through."""
    dt = inp.dtype
    t = lambda a: torch.tensor(decode(a, dt), dtype=torch.float64, requires_grad=True)
    X, Wg, Wu, Wd = t(inp.x), t(inp.w_gate), t(inp.w_up), t(inp.w_down)
    beta = torch.tensor(np.asarray(inp.gate_bias, np.float32).astype(np.float64))[:, None]
    hs = torch.tensor(decode(h, dt), dtype=torch.float64)
    pre = X @ Wg.T + beta
    hr = torch.relu(pre)
    hh = hr + (hs - hr).detach()  # value: the stored h; derivative: ReLU's
    y = (hh * (X @ Wu.T)) @ Wd
    loss = (y * torch.tensor(decode(dy, dt), dtype=torch.float64)).sum() + lam * hh.sum()
    loss.backward()
    return {"dx": X.grad.numpy(), "dw_gate": Wg.grad.numpy(), "dw_up": Wu.grad.numpy(),
            "dw_down": Wd.grad.numpy()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,d,F,seed,rho,lam", [(5, 16, 24, 0, 0.3, 0.0), (7, 32, 64, 1, 0.1, 2e-5),
                                                (3, 8, 40, 2, 0.5, 0.25), (12, 24, 16, 3, 0.05, 1.0)])
def test_matches_autograd(dtype, T, d, F, seed, rho, lam):
    inp, h, dy = _case(T, d, F, dtype, seed, rho)
    lam = float(np.float32(lam))
    ref = _autograd(inp, h, dy, lam)
    got = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, lam, dtype)
    for k in KEYS:
        assert got[k].shape == ref[k].shape
        assert rel_l2(got[k], ref[k]) <= 1e-12, k


def test_matches_finite_differences():
    rng = np.random.Generator(np.random.PCG64(11))
    T, d, F, lam = 4, 6, 10, 0.3
    X, Wg, Wu, Wd = (rng.standard_normal(s) for s in ((T, d), (F, d), (F, d), (F, d)))
    beta = rng.standard_normal((T, 1)) * 0.3
    dY = rng.standard_normal((T, d))

    def loss(X, Wg, Wu, Wd):
        pre = X @ Wg.T + beta
        h = np.maximum(pre, 0.0)
        y = (h * (X @ Wu.T)) @ Wd
        return float((y * dY).sum() + lam * h.sum())

    pre = X @ Wg.T + beta
    assert np.abs(pre).min() > 1e-3  # away from the kink
    g = grads64(X, Wg, Wu, Wd, np.maximum(pre, 0.0), pre > 0, dY, lam)
    params = {"dx": X, "dw_gate": Wg, "dw_up": Wu, "dw_down": Wd}
    eps = 1e-6
    for k, P in params.items():
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + eps
            lp = loss(X, Wg, Wu, Wd)
            P[idx] = old - eps
            lm = loss(X, Wg, Wu, Wd)
            P[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(fd - g[k])) <= 1e-6 * max(1.0, np.max(np.abs(fd))), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_l1_term_alone(dtype):
    # dy = 0: dx_t = lam * sum of W_g rows over t's active units,
    # dW_g[j] = lam * sum of x_t over the tokens where j is active, the rest 0
    inp, h, _ = _case(6, 16, 32, dtype, 4, 0.2)
    lam = 0.5
    dy = np.zeros_like(inp.x)
    got = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, lam, dtype)
    X, Wg, H = decode(inp.x, dtype), decode(inp.w_gate, dtype), decode(h, dtype)
    T, F = H.shape
    for t in range(T):
        want = sum((lam * Wg[j] for j in range(F) if H[t, j] > 0), np.zeros(Wg.shape[1]))
        assert np.allclose(got["dx"][t], want, rtol=1e-12, atol=1e-12)
    for j in range(F):
        want = sum((lam * X[t] for t in range(T) if H[t, j] > 0), np.zeros(X.shape[1]))
        assert np.allclose(got["dw_gate"][j], want, rtol=1e-12, atol=1e-12)
    assert not got["dw_up"].any() and not got["dw_down"].any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_inactive_gives_zero(dtype):
    inp, h, dy = _case(5, 16, 32, dtype, 5, 0.3)
    h0 = np.zeros_like(h)
    got = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h0, dy, 0.7, dtype)
    for k in KEYS:
        assert not got[k].any(), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width", [1, 3, 64])
def test_hybrid_form_is_the_same(dtype, width):
    inp, h, dy = _case(9, 16, 48, dtype, 6, 0.15)
    a = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, 2e-5, dtype)
    b = ffn_backward_hybrid(hybrid(h, dtype, width), 48, inp.x, inp.w_gate, inp.w_up, inp.w_down, dy, 2e-5)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k
