"""Backward pass of the ReLU-gated FFN layer from its hybrid activations (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Training keeps the layer's gate activations in the hybrid format, which makes
them cheap to store for back-propagation (gist.science "Sparser, Faster,
Lighter Transformer Language Models", Resumen Técnico §2.A, hybrid format
for training), and computes the gradients with hybrid-times-dense and
dense-times-hybrid matrix products and a sparse transpose (same summary,
§2.B, training kernels).  The pages name those kernels but write no formula;
the gradients are those of the forward layer (``oracle/ffn.py``)

    u = x W_u^T,   a = h * u,   y = a W_d,   h = ReLU(pre),  pre = x W_g^T + beta

plus the L1 penalty lam * ||h||_1 of the training recipe (§2.B, training
strategy).  With dy = dL/dy given by the caller, the chain rule gives

    da    = dy W_d^T             (sampled where h is active: elsewhere unused)
    du    = da * h
    dpre  = (da * u + lam) * [h > 0]
    dx    = du W_u + dpre W_g
    dW_u  = du^T x,   dW_g = dpre^T x,   dW_d = a^T dy

with W_g, W_u, W_d the stored [F, d] weight arrays (so dW_* has their layout).

Readings taken here (the pages are silent on them):

* h is the stored activation matrix (storage dtype) that the forward used; the
  backward uses it as stored: the rounding of the forward is passed through
  as the identity, and ReLU's derivative is 1 where the stored h is active
  (IEEE h > 0) and 0 elsewhere (0 at pre = 0).
* u is recomputed from x and W_u (the forward keeps only h).
* The per-token gate bias gets no gradient: it is an input of the synthetic
  workloads, not a parameter of the layer.
* Inputs are finite.

Arithmetic: float64 on the exact values of the stored inputs, numpy matmul.
"""

from __future__ import annotations

import numpy as np

from .hybrid import Hybrid, unhybrid
from .numerics import decode
from .twell import active


def grads64(X, Wg, Wu, Wd, H, M, dY, lam: float) -> dict:
    """The gradients from float64 arrays: X [T,d], W* [F,d], H [T,F] (the
    activations), M [T,F] bool (where H is active), dY [T,d]."""
    U = X @ Wu.T
    A = H * U
    dA = dY @ Wd.T
    dU = np.where(M, dA * H, 0.0)
    dP = np.where(M, dA * U + lam, 0.0)
    return {
        "dx": dU @ Wu + dP @ Wg,
        "dw_gate": dP.T @ X,
        "dw_up": dU.T @ X,
        "dw_down": np.where(M, A, 0.0).T @ dY,
    }


def ffn_backward(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
                 h: np.ndarray, dy: np.ndarray, lam: float, dtype: str) -> dict:
    """Gradients (float64) of <dy, y> + lam ||h||_1 for stored inputs and the
    stored activation matrix h [T, F] (storage dtype)."""
    M = active(h, dtype)
    H = np.where(M, decode(h, dtype), 0.0)
    return grads64(decode(x, dtype), decode(w_gate, dtype), decode(w_up, dtype), decode(w_down, dtype),
                   H, M, decode(dy, dtype), float(lam))


def ffn_backward_hybrid(hy: Hybrid, F: int, x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                        w_down: np.ndarray, dy: np.ndarray, lam: float) -> dict:
    """The same gradients with the activations given in the hybrid format."""
    return ffn_backward(x, w_gate, w_up, w_down, unhybrid(hy, F), dy, lam, hy.dtype)
