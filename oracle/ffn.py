"""Float64 dense ReGLU feed-forward layer (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The layer (ReLU gate in place of SiLU; gate, up and down projections):

    pre = x W_g^T + beta          beta: one gate bias per token (or none)
    h   = ReLU(pre)
    u   = x W_u^T
    y   = (h * u) W_d

Sources: q2bstudio post on TwELL (fourth paragraph, SiLU swapped for ReLU);
gist.science "Sparser, Faster, Lighter Transformer Language Models", Resumen
Técnico §2.B (the inference kernel runs the up and down projections from the
gate activations) and §5 (only the activation changes).  Skipping inactive
units is exact, so this dense formula is the value the sparse path must reach.

Weights are stored as rows per hidden unit: ``w_gate`` [F, d] (= W_g^T),
``w_up`` [F, d] (= W_u^T), ``w_down`` [F, d] (= W_d).  All arithmetic is
float64 on the exact values of the stored inputs (numpy matmul).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .numerics import decode


def gate_pre(x: np.ndarray, w_gate: np.ndarray, gate_bias: Optional[np.ndarray],
             dtype: str) -> np.ndarray:
    """pre[t, j] = sum_k x[t, k] * w_gate[j, k] + beta[t], in float64."""
    pre = decode(x, dtype) @ decode(w_gate, dtype).T
    if gate_bias is not None:
        pre = pre + np.asarray(gate_bias, dtype=np.float32).astype(np.float64)[:, None]
    return pre


def ffn_from_h(h: np.ndarray, x: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               dtype: str) -> np.ndarray:
    """y = (h * (x W_u^T)) W_d for given float64 gate activations h [T, F]."""
    u = decode(x, dtype) @ decode(w_up, dtype).T
    return (h * u) @ decode(w_down, dtype)


def ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
        gate_bias: Optional[np.ndarray], dtype: str) -> np.ndarray:
    """The dense ReGLU FFN output y [T, d] in float64."""
    pre = gate_pre(x, w_gate, gate_bias, dtype)
    h = np.where(pre > 0, pre, 0.0)
    return ffn_from_h(h, x, w_up, w_down, dtype)


def rel_l2(y_test: np.ndarray, y_ref: np.ndarray) -> float:
    """||y_test - y_ref||_F / ||y_ref||_F (0 when both are all zero)."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y_test - y_ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def row_rel_l2(y_test: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per-row relative L2 error; rows whose reference is all zero give 0 or inf."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.linalg.norm(y_test - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = num / den
    return np.where(den == 0, np.where(num == 0, 0.0, np.inf), r)
