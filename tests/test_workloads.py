"""Input-generator checks: determinism, realised density, skew (CPU only)."""

from statistics import NormalDist

import numpy as np
import pytest

from oracle.ffn import gate_pre
from workloads import CONFIGS, ffn_inputs, gate_bias_for_density, workload
from workloads.configs import SEQ, SWEEP_DENSITIES


def test_same_seed_same_inputs():
    a = ffn_inputs(8, 64, 128, "bf16", seed=0, gate_bias=-1.0)
    b = ffn_inputs(8, 64, 128, "bf16", seed=0, gate_bias=-1.0)
    for f in ("x", "w_gate", "w_up", "w_down", "gate_bias"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = ffn_inputs(8, 64, 128, "bf16", seed=1, gate_bias=-1.0)
    assert not np.array_equal(a.x, c.x)


def test_gate_bias_closed_form():
    assert gate_bias_for_density(0.01) == pytest.approx(-2.3263478740408408)
    assert gate_bias_for_density(0.5) == pytest.approx(0.0, abs=1e-12)
    for rho in SWEEP_DENSITIES:
        # P(z + beta > 0) = P(z > -beta) = Phi(beta)
        assert NormalDist().cdf(gate_bias_for_density(rho)) == pytest.approx(rho)


def test_weight_scaling_variance():
    inp = ffn_inputs(4, 512, 1024, "f32", seed=0)
    assert np.var(inp.w_gate) == pytest.approx(1 / 512, rel=0.05)
    assert np.var(inp.w_down) == pytest.approx(1 / 1024, rel=0.05)
    assert np.var(inp.x) == pytest.approx(1.0, rel=0.05)


@pytest.mark.parametrize("name,rho", [("layer_1p5b_bf16", 0.01), ("tiny_f32", 0.01)])
def test_realised_density(name, rho):
    w = CONFIGS[name]
    T = min(w.T, 256)
    inp = w.inputs(T=T)
    pre = gate_pre(inp.x, inp.w_gate, inp.gate_bias, w.dtype)
    assert (pre > 0).mean() == pytest.approx(rho, rel=0.10)


def test_skewed_hot_rows():
    w = CONFIGS["skewed_bf16"]
    b = w.bias_vector()
    hot = (np.arange(w.T) % SEQ) < 64
    assert hot.sum() == 4 * 64
    assert np.all(b[hot] == np.float32(gate_bias_for_density(0.2)))
    assert np.all(b[~hot] == np.float32(gate_bias_for_density(0.01)))


def test_sweep_names():
    assert workload("sweep@0.05").density == 0.05
    assert workload("sweep@0.05").F == 8192
