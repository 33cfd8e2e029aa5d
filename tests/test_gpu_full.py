"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: y on sampled rows (every row the oracle computes is checked
one by one), the overflow list on all rows, and sparse == dense agreement."""

import numpy as np
import pytest

from workloads import CONFIGS, workload
from workloads.configs import SEQ

from gpu_util import check_y, dev_inputs, from_dev, packed_to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


def _rows(T, extra=()):
    r = np.arange(0, T, max(1, T // 48))
    return np.unique(np.concatenate([r, [T - 1], np.asarray(extra, dtype=np.int64)]))


@pytest.mark.parametrize("name", ["tiny_f32", "layer_1p5b_bf16", "skewed_bf16", "large_bf16"])
def test_full_size(name):
    w = CONFIGS[name]
    print(f"full {name}", flush=True)
    inp = w.inputs()
    x, wg, wu, wd, b = dev_inputs(inp)
    y, packed = tw.twell_ffn_forward(x, wg, wu, wd, b, tile=w.tile, cap=w.cap)
    yh = from_dev(y, w.dtype)
    hot = [t for t in range(w.T) if t % SEQ < 3]
    rows = _rows(w.T, hot)
    check_y(yh, inp, w.dtype, rows=rows)
    host = packed_to_host(packed, w.dtype)
    cnt = host["cnt"].astype(np.int64)
    ovf = np.nonzero((cnt > w.cap).any(axis=1))[0]
    assert host["n_ovf"] == ovf.size and np.array_equal(host["ovf_rows"], ovf)
    if name == "skewed_bf16":
        # the 20%-dense first tokens of each sequence overflow and take the dense path
        hot_rows = np.nonzero((np.arange(w.T) % SEQ) < w.hot_tokens)[0]
        assert np.isin(hot_rows, ovf).mean() > 0.95
        check_y(yh, inp, w.dtype, rows=hot_rows[::8])
    if w.T * w.F <= 8192 * 8192:
        yd = tw.dense_ffn_forward(x, wg, wu, wd, b)
        check_y(from_dev(yd, w.dtype), inp, w.dtype, rows=rows)


@pytest.mark.parametrize("rho", [0.001, 0.005, 0.02, 0.05, 0.10])
def test_density_sweep_points(rho):
    w = workload(f"sweep@{rho}")
    print(f"sweep {rho}", flush=True)
    inp = w.inputs()
    x, wg, wu, wd, b = dev_inputs(inp)
    y, packed = tw.twell_ffn_forward(x, wg, wu, wd, b, tile=w.tile, cap=w.cap)
    check_y(from_dev(y, w.dtype), inp, w.dtype, rows=_rows(w.T))


@pytest.mark.parametrize("name", ["layer_1p5b_bf16", "skewed_bf16", "large_bf16"])
def test_full_size_fused_up_down(name):
    """The fused up+down kernel at full size, as the benchmark times it (gate,
    then twell_sparse_ffn_fused): y on sampled rows, dense-fallback rows of the
    skewed workload included."""
    w = CONFIGS[name]
    print(f"full fused {name}", flush=True)
    inp = w.inputs()
    x, wg, wu, wd, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=w.tile, cap=w.cap, scan=False)
    y = tw.twell_sparse_ffn_fused(p, x, wg, wu, wd, b)
    hot = [t for t in range(w.T) if t % SEQ < 3]
    check_y(from_dev(y, w.dtype), inp, w.dtype, rows=_rows(w.T, hot))


def test_full_size_grouped_up_down():
    """The hidden-group-major fused prototype at the 1.5B-class shape, as the
    benchmark times it (gate, then twell_sparse_ffn_grouped): y on sampled rows."""
    w = CONFIGS["layer_1p5b_bf16"]
    print("full grouped layer_1p5b_bf16", flush=True)
    inp = w.inputs()
    x, wg, wu, wd, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=w.tile, cap=w.cap, scan=False)
    y = tw.twell_sparse_ffn_grouped(p, x, wg, wu, wd, b)
    check_y(from_dev(y, w.dtype), inp, w.dtype, rows=_rows(w.T))
