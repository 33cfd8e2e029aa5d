"""twell_ffn_forward_noalloc (the forward with its workspace in the library's
static device scratch, for callers that cannot allocate) against the
allocating twell_ffn_forward on the same inputs, through the C ABI: three
calls in a row on one GPU, each smaller than the one before, so every call
after the first runs over the scratch the previous one left behind.

The two entry points run the same kernels with the same fallback chunking at
these shapes, so the TwELL matrix (integer and bit-copy work) must agree bit
for bit and y must too; y is also held to the float64 oracle's tolerance."""

import numpy as np
import pytest

from oracle.ffn import rel_l2
from oracle.numerics import decode
from workloads import CONFIGS
from workloads.synth import ffn_inputs

from gpu_util import TOL, assert_bitwise, check_y, dev_inputs, from_dev, packed_to_host

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


def _hot_bias(T):
    b = np.full(T, -2.3263, np.float32)
    b[(np.arange(T) % 128) < 8] = -0.8416   # first 8 tokens of every 128: ~20% active, rows overflow
    return b


def _case(name):
    if name == "layer_1p5b_bf16":
        w = CONFIGS[name]
        return w.inputs(), w.tile, w.cap
    if name == "mid_hot_bf16":
        return ffn_inputs(1024, 2048, 8192, "bf16", seed=21, gate_bias=_hot_bias(1024)), 256, 16
    return ffn_inputs(300, 512, 1024, "bf16", seed=22, gate_bias=-2.3263), 256, 16


def test_noalloc_matches_allocating_forward():
    import torch
    for name in ("layer_1p5b_bf16", "mid_hot_bf16", "small_bf16"):
        inp, tile, cap = _case(name)
        T, d = inp.x.shape
        F = inp.w_gate.shape[0]
        print(f"noalloc {name} T={T} d={d} F={F}", flush=True)
        x, wg, wu, wd, b = dev_inputs(inp)
        p_ref = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True)
        y_ref, _ = tw.twell_ffn_forward(x, wg, wu, wd, b, packed=p_ref)
        p_na = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True)
        y_na = torch.empty_like(y_ref)
        tw.twell_ffn_forward_noalloc(x, wg, wu, wd, p_na, y_na, b)
        torch.cuda.synchronize()
        h_ref, h_na = packed_to_host(p_ref, "bf16"), packed_to_host(p_na, "bf16")
        assert h_na["n_ovf"] == h_ref["n_ovf"]
        for k in ("cnt", "val", "idx", "ovf_rows", "dense"):
            assert_bitwise(h_na[k], h_ref[k], f"{name}: {k}")
        yr, yn = from_dev(y_ref, "bf16"), from_dev(y_na, "bf16")
        assert rel_l2(decode(yn, "bf16"), decode(yr, "bf16")) <= TOL["bf16"]
        assert_bitwise(yn, yr, f"{name}: y")
        rows = None if T <= 1024 else np.unique(np.r_[np.arange(0, T, 97), T - 1])
        check_y(yn, inp, "bf16", rows=rows)
        if name == "mid_hot_bf16":
            assert h_na["n_ovf"] > 0, "the case must exercise the dense fallback"
