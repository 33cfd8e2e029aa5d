"""GPU parity: the sparse TwELL FFN forward and the dense baseline against the
float64 oracle (relative L2 error <= 1e-5 for fp32, <= 1e-2 for bf16, on all
rows of small cases that span several tiles and a ragged tail)."""

import numpy as np
import pytest

from oracle.numerics import decode
from workloads.synth import ffn_inputs

from gpu_util import (TOL, check_fused_pack, check_y, dev_inputs, exact_gate_inputs, from_dev, gate_bound,
                      packed_to_host)

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")

SMALL = [
    # dtype, T, d, F, tile, cap, bias (None = no bias; "hot" = skewed rows)
    ("f32", 64, 256, 1024, 128, 8, -2.326),        # the tiny fp32 layer
    ("f32", 100, 512, 512, 256, 4, -1.5),
    ("bf16", 300, 512, 1024, 256, 16, -2.3263),
    ("bf16", 130, 1024, 2048, 128, 8, -2.0537),
    ("bf16", 257, 2048, 2048, 256, 16, "hot"),      # overflow rows -> dense fallback
    ("bf16", 1, 512, 512, 256, 16, -1.0),
    ("bf16", 64, 512, 512, 256, 16, 6.0),          # everything active: every row overflows
    ("bf16", 70, 512, 768, 256, 16, -1e30),        # nothing active: y == 0
    ("bf16", 40, 5120, 512, 256, 16, -1.5),        # wide rows: 10 chunks per lane, 2 entries in flight
    ("bf16", 20, 8192, 512, 128, 8, -1.0),         # widest bf16 rows
    ("f32", 33, 2560, 512, 128, 8, -1.0),          # wide fp32 rows
    ("f32", 17, 4096, 256, 256, 16, -0.5),         # widest fp32 rows
    ("bf16", 24, 512, 8448, 256, 16, -2.0),        # many hidden units per output slice
    ("f32", 20, 256, 4352, 128, 8, -1.5),          # fp32, many hidden units per output slice
    ("bf16", 31, 512, 8192, 128, 8, -2.0),         # 64 tiles per row: every lane holds a tile count
    ("bf16", 29, 512, 8960, 128, 8, -2.0),         # 70 tiles per row (more than one lane's worth)
    ("bf16", 37, 512, 4096, 256, 64, -1.0),        # ~16% dense, cap 64: ~160 entries per unit group
    # the fallback in chunks of 768 (bf16, T = 1100) or 512 (fp32, T = 600) rows
    ("bf16", 1100, 512, 1024, 256, 16, 6.0),       # every row overflows: two chunks
    ("bf16", 1100, 512, 1024, 256, 16, -1.55),     # ~6% dense: ~890 rows overflow, the second chunk partly
    ("f32", 600, 256, 512, 128, 8, 3.0),           # every row overflows: two chunks
]


def _bias(spec, T):
    if isinstance(spec, str):
        b = np.full(T, -2.3263, np.float32)
        b[(np.arange(T) % 128) < 8] = -0.8416   # first 8 tokens of every 128: ~20% active
        return b
    return spec


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", SMALL)
def test_twell_ffn_forward(dtype, T, d, F, tile, cap, bias):
    print(f"ffn {dtype} T={T} d={d} F={F} tile={tile} cap={cap} bias={bias if np.isscalar(bias) else 'hot'}",
          flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T, gate_bias=_bias(bias, T))
    x, wg, wu, wd, b = dev_inputs(inp)
    packed = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True)
    y, packed = tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed)
    yh = from_dev(y, dtype)
    check_y(yh, inp, dtype)
    if isinstance(bias, float) and bias < -1e20:
        assert not decode(yh, dtype).any()
    # the TwELL side output is the gate's TwELL matrix
    host = packed_to_host(packed, dtype)
    pre64, bound = gate_bound(inp)
    check_fused_pack(host, pre64, bound, dtype, tile, cap)
    # dense backup rows hold ReLU(round(pre)) of the overflow rows
    rel = 2.0 ** -8 if dtype == "bf16" else 0.0
    for r, t in enumerate(host["ovf_rows"]):
        h = decode(host["dense"][r], dtype)
        want = np.where(pre64[t] > 0, pre64[t], 0.0)
        assert np.all(np.abs(h - want) <= bound[t] + rel * (np.abs(pre64[t]) + bound[t]))
    if bias == "hot":
        assert host["n_ovf"] > 0
    if bias in (6.0, 3.0):
        assert host["n_ovf"] == T
    if bias == -1.55:
        assert 768 < host["n_ovf"] < T


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", SMALL)
def test_dense_ffn_forward(dtype, T, d, F, tile, cap, bias):
    print(f"dense {dtype} T={T} d={d} F={F}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T, gate_bias=_bias(bias, T))
    x, wg, wu, wd, b = dev_inputs(inp)
    y = tw.dense_ffn_forward(x, wg, wu, wd, b)
    check_y(from_dev(y, dtype), inp, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_inputs_sparse_equals_dense_up_to_rounding(dtype):
    # integer-valued operands: the gate decisions are exact on both paths
    T, d, F = 200, 512, 1024
    inp = exact_gate_inputs(T, d, F, dtype, seed=1, density=0.02)
    inp.w_up = inp.w_up.copy()
    x, wg, wu, wd, b = dev_inputs(inp)
    ys, _ = tw.twell_ffn_forward(x, wg, wu, wd, b, tile=256, cap=16)
    yd = tw.dense_ffn_forward(x, wg, wu, wd, b)
    check_y(from_dev(ys, dtype), inp, dtype)
    check_y(from_dev(yd, dtype), inp, dtype)


def test_stage_entry_points_compose():
    T, d, F = 300, 512, 1024
    inp = ffn_inputs(T, d, F, "bf16", seed=4, gate_bias=_bias("hot", T))
    x, wg, wu, wd, b = dev_inputs(inp)
    y1, _ = tw.twell_ffn_forward(x, wg, wu, wd, b, tile=256, cap=16)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=256, cap=16)
    y2 = tw.twell_sparse_ffn(p, x, wg, wu, wd, b)
    assert np.array_equal(from_dev(y1, "bf16"), from_dev(y2, "bf16"))


def test_deterministic():
    T, d, F = 257, 1024, 2048
    inp = ffn_inputs(T, d, F, "bf16", seed=6, gate_bias=_bias("hot", T))
    x, wg, wu, wd, b = dev_inputs(inp)
    outs = [from_dev(tw.twell_ffn_forward(x, wg, wu, wd, b)[0], "bf16") for _ in range(3)]
    outs += [from_dev(tw.dense_ffn_forward(x, wg, wu, wd, b), "bf16") for _ in range(2)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.array_equal(outs[3], outs[4])


def test_zero_tokens():
    import torch
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((512, 512), dtype=torch.bfloat16, device="cuda:0")
    y, p = tw.twell_ffn_forward(x, w, w, w, None)
    assert y.shape == (0, 512) and int(p.n_ovf.item()) == 0
    assert tw.dense_ffn_forward(x, w, w, w, None).shape == (0, 512)


FUSED_SMALL = [c for c in SMALL if c[2] <= (4096 if c[0] == "bf16" else 2048)]


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", FUSED_SMALL)
def test_fused_up_down(dtype, T, d, F, tile, cap, bias):
    """twell_sparse_ffn_fused (up and down in one kernel) after the gate: y
    against the oracle, every row, and the overflow rows listed as by the
    two-kernel route."""
    print(f"fused {dtype} T={T} d={d} F={F} tile={tile} cap={cap} bias={bias if np.isscalar(bias) else 'hot'}",
          flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T + 1, gate_bias=_bias(bias, T))
    x, wg, wu, wd, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap, scan=False)
    y = tw.twell_sparse_ffn_fused(p, x, wg, wu, wd, b)
    yh = from_dev(y, dtype)
    check_y(yh, inp, dtype)
    n_fused = int(p.n_ovf.item())
    rows_fused = p.ovf_rows[:n_fused].cpu().numpy().copy()
    tw.twell_sparse_ffn(p, x, wg, wu, wd, b)
    assert int(p.n_ovf.item()) == n_fused
    assert np.array_equal(p.ovf_rows[:n_fused].cpu().numpy(), rows_fused)


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", FUSED_SMALL)
def test_grouped_up_down(dtype, T, d, F, tile, cap, bias):
    """twell_sparse_ffn_grouped (hidden-group-major fused kernel, fp32 partial
    rows per group added in group order) after the gate: y against the oracle,
    every row; repeated calls are bitwise equal."""
    print(f"grouped {dtype} T={T} d={d} F={F} tile={tile} cap={cap}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T + 2, gate_bias=_bias(bias, T))
    x, wg, wu, wd, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap, scan=False)
    y = tw.twell_sparse_ffn_grouped(p, x, wg, wu, wd, b)
    yh = from_dev(y, dtype)
    check_y(yh, inp, dtype)
    y2 = tw.twell_sparse_ffn_grouped(p, x, wg, wu, wd, b)
    assert np.array_equal(from_dev(y2, dtype), yh)


def test_fused_rejects_wide_rows():
    import torch
    inp = ffn_inputs(4, 8192, 512, "bf16", seed=1, gate_bias=-1.0)
    x, wg, wu, wd, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=256, cap=16, scan=False)
    with pytest.raises(tw.TwellError):
        tw.twell_sparse_ffn_fused(p, x, wg, wu, wd, b)
    torch.cuda.synchronize()
