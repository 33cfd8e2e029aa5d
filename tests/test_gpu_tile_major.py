"""GPU parity of the tile-major TwELL layout (TWELL_LAYOUT_TILES): the record
of (row t, tile k) at position k * T + t.  It is written by the gate matmul's
TwELL epilogue, listed by the overflow scan and read by the hidden-group-major
fused up+down kernel (gist.science "Sparser, Faster, Lighter Transformer
Language Models", Resumen Técnico §2.B: the fused inference flow; the layout
keeps a tile's records of all tokens together for a walk over the hidden units
tile by tile).

* Exact gate inputs: the tile-major records equal the oracle's
  tile_major(pack(round(pre64))) bit for bit, and the overflow list equals the
  oracle's.
* Gaussian gate inputs: the records, put back in row order, pass the same
  float64-bound check as the row-major gate output.
* The grouped fused kernel over tile-major records: y against the float64
  oracle (relative L2 1e-5 fp32 / 1e-2 bf16, every row), and bit for bit the y
  of the same kernel over the row-major records of the same gate (the layout
  changes only where records are read from).
No GPU output enters an expectation of the oracle comparisons.
"""

import numpy as np
import pytest

from oracle.ffn import gate_pre
from oracle.numerics import round_to_storage
from oracle.twell import pack, tile_major
from workloads.synth import ffn_inputs

from gpu_util import (assert_bitwise, check_fused_pack, check_y, dev_inputs, exact_gate_inputs, from_dev,
                      gate_bound, packed_to_host)

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


def _tiles(T, F, tile, cap, x):
    return tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True, layout="tiles")


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,rho", [
    ("bf16", 300, 512, 1024, 256, 16, 0.03),
    ("bf16", 70, 1024, 512, 128, 4, 0.05),      # cap 4 at 5%: overflow rows
    ("bf16", 257, 2048, 2048, 256, 16, 0.01),
    ("f32", 64, 256, 1024, 128, 8, 0.02),
    ("f32", 100, 512, 512, 256, 4, 0.05),
])
def test_gate_tile_major_exact_inputs_bitwise(dtype, T, d, F, tile, cap, rho):
    print(f"tile-major gate exact {dtype} T={T} d={d} F={F} tile={tile} cap={cap}", flush=True)
    inp = exact_gate_inputs(T, d, F, dtype, seed=T + d, density=rho)
    x, wg, _, _, b = dev_inputs(inp)
    p, pre = tw.twell_gate_pack(x, wg, b, packed=_tiles(T, F, tile, cap, x), pre_out=True)
    want_pre = round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype), dtype)
    assert_bitwise(from_dev(pre, dtype), want_pre, "pre_out (row-major whatever the TwELL layout)")
    ref = pack(want_pre, dtype, tile, cap)
    cnt_t, val_t, idx_t = tile_major(ref)
    host = packed_to_host(p, dtype)
    assert_bitwise(host["cnt"], cnt_t, "cnt")
    assert_bitwise(host["val"], val_t, "val")
    assert_bitwise(host["idx"], idx_t, "idx")
    assert host["n_ovf"] == ref.n_ovf
    assert_bitwise(host["ovf_rows"].astype(np.int32), ref.ovf_rows.astype(np.int32), "ovf_rows")
    if rho >= 0.05 and cap == 4:
        assert ref.n_ovf > 0, "the case must hold overflow rows"


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", [
    ("bf16", 300, 512, 1024, 256, 16, -2.3263),
    ("bf16", 129, 1024, 2048, 128, 8, -1.6449),
    ("f32", 80, 512, 512, 256, 16, -1.0),
])
def test_gate_tile_major_gaussian_inputs(dtype, T, d, F, tile, cap, bias):
    print(f"tile-major gate gauss {dtype} T={T} d={d} F={F}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=5, gate_bias=bias)
    x, wg, _, _, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, packed=_tiles(T, F, tile, cap, x))
    host = packed_to_host(p, dtype)
    rows = dict(host, cnt=host["cnt"].T, val=host["val"].transpose(1, 0, 2), idx=host["idx"].transpose(1, 0, 2))
    pre64, bound = gate_bound(inp)
    check_fused_pack(rows, pre64, bound, dtype, tile, cap)


GROUPED = [
    # dtype, T, d, F, tile, cap, bias ("hot": every 128th token block starts with 8 denser rows)
    ("f32", 64, 256, 1024, 128, 8, -2.326),
    ("bf16", 300, 512, 1024, 256, 16, -2.3263),
    ("bf16", 130, 1024, 2048, 128, 8, -2.0537),
    ("bf16", 257, 2048, 2048, 256, 16, "hot"),      # overflow rows -> dense fallback
    ("bf16", 64, 512, 512, 256, 16, 6.0),          # every row overflows
    ("bf16", 24, 512, 8448, 256, 16, -2.0),        # many tiles per row
    ("f32", 100, 512, 512, 256, 4, -1.5),
]


def _bias(spec, T):
    if isinstance(spec, str):
        b = np.full(T, -2.3263, np.float32)
        b[(np.arange(T) % 128) < 8] = -0.8416
        return b
    return spec


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", GROUPED)
def test_grouped_over_tile_major(dtype, T, d, F, tile, cap, bias):
    print(f"grouped tile-major {dtype} T={T} d={d} F={F} tile={tile} cap={cap}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T + 7, gate_bias=_bias(bias, T))
    x, wg, wu, wd, b = dev_inputs(inp)
    pt, _ = tw.twell_gate_pack(x, wg, b, packed=_tiles(T, F, tile, cap, x), scan=False)
    y_t = tw.twell_sparse_ffn_grouped(pt, x, wg, wu, wd, b)
    yh = from_dev(y_t, dtype)
    check_y(yh, inp, dtype)
    pr, _ = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap, scan=False)
    y_r = tw.twell_sparse_ffn_grouped(pr, x, wg, wu, wd, b)
    assert_bitwise(yh, from_dev(y_r, dtype), "y over tile-major vs row-major records")
    assert int(pt.n_ovf.item()) == int(pr.n_ovf.item())


@pytest.mark.slow
@pytest.mark.parametrize("name", ["layer_1p5b_bf16", "skewed_bf16"])
def test_grouped_over_tile_major_full_size(name):
    """Full shapes in the launch configuration the bench times, on sampled rows
    (the skewed layer's overflow rows included)."""
    from workloads.configs import workload
    w = workload(name)
    print(f"grouped tile-major full size {name}", flush=True)
    inp = w.inputs()
    x, wg, wu, wd, b = dev_inputs(inp)
    pt, _ = tw.twell_gate_pack(x, wg, b, packed=_tiles(w.T, w.F, w.tile, w.cap, x), scan=False)
    y = tw.twell_sparse_ffn_grouped(pt, x, wg, wu, wd, b)
    yh = from_dev(y, w.dtype)
    n_ovf = int(pt.n_ovf.item())
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(w.T, 24, replace=False), pt.ovf_rows[:min(n_ovf, 8)].cpu().numpy()]))
    check_y(yh, inp, w.dtype, rows=rows)


def test_tile_major_empty_batch():
    """T = 0: the gate writes nothing and the grouped kernel returns an empty y
    with n_ovf = 0."""
    import torch
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((512, 512), dtype=torch.bfloat16, device="cuda:0")
    pt = tw.TwellMatrix.empty(0, 512, 256, 16, x.dtype, x.device, 0, dense=True, layout="tiles")
    tw.twell_gate_pack(x, w, None, packed=pt)
    y = tw.twell_sparse_ffn_grouped(pt, x, w, w, w, None)
    torch.cuda.synchronize()
    assert y.shape == (0, 512) and int(pt.n_ovf.item()) == 0
