"""GPU robustness of the forward and of the binding.

* Zero activations contribute nothing: a non-finite weight row of a unit that
  is inactive for a token must not reach that token's output (the sparse path
  never reads such a row; the list padding of the down projection reads
  zeros).  The reference is the float64 oracle with that unit's W_u and W_d
  rows replaced by zeros, which is the exact value for every token where the
  unit is inactive (gist.science "Sparser, Faster, Lighter Transformer
  Language Models", Resumen Técnico §2.B: the projections run only over the
  active gate units).
* A local column index at or above the tile width is taken modulo the tile
  width (the library documents this for malformed TwELL input).
* The Python binding rejects mismatched outputs and TwELL buffers before any
  launch, and leaves the outputs untouched.
"""

import numpy as np
import pytest

from workloads.synth import ffn_inputs

from gpu_util import check_y, dev_inputs, from_dev, gate_bound

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


@pytest.mark.parametrize("dtype,T,d,F,tile,cap", [
    ("bf16", 300, 512, 1024, 256, 64),
    ("f32", 130, 256, 1024, 128, 32),
])
@pytest.mark.parametrize("route", ["split", "fused"])
def test_nonfinite_rows_of_inactive_units(dtype, T, d, F, tile, cap, route):
    import torch
    print(f"nonfinite {route} {dtype} T={T} d={d} F={F}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=11, gate_bias=-2.3263)
    pre64, bound = gate_bound(inp)
    # unit 0: inactive for sure on these rows, active for sure on those
    off = np.nonzero(pre64[:, 0] < -bound[:, 0])[0]
    assert off.size > 0.9 * T
    x, wg, wu, wd, b = dev_inputs(inp)
    wu_bad, wd_bad = wu.clone(), wd.clone()
    wu_bad[0, ::3] = float("nan")
    wd_bad[0, ::2] = float("inf")
    wd_bad[0, 1::4] = float("nan")
    packed = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=False)
    if route == "split":
        y, packed = tw.twell_ffn_forward(x, wg, wu_bad, wd_bad, b, packed=packed)
    else:
        tw.twell_gate_pack(x, wg, b, packed=packed, scan=False)
        y = tw.twell_sparse_ffn_fused(packed, x, wg, wu_bad, wd_bad, b)
    torch.cuda.synchronize()
    assert int(packed.n_ovf.item()) == 0, "the case must not reach the dense fallback"
    # the oracle with unit 0's up and down rows zeroed: exact wherever unit 0 is inactive
    ref = inp.__class__(inp.dtype, inp.x, inp.w_gate, inp.w_up.copy(), inp.w_down.copy(), inp.gate_bias, inp.seed)
    ref.w_up[0] = 0
    ref.w_down[0] = 0
    assert bool(torch.isfinite(y[torch.from_numpy(off).to(y.device)].float()).all())
    check_y(from_dev(y, dtype), ref, dtype, rows=off)


def test_index_taken_modulo_tile():
    """Indices >= tile (malformed TwELL input) address the tile's own columns:
    the result equals that of the indices reduced modulo the tile width."""
    import torch
    T, d, F, tile, cap = 96, 512, 1024, 128, 8
    inp = ffn_inputs(T, d, F, "bf16", seed=5, gate_bias=-2.0)
    x, wg, wu, wd, b = dev_inputs(inp)
    packed, _ = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap)
    bad = tw.TwellMatrix(packed.rows, packed.cols, tile, cap, packed.dtype, packed.cnt, packed.val,
                         packed.idx.clone(), packed.ovf_rows, packed.n_ovf, None, packed.ovf_cap)
    bad.idx.add_(128)   # uint8: every index i becomes i + 128 (< 256), i.e. i modulo 128 is unchanged
    y_ok = tw.twell_sparse_ffn(packed, x, wg, wu, wd, b)
    y_bad = tw.twell_sparse_ffn(bad, x, wg, wu, wd, b)
    y_fused = tw.twell_sparse_ffn_fused(bad, x, wg, wu, wd, b)
    torch.cuda.synchronize()
    assert torch.equal(y_ok.view(torch.int16), y_bad.view(torch.int16))
    check_y(from_dev(y_fused, "bf16"), inp, "bf16")


def _bad_calls(x, wg, wu, wd, b, T, d, F, packed, y_sentinel):
    import torch
    dev = x.device
    wrong_rows = tw.TwellMatrix.empty(T - 1, F, 256, 16, x.dtype, dev, T)
    wrong_cols = tw.TwellMatrix.empty(T, F - 256, 256, 16, x.dtype, dev, T)
    wrong_dtype = tw.TwellMatrix.empty(T, F, 256, 16, torch.float32, dev, T)
    short_val = tw.TwellMatrix.empty(T, F, 256, 16, x.dtype, dev, T)
    short_val.val = short_val.val[:, :, :8]
    short_ovf = tw.TwellMatrix.empty(T, F, 256, 16, x.dtype, dev, T)
    short_ovf.ovf_rows = short_ovf.ovf_rows[:T // 2]
    yield "forward: y too small", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed,
                                                                 y=y_sentinel[:-1])
    yield "forward: y fp32", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed,
                                                            y=torch.empty((T, d), device=dev))
    yield "forward: packed rows", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=wrong_rows, y=y_sentinel)
    yield "forward: packed cols", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=wrong_cols, y=y_sentinel)
    yield "forward: packed dtype", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=wrong_dtype,
                                                                  y=y_sentinel)
    yield "forward: short val", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=short_val, y=y_sentinel)
    yield "forward: short ovf_rows", lambda: tw.twell_ffn_forward(x, wg, wu, wd, b, packed=short_ovf,
                                                                    y=y_sentinel)
    yield "forward: fp32 workspace", lambda: tw.twell_ffn_forward(
        x, wg, wu, wd, b, packed=packed, y=y_sentinel, workspace=torch.empty((1 << 20,), device=dev))
    yield "gate_pack: packed rows", lambda: tw.twell_gate_pack(x, wg, b, packed=wrong_rows)
    yield "gate_pack: packed dtype", lambda: tw.twell_gate_pack(x, wg, b, packed=wrong_dtype)
    yield "sparse_ffn: packed rows", lambda: tw.twell_sparse_ffn(wrong_rows, x, wg, wu, wd, b, y=y_sentinel)
    yield "sparse_ffn: y shape", lambda: tw.twell_sparse_ffn(packed, x, wg, wu, wd, b, y=y_sentinel.t())
    yield "fused: packed cols", lambda: tw.twell_sparse_ffn_fused(wrong_cols, x, wg, wu, wd, b, y=y_sentinel)
    yield "dense: y dtype", lambda: tw.dense_ffn_forward(x, wg, wu, wd, b, y=y_sentinel.float())
    yield "dense: y rows", lambda: tw.dense_ffn_forward(x, wg, wu, wd, b, y=y_sentinel[1:])
    pre = torch.zeros((T, F), dtype=x.dtype, device=dev)
    yield "pack: out rows", lambda: tw.twell_pack(pre, 256, 16, out=wrong_rows)
    yield "pack: out dtype", lambda: tw.twell_pack(pre, 256, 16, out=wrong_dtype)
    yield "pack: out cap", lambda: tw.twell_pack(pre, 256, 8, out=packed)
    yield "l1 grad: grad_val shape", lambda: tw.twell_l1_grad(packed, 1e-3, grad_val=packed.val[:, :, :4])
    yield "to_hybrid: short val", lambda: tw.twell_to_hybrid(short_val, 16)


def test_binding_rejects_mismatches():
    import torch
    T, d, F = 64, 512, 1024
    inp = ffn_inputs(T, d, F, "bf16", seed=3, gate_bias=-2.0)
    x, wg, wu, wd, b = dev_inputs(inp)
    packed = tw.TwellMatrix.empty(T, F, 256, 16, x.dtype, x.device, T)
    y = torch.full((T, d), 7.0, dtype=x.dtype, device=x.device)
    for what, call in _bad_calls(x, wg, wu, wd, b, T, d, F, packed, y):
        with pytest.raises((ValueError, TypeError)):
            call()
            pytest.fail(f"{what}: accepted")
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote its output"
