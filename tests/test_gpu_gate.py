"""GPU parity: the gate matmul with the TwELL epilogue (twell_gate_pack).

Two kinds of input:
* exact: integer-valued operands whose fp32 accumulation is exact in any order,
  so the rounded pre-activations and the TwELL matrix are unique and must match
  the oracle (round the float64 gate, then pack) bit for bit;
* Gaussian: the float64 gate with a forward error bound decides every entry
  whose sign is certain; the remaining ones are checked for validity.
"""

import numpy as np
import pytest

from oracle.ffn import gate_pre
from oracle.numerics import decode, round_to_storage
from oracle.twell import pack
from workloads.synth import ffn_inputs

from gpu_util import (assert_bitwise, assert_packed_equal, check_fused_pack, dev_inputs, exact_gate_inputs,
                      from_dev, gate_bound, packed_to_host)

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,rho", [
    ("bf16", 300, 512, 1024, 256, 16, 0.03),
    ("bf16", 70, 1024, 512, 128, 4, 0.05),
    ("bf16", 257, 2048, 2048, 256, 16, 0.01),
    ("f32", 64, 256, 1024, 128, 8, 0.02),
    ("f32", 100, 512, 512, 256, 4, 0.05),
])
def test_gate_pack_exact_inputs_bitwise(dtype, T, d, F, tile, cap, rho):
    print(f"gate exact {dtype} T={T} d={d} F={F} tile={tile} cap={cap}", flush=True)
    inp = exact_gate_inputs(T, d, F, dtype, seed=T + d, density=rho)
    x, wg, _, _, b = dev_inputs(inp)
    p, pre = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap, pre_out=True)
    pre64 = gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype)
    want_pre = round_to_storage(pre64, dtype)
    assert_bitwise(from_dev(pre, dtype), want_pre, "pre_out")
    ref = pack(want_pre, dtype, tile, cap)
    assert_packed_equal(packed_to_host(p, dtype), ref, check_dense=False)
    # the launch without the dump (the kernel the forward runs) gives the same matrix
    p2, _ = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap)
    assert_packed_equal(packed_to_host(p2, dtype), ref, check_dense=False)


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,bias", [
    ("bf16", 300, 512, 1024, 256, 16, -2.3263),
    ("bf16", 129, 1024, 2048, 128, 8, -1.6449),
    ("f32", 64, 256, 1024, 128, 8, -2.326),
    ("f32", 80, 512, 512, 256, 16, -1.0),
])
def test_gate_pack_gaussian_inputs(dtype, T, d, F, tile, cap, bias):
    print(f"gate gauss {dtype} T={T} d={d} F={F}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=3, gate_bias=bias)
    x, wg, _, _, b = dev_inputs(inp)
    p, pre = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap, pre_out=True)
    pre64, bound = gate_bound(inp)
    host = packed_to_host(p, dtype)
    check_fused_pack(host, pre64, bound, dtype, tile, cap)
    # the launch without the dump accumulates in the same order: the same matrix
    host2 = packed_to_host(tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap)[0], dtype)
    for f in ("cnt", "val", "idx"):
        assert_bitwise(host2[f], host[f], f)
    # the debugging dump agrees with the float64 gate within the bound plus one rounding
    g = decode(from_dev(pre, dtype), dtype)
    rel = 2.0 ** -8 if dtype == "bf16" else 0.0
    assert np.all(np.abs(g - pre64) <= bound + rel * (np.abs(pre64) + bound))


def test_gate_pack_without_bias_and_all_inactive():
    inp = ffn_inputs(40, 512, 512, "bf16", seed=8, gate_bias=-1e30)
    x, wg, _, _, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=256, cap=16)
    host = packed_to_host(p, "bf16")
    assert not host["cnt"].any() and host["n_ovf"] == 0
    assert not host["val"].any() and not host["idx"].any()
    p2, _ = tw.twell_gate_pack(x, wg, None, tile=256, cap=16)   # no bias: ~half active, all overflow
    host2 = packed_to_host(p2, "bf16")
    inp.gate_bias = None
    pre64, bound = gate_bound(inp)
    check_fused_pack(host2, pre64, bound, "bf16", 256, 16)
    assert host2["n_ovf"] == 40


@pytest.mark.slow
def test_gate_pack_full_size_sampled_rows():
    # 1.5B-class layer at full size: check a sample of rows against the float64 gate.
    from workloads import CONFIGS
    w = CONFIGS["layer_1p5b_bf16"]
    inp = w.inputs()
    x, wg, _, _, b = dev_inputs(inp)
    p, _ = tw.twell_gate_pack(x, wg, b, tile=w.tile, cap=w.cap)
    host = packed_to_host(p, w.dtype)
    rows = np.unique(np.concatenate([np.arange(0, w.T, 97), [w.T - 1]]))
    sub = type(inp)(inp.dtype, inp.x[rows], inp.w_gate, inp.w_up, inp.w_down, inp.gate_bias[rows], 0)
    pre64, bound = gate_bound(sub)
    check_fused_pack(host, pre64, bound, w.dtype, w.tile, w.cap, rows=rows)
    cnt = host["cnt"].astype(np.int64)
    # density sanity: about 1% of the gate units are active
    assert abs(cnt.sum() / (w.T * w.F) - 0.01) < 0.001
