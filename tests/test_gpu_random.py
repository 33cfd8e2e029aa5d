"""GPU parity on seeded random shapes: forward (two-kernel, fused, and the
hidden-group-major fused kernel over tile-major records), the training forward
that saves u, TwELL -> hybrid, and backward (u recomputed, and u carried from
the TwELL matrix), each against the oracle, over shapes, tiles, capacities,
densities and ELL widths drawn within the documented limits.

The cases are drawn once from a fixed seed, so every run checks the same
ones; each prints its parameters before it runs.
"""

import numpy as np
import pytest

from oracle.backward import ffn_backward
from oracle.ffn import gate_pre, rel_l2
from oracle.hybrid import hybrid
from oracle.numerics import decode, round_to_storage
from oracle.twell import pack, relu_storage
from workloads.synth import ffn_inputs, gate_bias_for_density, grad_output

from gpu_util import TOL, assert_bitwise, check_y, dev_inputs, from_dev, packed_to_host, to_dev, torch_dtype
from test_gpu_saved_u import _check_forward_u, _slot_units, _u64

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


def _cases(n=14, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = str(rng.choice(["bf16", "f32"]))
        q = 512 if dtype == "bf16" else 256
        d = int(q * rng.integers(1, 9 if dtype == "bf16" else 9))  # the backward takes up to 8 chunks
        tile = int(rng.choice([128, 256]))
        F = int(tile * rng.integers(1, 13))
        cap = int(rng.choice([1, 4, 8, 16, 32, min(64, tile)]))
        T = int(rng.integers(1, 300))
        rho = float(rng.choice([0.002, 0.01, 0.03, 0.1]))
        n_hot = int(rng.integers(0, 4))
        hot = tuple(int(v) for v in rng.choice(T, size=min(n_hot, T), replace=False))
        width = int(rng.choice([1, 4, 16, 64, 256]))
        out.append((dtype, T, d, F, tile, cap, rho, hot, width))
    return out


CASES = _cases()


def _bias(T, rho, hot):
    b = np.full(T, gate_bias_for_density(rho))
    if hot:
        b[np.asarray(hot)] = gate_bias_for_density(0.4)
    return b


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,rho,hot,width", CASES)
def test_random_case(dtype, T, d, F, tile, cap, rho, hot, width):
    import torch
    print(f"random {dtype} T={T} d={d} F={F} tile={tile} cap={cap} rho={rho} hot={hot} width={width}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T * 7 + d + F, gate_bias=_bias(T, rho, hot))
    x, wg, wu, wd, b = dev_inputs(inp)
    fused_ok = d <= (4096 if dtype == "bf16" else 2048)

    # forward, two-kernel route (with the dense backup rows)
    packed = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True)
    y, packed = tw.twell_ffn_forward(x, wg, wu, wd, b, packed=packed)
    check_y(from_dev(y, dtype), inp, dtype)
    # forward, fused up+down; the hidden-group-major one also over tile-major records
    if fused_ok:
        p2, _ = tw.twell_gate_pack(x, wg, b, tile=tile, cap=cap, scan=False)
        check_y(from_dev(tw.twell_sparse_ffn_fused(p2, x, wg, wu, wd, b), dtype), inp, dtype)
        pt = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True, layout="tiles")
        tw.twell_gate_pack(x, wg, b, packed=pt, scan=False)
        check_y(from_dev(tw.twell_sparse_ffn_grouped(pt, x, wg, wu, wd, b), dtype), inp, dtype)
    # the training forward saving u: y bit for bit the same, every saved u within
    # the fp32 bound of its float64 dot product
    pu = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True, u=True)
    yu, _ = tw.twell_ffn_forward(x, wg, wu, wd, b, packed=pu)
    assert_bitwise(from_dev(yu, dtype), from_dev(y, dtype), "y with u")
    _check_forward_u(pu.u.cpu().numpy(), packed_to_host(pu, dtype), inp, tile, cap, np.arange(T))

    # TwELL -> hybrid on an oracle-packed matrix, bit for bit
    h = relu_storage(round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype), dtype), dtype)
    ref_p = pack(h, dtype, tile, cap)
    pd = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True)
    pd.cnt.copy_(torch.from_numpy(ref_p.cnt.view(np.int16)))
    pd.val.copy_(to_dev(ref_p.val, dtype))
    pd.idx.copy_(torch.from_numpy(ref_p.idx))
    pd.n_ovf.fill_(ref_p.n_ovf)
    if ref_p.n_ovf:
        pd.ovf_rows[:ref_p.n_ovf].copy_(torch.from_numpy(ref_p.ovf_rows))
        pd.dense[:ref_p.n_ovf].copy_(to_dev(ref_p.dense, dtype))
    hy_dev = tw.twell_to_hybrid(pd, width)
    hy = hybrid(h, dtype, width)
    torch.cuda.synchronize()
    assert_bitwise(hy_dev.cnt.cpu().numpy(), hy.cnt, "cnt")
    assert_bitwise(from_dev(hy_dev.val, dtype), hy.val, "val")
    assert_bitwise(hy_dev.col.cpu().numpy(), hy.col, "col")
    assert int(hy_dev.n_dense.item()) == hy.n_dense
    assert_bitwise(hy_dev.dense_rows.cpu().numpy()[:hy.n_dense], hy.dense_rows, "dense_rows")
    if hy.n_dense:
        assert_bitwise(from_dev(hy_dev.dense, dtype)[:hy.n_dense], hy.dense, "dense")

    # backward from those hybrid activations, then again with the oracle's u
    # (float64 dot products rounded to fp32, NaN for overflow rows) carried
    # through the conversion
    if F <= 16384:
        dy = grad_output(T, d, dtype, seed=T + 1)
        lam = float(np.float32(2e-5))
        ref = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, lam, dtype)
        units = _slot_units(ref_p.cnt, ref_p.idx, tile, cap).reshape(T, -1)
        u64, _ = _u64(inp, np.arange(T), units)
        u32 = np.where(units >= 0, u64, 0.0).astype(np.float32)
        u32[(ref_p.cnt > cap).any(axis=1)] = np.nan
        pd.u = torch.from_numpy(np.ascontiguousarray(u32.reshape(ref_p.val.shape))).to(x.device)
        hy_u = tw.twell_to_hybrid(pd, width)
        for hy_in in (hy_dev, hy_u):
            dx, dwg, dwu, dwd = tw.twell_ffn_backward(hy_in, x, wg, wu, wd, to_dev(dy, dtype), lam)
            torch.cuda.synchronize()
            assert rel_l2(decode(from_dev(dx, dtype), dtype), ref["dx"]) <= TOL[dtype]
            for k, g in (("dw_gate", dwg), ("dw_up", dwu), ("dw_down", dwd)):
                err = rel_l2(g.cpu().numpy().astype(np.float64), ref[k])
                assert err <= 1e-5, f"{k}: {err:.3e}"
