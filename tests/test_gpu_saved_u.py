"""GPU parity of the saved up-projection value u (the training forward's extra
output, carried through the hybrid conversion into the backward).

* Forward: with ``packed.u`` the up kernel stores u = x_t . W_u[j] of every used
  slot of a non-overflow row (NaN in every slot of an overflow row).  Each
  saved u is checked against the float64 dot product of the stored inputs,
  within the forward error bound of an fp32 accumulation (Higham,
  gamma_d * sum |x_k w_k|, x4 for the unspecified order), both for the plan
  that takes whole rows of d and the one that adds two halves.  y and the
  TwELL matrix must be bit for bit those of the same forward without u.
* Conversion: the hybrid's u of an ELL row equals the TwELL slots' u in the
  row's entry order, bit for bit; a row that overflowed TwELL is marked NaN.
* Backward: from a TwELL matrix and u built entirely on the CPU (the oracle's
  pack of round(x W_g^T + beta) and float64 dot products rounded to fp32),
  converted on the GPU, the backward that takes u from the hybrid matches the
  float64 oracle with the tolerances of the other backward tests, including
  rows whose u is marked as not saved.
No GPU output enters an expectation.
"""

import numpy as np
import pytest

from oracle.backward import ffn_backward
from oracle.ffn import gate_pre
from oracle.numerics import decode, round_to_storage
from oracle.twell import pack, relu_storage
from workloads.synth import ffn_inputs, gate_bias_for_density, grad_output

from gpu_util import U32, assert_bitwise, dev_inputs, from_dev, packed_to_host, to_dev

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")

DX_TOL = {"f32": 1e-5, "bf16": 1e-2}
DW_TOL = 1e-5
KEYS = ("dx", "dw_gate", "dw_up", "dw_down")


def _bias(T, rho, hot, hot_rho):
    b = np.full(T, gate_bias_for_density(rho))
    if hot:
        b[np.asarray(hot)] = gate_bias_for_density(hot_rho)
    return b


def _slot_units(cnt, idx, tile, cap):
    """[T][nt][cap] unit index of every used slot, -1 for unused slots."""
    T, nt = cnt.shape
    used = np.arange(cap)[None, None, :] < np.minimum(cnt.astype(np.int64), cap)[:, :, None]
    units = np.arange(nt)[None, :, None] * tile + (idx.astype(np.int64) & (tile - 1))
    return np.where(used, units, -1)


def _u64(inp, rows, units):
    """float64 u = x_t . W_u[j] and its fp32 forward error bound, per (row, slot)."""
    X = decode(inp.x, inp.dtype)[rows]
    WU = decode(inp.w_up, inp.dtype)
    j = np.maximum(units, 0)
    r = np.arange(len(rows))[:, None]
    u = (X @ WU.T)[r, j]
    ab = (np.abs(X) @ np.abs(WU).T)[r, j]
    n = X.shape[1]
    return u, 4.0 * n * U32 / (1 - n * U32) * ab


def _check_forward_u(u_dev, host, inp, tile, cap, rows):
    cnt, idx = host["cnt"][rows], host["idx"][rows]
    ovf = (cnt > cap).any(axis=1)
    units = _slot_units(cnt, idx, tile, cap).reshape(len(rows), -1)
    got = u_dev[rows].reshape(len(rows), -1)
    assert np.isnan(got[ovf]).all(), "every slot of an overflow row holds NaN"
    keep = ~ovf
    if not keep.any():
        return
    u, bound = _u64(inp, np.asarray(rows)[keep], units[keep])
    used = units[keep] >= 0
    err = np.abs(got[keep].astype(np.float64) - u)
    assert np.all(err[used] <= bound[used]), f"u off by up to {err[used].max():.3e}"


FWD_CASES = [
    # dtype, T, d, F, tile, cap, density, hot rows
    ("bf16", 300, 512, 1024, 256, 16, 0.01, (7, 100)),
    ("bf16", 97, 2048, 2048, 128, 8, 0.02, (0,)),
    ("f32", 67, 256, 768, 128, 8, 0.03, (5, 40)),
    # d = 1024, F = 40960: more than 8 unit groups, so the up projection adds
    # two halves of d into the saved u
    ("bf16", 40, 1024, 40960, 256, 16, 0.01, (3,)),
]


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,rho,hot", FWD_CASES)
def test_forward_saves_u(dtype, T, d, F, tile, cap, rho, hot):
    import torch
    print(f"saved u forward {dtype} T={T} d={d} F={F} tile={tile} cap={cap}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=T + F, gate_bias=_bias(T, rho, hot, 0.4))
    x, wg, wu, wd, b = dev_inputs(inp)
    p_u = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True, u=True)
    y_u, _ = tw.twell_ffn_forward(x, wg, wu, wd, b, packed=p_u)
    p0 = tw.TwellMatrix.empty(T, F, tile, cap, x.dtype, x.device, T, dense=True)
    y0, _ = tw.twell_ffn_forward(x, wg, wu, wd, b, packed=p0)
    torch.cuda.synchronize()
    assert_bitwise(from_dev(y_u, dtype), from_dev(y0, dtype), "y with and without u")
    h_u, h0 = packed_to_host(p_u, dtype), packed_to_host(p0, dtype)
    for k in ("cnt", "val", "idx", "ovf_rows", "dense"):
        assert_bitwise(h_u[k], h0[k], k)
    _check_forward_u(p_u.u.cpu().numpy(), h_u, inp, tile, cap, np.arange(T))


def _oracle_twell_with_u(inp, dtype, tile, cap):
    """The oracle's TwELL matrix of round(x W_g^T + beta) and the fp32 u of its slots."""
    pre = round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype), dtype)
    P = pack(pre, dtype, tile, cap)
    T = pre.shape[0]
    units = _slot_units(P.cnt, P.idx, tile, cap).reshape(T, -1)
    u, _ = _u64(inp, np.arange(T), units)
    u32 = u.astype(np.float32)
    ovf = (P.cnt > cap).any(axis=1)
    u32[ovf] = np.nan
    u32[units < 0] = 0.0
    return pre, P, u32.reshape(P.cnt.shape + (cap,))


def _upload_twell(P, u32, pre, dtype, tile, cap):
    """A device TwellMatrix of the oracle's pack: packed on the GPU from the same
    stored pre-activations (bitwise equal to the oracle's, tested elsewhere), then
    checked against it here, with the CPU-computed u copied in."""
    import torch
    T, F = pre.shape
    p = tw.TwellMatrix.empty(T, F, tile, cap, torch.bfloat16 if dtype == "bf16" else torch.float32, "cuda:0", T,
                             dense=True)
    tw.twell_pack(to_dev(pre, dtype), tile, cap, out=p)
    host = packed_to_host(p, dtype)
    assert_bitwise(host["cnt"], P.cnt, "cnt")
    assert_bitwise(host["idx"], P.idx, "idx")
    p.u = torch.from_numpy(np.ascontiguousarray(u32)).to("cuda:0")
    return p


BW_CASES = [
    # dtype, T, d, F, tile, cap, width, density, hot rows
    ("bf16", 130, 512, 2048, 256, 16, 32, 0.01, (3, 64, 129)),   # dense rows beside saved-u ELL rows
    ("f32", 67, 256, 768, 128, 8, 24, 0.02, (5, 40)),
    ("bf16", 96, 512, 1024, 128, 2, 64, 0.03, (5, 6)),           # cap 2: TwELL-overflow rows in the ELL (u not saved)
]


@pytest.mark.parametrize("dtype,T,d,F,tile,cap,width,rho,hot", BW_CASES)
def test_hybrid_carries_u_and_backward_uses_it(dtype, T, d, F, tile, cap, width, rho, hot):
    import torch
    print(f"saved u backward {dtype} T={T} d={d} F={F} tile={tile} cap={cap} width={width}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=3 * T + d, gate_bias=_bias(T, rho, hot, 0.4))
    pre, P, u32 = _oracle_twell_with_u(inp, dtype, tile, cap)
    p = _upload_twell(P, u32, pre, dtype, tile, cap)
    hy = tw.twell_to_hybrid(p, width)
    assert hy.u is not None
    torch.cuda.synchronize()
    # the hybrid's u: the slots' u in entry order for rows that fit TwELL, NaN
    # in slot 0 for rows that overflowed it
    cnt = hy.cnt.cpu().numpy()
    hu = hy.u.cpu().numpy()
    tw_ovf = (P.cnt > cap).any(axis=1)
    n_marked = 0
    for t in range(T):
        if cnt[t] > width or cnt[t] == 0:
            continue
        if tw_ovf[t]:
            assert np.isnan(hu[t, 0]), f"row {t}: u of a TwELL-overflow row must be marked"
            n_marked += 1
            continue
        k, s = np.nonzero(np.arange(cap)[None, :] < np.minimum(P.cnt[t].astype(np.int64), cap)[:, None])
        assert_bitwise(hu[t, :cnt[t]], u32[t, k, s], f"row {t} u")
    if cap == 2:
        assert n_marked > 0, "the case must hold ELL rows whose u was not saved"
    # the backward with u from the hybrid against the float64 oracle
    h = relu_storage(pre, dtype)
    dy = grad_output(T, d, dtype, seed=T)
    lam = float(np.float32(2e-5))
    ref = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, lam, dtype)
    x, wg, wu, wd, _ = dev_inputs(inp)
    out = tw.twell_ffn_backward(hy, x, wg, wu, wd, to_dev(dy, dtype), lam)
    torch.cuda.synchronize()
    got = {"dx": decode(from_dev(out[0], dtype), dtype)}
    for k, t_ in zip(KEYS[1:], out[1:]):
        got[k] = t_.cpu().numpy().astype(np.float64)
    for k in KEYS:
        tol = DX_TOL[dtype] if k == "dx" else DW_TOL
        g, r = got[k], ref[k]
        err = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
        assert err <= tol, f"{k}: relative L2 error {err:.3e} > {tol:g}"
        zero = np.linalg.norm(r, axis=1) == 0
        assert np.all(g[zero] == 0), f"{k}: rows with no active entry must be exactly zero"


@pytest.mark.slow
@pytest.mark.parametrize("name", ["layer_1p5b_bf16", "skewed_bf16", "large_bf16"])
def test_forward_saves_u_full_size(name):
    """Full shapes (the larger layer adds two halves of d) on sampled rows,
    including the skewed layer's overflow rows (all NaN)."""
    import torch
    from workloads.configs import workload
    w = workload(name)
    print(f"saved u forward full size {name}", flush=True)
    inp = w.inputs()
    x, wg, wu, wd, b = dev_inputs(inp)
    p = tw.TwellMatrix.empty(w.T, w.F, w.tile, w.cap, x.dtype, x.device, w.T, dense=False, u=True)
    tw.twell_ffn_forward(x, wg, wu, wd, b, packed=p)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(w.T, 24, replace=False), np.arange(0, w.T, 2048)[:4]]))
    host = {"cnt": p.cnt.cpu().numpy().view(np.uint16), "idx": p.idx.cpu().numpy()}
    _check_forward_u(p.u.cpu().numpy(), host, inp, w.tile, w.cap, rows)


WALKED_CASES = [
    # dtype, T, d, F, width, density, hot rows (hidden sizes that are not a
    # multiple of 128: the dense rows are walked entry by entry beside the
    # saved-u ELL rows)
    ("bf16", 61, 512, 320, 8, 0.01, (2, 30)),
    ("f32", 50, 256, 448, 4, 0.005, (1, 7)),
]


@pytest.mark.parametrize("dtype,T,d,F,width,rho,hot", WALKED_CASES)
def test_caller_built_hybrid_with_u_and_walked_dense_rows(dtype, T, d, F, width, rho, hot):
    """A hybrid built by the oracle and uploaded, with the float64 u of every
    ELL entry rounded to fp32 and every third ELL row marked not saved (NaN
    in its first slot): the backward takes u from the hybrid where it is
    saved, recomputes it elsewhere (marked rows, dense rows) and must match the
    float64 oracle with the tolerances of the other backward tests."""
    import torch
    from oracle.hybrid import hybrid
    from test_gpu_backward import hybrid_to_dev
    print(f"caller-built hybrid with u {dtype} T={T} d={d} F={F} width={width}", flush=True)
    inp = ffn_inputs(T, d, F, dtype, seed=5 * T + F, gate_bias=_bias(T, rho, hot, 0.4))
    pre = round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype), dtype)
    h = relu_storage(pre, dtype)
    hy = hybrid(h, dtype, width)
    assert hy.n_dense > 0, "the case must hold dense rows"
    ell = np.nonzero(hy.cnt <= width)[0]
    used = np.arange(width)[None, :] < np.minimum(hy.cnt, width)[:, None]
    units = np.where(used, hy.col, -1)
    u64, _ = _u64(inp, np.arange(T), units)
    u32 = np.where(used, u64, 0.0).astype(np.float32)
    marked = ell[(hy.cnt[ell] > 0)][::3]
    u32[marked, 0] = np.nan
    assert marked.size > 0
    hd = hybrid_to_dev(hy, F, dtype)
    hd.u = torch.from_numpy(np.ascontiguousarray(u32)).to("cuda:0")
    dy = grad_output(T, d, dtype, seed=T)
    lam = float(np.float32(2e-5))
    ref = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, lam, dtype)
    x, wg, wu, wd, _ = dev_inputs(inp)
    out = tw.twell_ffn_backward(hd, x, wg, wu, wd, to_dev(dy, dtype), lam)
    torch.cuda.synchronize()
    got = {"dx": decode(from_dev(out[0], dtype), dtype)}
    for k, t_ in zip(KEYS[1:], out[1:]):
        got[k] = t_.cpu().numpy().astype(np.float64)
    for k in KEYS:
        tol = DX_TOL[dtype] if k == "dx" else DW_TOL
        g, r = got[k], ref[k]
        err = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
        assert err <= tol, f"{k}: relative L2 error {err:.3e} > {tol:g}"
        zero = np.linalg.norm(r, axis=1) == 0
        assert np.all(g[zero] == 0), f"{k}: rows with no active entry must be exactly zero"
