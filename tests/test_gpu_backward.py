"""GPU parity: FFN backward from hybrid activations (HIP) against the float64 oracle.

The activations are the oracle's: h = ReLU(round(x W_g^T + beta)) in the
storage dtype, converted to the hybrid format by the oracle and uploaded; the
upstream gradient dy is seeded.  No GPU output enters an expectation.

Tolerances (relative L2 over the whole tensor, written per output):
* dw_gate, dw_up, dw_down are fp32 sums of fp32 products of stored values
  (u and da are fp32 dot products over d terms): 1e-5, as for the fp32
  forward.
* dx is rounded once to the activation dtype: 1e-5 for fp32, 1e-2 for bf16
  (unit roundoff 2^-8, as for the forward's y).
Rows of dx and rows of dW whose reference is exactly zero (no active entry)
must be exactly zero.  Per row, the error must stay within 8x the tolerance
of the larger of the row's norm and the RMS row norm: a row whose value
nearly cancels (da = dy_t . W_d[j] close to zero, say) carries fp32 rounding
of the size of a typical row, not of its own.
"""

import numpy as np
import pytest

from oracle.backward import ffn_backward
from oracle.ffn import gate_pre, rel_l2
from oracle.hybrid import hybrid
from oracle.numerics import decode, round_to_storage
from oracle.twell import relu_storage
from workloads.synth import ffn_inputs, gate_bias_for_density, grad_output

from gpu_util import dev_inputs, from_dev, to_dev, torch_dtype

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


def _case(T, d, F, dtype, seed, rho, hot=(), hot_rho=0.4):
    inp = ffn_inputs(T, d, F, dtype, seed=seed, gate_bias=_bias(T, rho, hot, hot_rho))
    h = relu_storage(round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype), dtype), dtype)
    dy = grad_output(T, d, dtype, seed=seed)
    return inp, h, dy


def hybrid_to_dev(hy, F, dtype, dense_cap=None, device="cuda:0"):
    import torch
    T = hy.cnt.shape[0]
    n = hy.n_dense
    dense_cap = n if dense_cap is None else dense_cap
    out = tw.TwellHybrid.empty(T, F, hy.width, torch_dtype(dtype), device, dense_cap)
    if T:
        out.cnt.copy_(torch.from_numpy(hy.cnt))
        out.val.copy_(to_dev(hy.val, dtype, device))
        out.col.copy_(torch.from_numpy(hy.col))
    out.n_dense.fill_(n)
    k = min(n, dense_cap)
    if k:
        out.dense_rows[:k].copy_(torch.from_numpy(hy.dense_rows[:k]))
        out.dense[:k].copy_(to_dev(hy.dense[:k], dtype, device))
    return out


def run_gpu(inp, hy, F, dy, lam, dtype, dense_cap=None):
    import torch
    hd = hybrid_to_dev(hy, F, dtype, dense_cap)
    x, wg, wu, wd, _ = dev_inputs(inp)
    dyd = to_dev(dy, dtype)
    out = tw.twell_ffn_backward(hd, x, wg, wu, wd, dyd, lam)
    torch.cuda.synchronize()
    return {"dx": decode(from_dev(out[0], dtype), dtype), "dw_gate": out[1].cpu().numpy().astype(np.float64),
            "dw_up": out[2].cpu().numpy().astype(np.float64), "dw_down": out[3].cpu().numpy().astype(np.float64)}


def check(got, ref, dtype):
    for k in KEYS:
        tol = DX_TOL[dtype] if k == "dx" else DW_TOL
        g, r = got[k], ref[k]
        assert g.shape == r.shape, k
        err = rel_l2(g, r)
        assert err <= tol, f"{k}: relative L2 error {err:.3e} > {tol:g}"
        zero = np.linalg.norm(r, axis=1) == 0
        assert np.all(g[zero] == 0), f"{k}: rows with no active entry must be exactly zero"
        if (~zero).any():
            norms = np.linalg.norm(r, axis=1)
            scale = np.maximum(norms, np.sqrt(np.mean(norms[~zero] ** 2)))
            worst = float(np.max((np.linalg.norm(g - r, axis=1) / scale)[~zero]))
            assert worst <= 8 * tol, f"{k}: worst row error {worst:.3e} (relative to max(row, RMS row) norm)"


CASES = [
    # dtype, T, d, F, width, density, hot rows, lam
    ("f32", 64, 256, 1024, 16, 0.01, (), 0.0),                 # the tiny fp32 layer's shape
    ("f32", 67, 512, 768, 8, 0.03, (5, 40), 2e-5),             # ragged T, dense rows
    ("f32", 40, 2048, 512, 32, 0.05, (), 0.25),                # d = 2048 fp32: one entry in flight
    ("bf16", 130, 512, 2048, 32, 0.02, (3, 64, 129), 2e-5),    # several XCD groups, dense rows
    ("bf16", 97, 1024, 1024, 8, 0.05, (), 0.5),
    ("bf16", 33, 2048, 4096, 64, 0.01, (0, 32), 2e-5),          # the 1.5B-class d
    ("bf16", 50, 4096, 1024, 16, 0.02, (7,), 0.0),             # d = 4096: one entry in flight
    ("bf16", 45, 512, 1536, 1, 0.01, (), 0.1),                 # width 1: most rows dense
    ("bf16", 70, 1536, 640, 300, 0.2, (), 0.0),                # wide ELL: no dense row; F not a power of 2
    # dense rows on the matrix cores: several row tiles, R not a multiple of 64
    ("bf16", 300, 512, 1024, 2, 0.02, (), 2e-5),               # width 2: nearly every row dense
    ("f32", 150, 256, 512, 2, 0.03, (), 0.1),
    ("bf16", 530, 1024, 2048, 20, 0.01, (0, 17, 256, 529), 2e-5),  # about half the rows dense
    # F not a multiple of 128: the dense rows' entries are walked like the others
    ("bf16", 61, 512, 320, 4, 0.03, (2, 30), 2e-5),
    ("f32", 50, 256, 448, 4, 0.05, (1,), 2e-5),
]


@pytest.mark.parametrize("dtype,T,d,F,width,rho,hot,lam", CASES)
def test_backward_parity(dtype, T, d, F, width, rho, hot, lam):
    print(f"backward {dtype} T={T} d={d} F={F} width={width} rho={rho} hot={hot} lam={lam}", flush=True)
    inp, h, dy = _case(T, d, F, dtype, seed=T + d + F, rho=rho, hot=hot)
    lam = float(np.float32(lam))
    hy = hybrid(h, dtype, width)
    ref = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h, dy, lam, dtype)
    got = run_gpu(inp, hy, F, dy, lam, dtype)
    check(got, ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_deterministic(dtype):
    print(f"backward determinism {dtype}", flush=True)
    inp, h, dy = _case(90, 512, 1024, dtype, seed=3, rho=0.05, hot=(1, 2))
    hy = hybrid(h, dtype, 16)
    a = run_gpu(inp, hy, 1024, dy, 2e-5, dtype)
    b = run_gpu(inp, hy, 1024, dy, 2e-5, dtype)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_all_inactive_and_empty(dtype):
    print(f"backward all-inactive / T=0 {dtype}", flush=True)
    inp, h, dy = _case(20, 512, 512, dtype, seed=4, rho=0.05)
    h0 = np.zeros_like(h)
    got = run_gpu(inp, hybrid(h0, dtype, 8), 512, dy, 0.3, dtype)
    for k in KEYS:
        assert not got[k].any(), k
    # T = 0: every weight gradient is zero
    inp0, h0, dy0 = _case(0, 512, 512, dtype, seed=5, rho=0.05)
    got = run_gpu(inp0, hybrid(h0, dtype, 8), 512, dy0, 0.3, dtype)
    assert got["dx"].shape == (0, 512)
    for k in KEYS[1:]:
        assert got[k].shape == (512, 512) and not got[k].any(), k


def test_backward_unstored_dense_rows_contribute_nothing():
    # dense_cap below n_dense: the rows not stored are taken as empty
    dtype = "bf16"
    print("backward dense_cap < n_dense", flush=True)
    inp, h, dy = _case(60, 512, 1024, dtype, seed=6, rho=0.01, hot=(2, 9, 30, 31), hot_rho=0.5)
    hy = hybrid(h, dtype, 16)
    assert hy.n_dense >= 4
    cap = hy.n_dense - 2
    h_kept = h.copy()
    h_kept[hy.dense_rows[cap:]] = 0
    lam = float(np.float32(2e-5))
    ref = ffn_backward(inp.x, inp.w_gate, inp.w_up, inp.w_down, h_kept, dy, lam, dtype)
    got = run_gpu(inp, hy, 1024, dy, lam, dtype, dense_cap=cap)
    check(got, ref, dtype)


@pytest.mark.slow
@pytest.mark.parametrize("name,width", [("layer_1p5b_bf16", 256), ("skewed_bf16", 256), ("layer_1p5b_bf16", 64)])
def test_backward_full_size(name, width):
    """The 1.5B-class layer (and its skewed variant) at full size, hybrid width 256
    as timed by the bench: dx on sampled rows, the weight gradients on sampled
    hidden units (each depends only on its own row / unit of h).  Width 64
    makes nearly every row dense (~82 active units per row): the dense-row
    matmuls then fill the grid without a K split."""
    import torch
    from workloads.configs import workload
    w = workload(name)
    T, d, F, dtype = w.T, w.d, w.F, w.dtype
    print(f"backward full size {name} width {width}", flush=True)
    inp = w.inputs()
    h = relu_storage(round_to_storage(gate_pre(inp.x, inp.w_gate, inp.gate_bias, dtype), dtype), dtype)
    dy = grad_output(T, d, dtype, seed=0)
    hy = hybrid(h, dtype, width)
    lam = float(np.float32(2e-5))
    got_dev = hybrid_to_dev(hy, F, dtype, dense_cap=T)
    x, wg, wu, wd, _ = dev_inputs(inp)
    out = tw.twell_ffn_backward(got_dev, x, wg, wu, wd, to_dev(dy, dtype), lam)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(T, 48, replace=False), hy.dense_rows[:16]]))
    units = np.sort(rng.choice(F, 48, replace=False))
    ref_r = ffn_backward(inp.x[rows], inp.w_gate, inp.w_up, inp.w_down, h[rows], dy[rows], lam, dtype)
    ref_u = ffn_backward(inp.x, inp.w_gate[units], inp.w_up[units], inp.w_down[units], h[:, units], dy, lam,
                         dtype)
    got = {"dx": decode(from_dev(out[0], dtype), dtype)[rows]}
    for k, t in zip(KEYS[1:], out[1:]):
        got[k] = t[torch.from_numpy(units).to(t.device)].cpu().numpy().astype(np.float64)
    ref = {"dx": ref_r["dx"], **{k: ref_u[k] for k in KEYS[1:]}}
    check(got, ref, dtype)
