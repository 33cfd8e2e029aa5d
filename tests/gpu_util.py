"""Helpers for the GPU parity tests: host <-> device conversion of storage
tensors, and the checks that compare the HIP results with the oracle."""

from __future__ import annotations

import numpy as np

from oracle.ffn import ffn, gate_pre, rel_l2
from oracle.numerics import decode, round_to_storage
from oracle.twell import active, pack

U32 = 2.0 ** -24  # unit roundoff of fp32
TOL = {"f32": 1e-5, "bf16": 1e-2}  # relative L2 error of y against the float64 oracle


def torch_dtype(dtype: str):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def to_dev(a: np.ndarray, dtype: str, device="cuda:0"):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def from_dev(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "f32":
        return t.detach().float().cpu().numpy()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_inputs(inp, device="cuda:0"):
    import torch
    x = to_dev(inp.x, inp.dtype, device)
    wg = to_dev(inp.w_gate, inp.dtype, device)
    wu = to_dev(inp.w_up, inp.dtype, device)
    wd = to_dev(inp.w_down, inp.dtype, device)
    b = None if inp.gate_bias is None else torch.from_numpy(inp.gate_bias).to(device)
    return x, wg, wu, wd, b


def packed_to_host(p, dtype: str):
    """Host copies of a device TwellMatrix: dict of numpy arrays."""
    n_ovf = int(p.n_ovf.cpu().item())
    out = {
        "cnt": p.cnt.cpu().numpy().view(np.uint16),
        "val": from_dev(p.val, dtype),
        "idx": p.idx.cpu().numpy(),
        "n_ovf": n_ovf,
        "ovf_rows": p.ovf_rows.cpu().numpy()[:min(n_ovf, p.ovf_cap)],
    }
    if p.dense is not None:
        out["dense"] = from_dev(p.dense, dtype)[:min(n_ovf, p.ovf_cap)]
    return out


def assert_bitwise(a: np.ndarray, b: np.ndarray, what: str):
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    a8 = np.ascontiguousarray(a).view(np.uint8)
    b8 = np.ascontiguousarray(b).view(np.uint8)
    if not np.array_equal(a8, b8):
        bad = np.nonzero(a8 != b8)[0]
        raise AssertionError(f"{what}: {bad.size} differing bytes, first at byte {bad[0]}")


def assert_packed_equal(host: dict, ref, check_dense: bool = True):
    """Bit-exact comparison of a device pack (host copy) with an oracle Packed."""
    assert_bitwise(host["cnt"], ref.cnt, "cnt")
    assert_bitwise(host["val"], ref.val, "val")
    assert_bitwise(host["idx"], ref.idx, "idx")
    assert host["n_ovf"] == ref.n_ovf, f"n_ovf {host['n_ovf']} != {ref.n_ovf}"
    k = host["ovf_rows"].shape[0]
    assert_bitwise(host["ovf_rows"].astype(np.int32), ref.ovf_rows[:k].astype(np.int32), "ovf_rows")
    if check_dense and "dense" in host:
        assert_bitwise(host["dense"], ref.dense[:k], "dense")


def gate_bound(inp, slack: float = 4.0):
    """Float64 gate pre-activations and a forward error bound for an fp32 accumulation.

    |fl(sum) - sum| <= gamma_n * sum |terms| with gamma_n = n u / (1 - n u), n = d + 1
    (d products and the bias), u = 2^-24; ``slack`` covers the unspecified
    summation order inside the matrix-core instructions.
    """
    X = decode(inp.x, inp.dtype)
    G = decode(inp.w_gate, inp.dtype)
    beta = 0.0 if inp.gate_bias is None else inp.gate_bias.astype(np.float64)[:, None]
    pre = X @ G.T + beta
    absum = np.abs(X) @ np.abs(G).T + np.abs(beta)
    n = X.shape[1] + 1
    gamma = n * U32 / (1 - n * U32)
    return pre, slack * gamma * absum


def check_fused_pack(host: dict, pre64: np.ndarray, bound: np.ndarray, dtype: str, tile: int, cap: int,
                     rows=None):
    """Check a TwELL matrix produced from fp32-accumulated gate values against the
    float64 gate: every entry whose sign is certain must agree, the rest must be
    valid (structure, ordering, values within the bound, overflow rule)."""
    T, F = pre64.shape
    nt = F // tile
    rows = np.arange(T) if rows is None else np.asarray(rows)
    cnt = host["cnt"].astype(np.int64)
    rel = 2.0 ** -8 if dtype == "bf16" else 0.0  # RNE to bf16: unit roundoff of an 8-bit significand
    for i, t in enumerate(rows):
        for k in range(nt):
            c = cnt[t, k]
            n = min(c, cap)
            seg = pre64[i, k * tile:(k + 1) * tile]
            b = bound[i, k * tile:(k + 1) * tile]
            certain = np.nonzero(seg > b)[0]
            possible = np.nonzero(seg > -b)[0]
            assert certain.size <= c <= possible.size, (t, k, c, certain.size, possible.size)
            ids = host["idx"][t, k, :n].astype(np.int64)
            assert np.all(np.diff(ids) > 0) and np.all(ids < tile), (t, k, ids)
            assert np.isin(ids, possible).all(), (t, k)
            v = decode(host["val"][t, k, :n], dtype)
            assert np.all(v > 0), (t, k, v)
            err = np.abs(v - seg[ids])
            assert np.all(err <= b[ids] + rel * (np.abs(seg[ids]) + b[ids])), (t, k, err.max())
            # padding
            assert not host["idx"][t, k, n:].any() and not np.ascontiguousarray(host["val"][t, k, n:]).view(np.uint8).any()
            # no certainly-active column below the last stored one is missing
            last = ids[-1] if n else -1
            if c <= cap:
                assert np.isin(certain, ids).all(), (t, k)
            else:
                assert np.isin(certain[certain <= last], ids).all(), (t, k)
    ovf = np.nonzero((cnt > cap).any(axis=1))[0]
    assert host["n_ovf"] == ovf.size
    assert np.array_equal(host["ovf_rows"], ovf[:host["ovf_rows"].size])


def exact_gate_inputs(T: int, d: int, F: int, dtype: str, seed: int, density: float):
    """Gate inputs whose fp32 accumulation is exact in any order.

    x is an integer in [-4, 4], every weight a multiple of 1/8 in [-1, 1] with
    at most 4 significant bits; every partial sum is then a multiple of 1/8
    below 2^22 in magnitude, exactly representable in fp32.  The bias is a
    multiple of 1/8 chosen for the requested density.
    """
    from statistics import NormalDist
    from workloads.synth import FfnInputs, to_storage
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, size=(T, d)).astype(np.float64)
    wg = rng.integers(-8, 9, size=(F, d)).astype(np.float64) / 8.0
    wu = rng.integers(-8, 9, size=(F, d)).astype(np.float64) / 8.0
    wd = rng.integers(-8, 9, size=(F, d)).astype(np.float64) / 8.0
    sigma = np.sqrt(d * np.mean(x ** 2) * np.mean(wg ** 2))
    b = np.round(NormalDist().inv_cdf(density) * sigma * 8) / 8
    bias = np.full(T, b, dtype=np.float32)
    return FfnInputs(dtype, *(to_storage(a, dtype) for a in (x, wg, wu, wd)), bias, seed)


def check_y(y_dev_np: np.ndarray, inp, dtype: str, rows=None, per_row=True):
    """y against the float64 oracle on all rows (or the given sample of rows)."""
    if rows is None:
        y64 = ffn(inp.x, inp.w_gate, inp.w_up, inp.w_down, inp.gate_bias, dtype)
        yg = decode(y_dev_np, dtype)
    else:
        rows = np.asarray(rows)
        b = None if inp.gate_bias is None else inp.gate_bias[rows]
        y64 = ffn(inp.x[rows], inp.w_gate, inp.w_up, inp.w_down, b, dtype)
        yg = decode(y_dev_np[rows], dtype)
    tol = TOL[dtype]
    err = rel_l2(yg, y64)
    assert err <= tol, f"relative L2 error {err:.3e} > {tol:g}"
    if per_row:
        # Each row's error relative to the larger of its own norm and the RMS
        # row norm: a row that nearly cancels (few entries whose u or v is
        # near zero) carries fp32 rounding the size of a typical row's, not
        # of its own.
        norms = np.linalg.norm(y64, axis=1)
        zero_rows = norms == 0
        assert np.all(yg[zero_rows] == 0), "rows with no active unit must be exactly zero"
        if (~zero_rows).any():
            scale = np.maximum(norms, np.sqrt(np.mean(norms[~zero_rows] ** 2)))
            worst = float(np.max((np.linalg.norm(yg - y64, axis=1) / scale)[~zero_rows]))
            assert worst <= 4 * tol, f"worst row error {worst:.3e} (relative to max(row, RMS row) norm)"
    return err


__all__ = ["TOL", "torch_dtype", "to_dev", "from_dev", "dev_inputs", "packed_to_host", "assert_bitwise",
           "assert_packed_equal", "gate_bound", "check_fused_pack", "exact_gate_inputs", "check_y",
           "ffn", "gate_pre", "pack", "round_to_storage", "active"]
