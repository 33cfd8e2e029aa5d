"""GPU parity: TwELL -> hybrid conversion (HIP) against the oracle, bit for bit.

The TwELL input is packed on the GPU from seeded pre-activations; the expected
hybrid is the oracle's hybrid of ReLU(pre), computed from the same
pre-activations on the CPU (no GPU output enters the expectation)."""

import numpy as np
import pytest

from oracle.hybrid import hybrid
from oracle.twell import relu_storage
from workloads.synth import pre_activations

from gpu_util import assert_bitwise, from_dev, to_dev

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


def _hybrid_to_host(h, dtype):
    n = int(h.n_dense.cpu().item())
    k = min(n, h.dense_cap)
    out = {"cnt": h.cnt.cpu().numpy(), "val": from_dev(h.val, dtype), "col": h.col.cpu().numpy(),
           "n_dense": n, "dense_rows": h.dense_rows.cpu().numpy()[:k]}
    if h.dense is not None:
        out["dense"] = from_dev(h.dense, dtype)[:k]
    return out


def _check(got, ref, dense_cap=None):
    assert_bitwise(got["cnt"], ref.cnt, "cnt")
    assert_bitwise(got["val"], ref.val, "val")
    assert_bitwise(got["col"], ref.col, "col")
    assert got["n_dense"] == ref.n_dense
    k = ref.n_dense if dense_cap is None else min(ref.n_dense, dense_cap)
    assert_bitwise(got["dense_rows"], ref.dense_rows[:k], "dense_rows")
    if "dense" in got:
        assert_bitwise(got["dense"], ref.dense[:k], "dense")


CASES = [
    # T, F, tile, cap, width, density, hot rows, specials
    (1, 256, 256, 16, 8, 0.01, (), False),
    (67, 1024, 256, 16, 16, 0.01, (), False),            # ragged rows
    (130, 1024, 128, 8, 24, 0.05, (3, 64, 129), True),   # TwELL-overflow rows, some ELL, some dense
    (96, 512, 128, 2, 64, 0.04, (5, 6), True),           # cap 2: many TwELL-overflow rows fit the ELL
    (80, 2048, 256, 16, 4, 0.002, (), False),            # narrow ELL: dense rows without TwELL overflow
    (50, 768, 256, 16, 8, 0.0, (), False),               # nothing active
    (40, 512, 256, 16, 600, 1.0 - 1e-9, (), False),      # width > F: every row is an ELL row
    (33, 512, 128, 64, 1, 0.3, (), True),                # width 1: nearly every row is dense
    (29, 8192, 128, 16, 256, 0.01, (4, 17), True),       # 64 tiles: one lane per ELL position, a full search
    (23, 8960, 128, 16, 256, 0.01, (), False),           # 70 tiles: one lane per tile, two passes
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,F,tile,cap,width,rho,hot,specials", CASES)
def test_to_hybrid_bitwise(dtype, T, F, tile, cap, width, rho, hot, specials):
    print(f"hybrid {dtype} T={T} F={F} tile={tile} cap={cap} width={width} rho={rho}", flush=True)
    pre = pre_activations(T, F, dtype, seed=7 * T + F, density=max(rho, 1e-12), hot_rows=hot,
                          hot_density=0.4, specials=specials)
    if rho == 0.0:
        pre = np.where(np.zeros_like(pre, dtype=bool), pre, (np.float32(-1.0) if dtype == "f32"
                                                              else np.uint16(0xBF80)))
    p = tw.twell_pack(to_dev(pre, dtype), tile, cap, dense=True)
    h = tw.twell_to_hybrid(p, width)
    _check(_hybrid_to_host(h, dtype), hybrid(relu_storage(pre, dtype), dtype, width))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dense_cap_truncates_list_but_counts_all(dtype):
    pre = pre_activations(64, 512, dtype, seed=3, density=0.05, hot_rows=(1, 9, 17, 40), hot_density=0.5)
    p = tw.twell_pack(to_dev(pre, dtype), 256, 16, dense=True)
    h = tw.twell_to_hybrid(p, 12, dense_cap=2)
    ref = hybrid(relu_storage(pre, dtype), dtype, 12)
    assert ref.n_dense > 2
    _check(_hybrid_to_host(h, dtype), ref, dense_cap=2)


def test_without_dense_rows_and_zero_rows():
    pre = pre_activations(48, 512, "bf16", seed=11, density=0.05, hot_rows=(2, 30), hot_density=0.6)
    p = tw.twell_pack(to_dev(pre, "bf16"), 256, 16, dense=True)
    h = tw.twell_to_hybrid(p, 16, dense=False)
    got = _hybrid_to_host(h, "bf16")
    ref = hybrid(relu_storage(pre, "bf16"), "bf16", 16)
    assert "dense" not in got
    _check(got, ref)
    # zero rows: only n_dense is written
    p0 = tw.twell_pack(to_dev(pre[:0], "bf16"), 256, 16, dense=True)
    h0 = tw.twell_to_hybrid(p0, 16)
    assert int(h0.n_dense.cpu().item()) == 0


@pytest.mark.slow
def test_to_hybrid_full_size():
    # 1.5B-class layer shape, 1% density plus the first 64 tokens of every 2048 at 20%
    T, F = 8192, 8192
    hot = [t for t in range(T) if t % 2048 < 64]
    pre = pre_activations(T, F, "bf16", seed=5, density=0.01, hot_rows=hot, hot_density=0.2)
    p = tw.twell_pack(to_dev(pre, "bf16"), 256, 16, dense=True)
    h = tw.twell_to_hybrid(p, 256)
    _check(_hybrid_to_host(h, "bf16"), hybrid(relu_storage(pre, "bf16"), "bf16", 256))
