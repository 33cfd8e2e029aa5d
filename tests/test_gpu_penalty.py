"""GPU parity: the L1 activation penalty ||h||_1 and its gradient from TwELL (HIP)
against the oracle.  The norm is a float64 sum in a fixed order: it must equal
the exactly rounded sum up to float64 accumulation error (relative 1e-10 for
these sizes), and exactly when every partial sum is representable.  The
gradient is compared bit for bit."""

import numpy as np
import pytest

from oracle.penalty import l1_grad_twell, l1_norm
from oracle.twell import pack, relu_storage
from workloads.synth import pre_activations, to_storage

from gpu_util import assert_bitwise, from_dev, to_dev

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")

CASES = [
    # T, F, tile, cap, density, hot rows, specials
    (1, 256, 256, 16, 0.01, (), False),
    (67, 1024, 256, 16, 0.01, (), False),
    (130, 1024, 128, 8, 0.05, (3, 64, 129), True),     # overflow rows (dense backup), +inf values
    (96, 512, 128, 2, 0.04, (5, 6), False),
    (50, 768, 256, 16, 0.0, (), False),                # nothing active: 0
    (2048, 2048, 256, 16, 0.01, tuple(range(0, 2048, 64)), False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,F,tile,cap,rho,hot,specials", CASES)
def test_l1_norm_and_grad(dtype, T, F, tile, cap, rho, hot, specials):
    print(f"l1 {dtype} T={T} F={F} tile={tile} cap={cap} rho={rho}", flush=True)
    pre = pre_activations(T, F, dtype, seed=3 * T + F, density=max(rho, 1e-12), hot_rows=hot,
                          hot_density=0.4, specials=specials)
    if rho == 0.0:
        pre = to_storage(np.full((T, F), -1.0), dtype)
    p = tw.twell_pack(to_dev(pre, dtype), tile, cap, dense=True)
    got = float(tw.twell_l1_norm(p).cpu().item())
    want = l1_norm(relu_storage(pre, dtype), dtype)
    if np.isinf(want):
        assert got == want
    else:
        assert abs(got - want) <= 1e-10 * want, (got, want)
    lam = 2e-5
    gv, gd = tw.twell_l1_grad(p, lam)
    ref = pack(pre, dtype, tile, cap)
    want_v, want_d = l1_grad_twell(ref, lam)
    assert_bitwise(from_dev(gv, dtype), want_v, "grad_val")
    n = ref.n_ovf
    assert_bitwise(from_dev(gd, dtype)[:n], want_d, "grad_dense")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_l1_norm_exact_on_dyadic_values(dtype):
    # values 2^-k (k <= 6): every partial sum of a few thousand of them is exact
    rng = np.random.default_rng(1)
    v = np.where(rng.random((300, 512)) < 0.03, 2.0 ** -rng.integers(0, 7, (300, 512)), -1.0)
    pre = to_storage(v, dtype)
    p = tw.twell_pack(to_dev(pre, dtype), 256, 4, dense=True)
    assert float(tw.twell_l1_norm(p).cpu().item()) == l1_norm(relu_storage(pre, dtype), dtype)
