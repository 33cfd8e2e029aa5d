"""GPU parity: twell_pack (HIP) against the oracle packer, bit for bit."""

import numpy as np
import pytest

from oracle.twell import pack
from workloads.synth import pre_activations

from gpu_util import assert_packed_equal, from_dev, packed_to_host, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


def _run(pre_np, dtype, tile, cap, ovf_cap=None, dense=True):
    pre = to_dev(pre_np, dtype)
    p = tw.twell_pack(pre, tile, cap, ovf_cap=ovf_cap, dense=dense)
    return packed_to_host(p, dtype)


CASES = [
    # T, F, tile, cap, density, hot rows, specials
    (1, 256, 256, 16, 0.01, (), False),
    (67, 1024, 256, 16, 0.01, (), False),          # ragged rows, 4 tiles
    (130, 1024, 128, 8, 0.05, (3, 64, 129), True),  # overflow rows, special values
    (256, 2048, 256, 1, 0.002, (), False),          # cap 1
    (96, 512, 128, 64, 0.3, (), True),              # cap 64, dense rows
    (50, 768, 256, 16, 0.0, (), False),             # no active unit at all
    (40, 512, 256, 16, 1.0 - 1e-9, (), False),      # (almost) everything active: every row overflows
    # rows over several chunks of 8 loads, the last one partial (bf16: 16 + 5
    # tiles; fp32: 8 + 8 + 5), and long per-lane walks with tiles past the cap
    # in every chunk (bf16: 32 + 13 tiles of 128; fp32: 16 + 16 + 13)
    (37, 5376, 256, 16, 0.04, (5, 20), True),
    (29, 5760, 128, 32, 0.2, (), False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,F,tile,cap,rho,hot,specials", CASES)
def test_pack_bitwise(dtype, T, F, tile, cap, rho, hot, specials):
    print(f"pack {dtype} T={T} F={F} tile={tile} cap={cap} rho={rho}", flush=True)
    pre = pre_activations(T, F, dtype, seed=T + F, density=max(rho, 1e-12), hot_rows=hot,
                          hot_density=0.4, specials=specials)
    if rho == 0.0:
        pre = -np.abs(pre) if dtype == "f32" else (pre | np.uint16(0x8000))
    host = _run(pre, dtype, tile, cap)
    assert_packed_equal(host, pack(pre, dtype, tile, cap))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_ovf_cap_truncates_list_but_counts_all(dtype):
    T, F = 64, 512
    pre = pre_activations(T, F, dtype, seed=5, density=0.01, hot_rows=range(0, 64, 3), hot_density=0.5)
    ref = pack(pre, dtype, 256, 4)
    assert ref.n_ovf > 5
    host = _run(pre, dtype, 256, 4, ovf_cap=5)
    assert host["n_ovf"] == ref.n_ovf
    assert np.array_equal(host["ovf_rows"], ref.ovf_rows[:5])
    assert np.array_equal(host["dense"].view(np.uint8), np.ascontiguousarray(ref.dense[:5]).view(np.uint8))


def test_pack_without_dense_rows():
    pre = pre_activations(32, 256, "bf16", seed=9, density=0.2)
    host = _run(pre, "bf16", 128, 4, dense=False)
    assert_packed_equal(host, pack(pre, "bf16", 128, 4), check_dense=False)


def test_pack_zero_rows():
    import torch
    pre = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda:0")
    p = tw.twell_pack(pre, 256, 16)
    assert int(p.n_ovf.item()) == 0


@pytest.mark.slow
@pytest.mark.parametrize("dtype,T,F,tile,cap,hot", [
    ("bf16", 8192, 8192, 256, 16, ()),                            # 1.5B-class layer shape
    ("bf16", 8192, 8192, 256, 16, tuple(t for t in range(8192) if t % 2048 < 64)),  # skewed
])
def test_pack_full_size(dtype, T, F, tile, cap, hot):
    print(f"pack full {dtype} T={T} F={F} hot={len(hot)}", flush=True)
    pre = pre_activations(T, F, dtype, seed=1, density=0.01, hot_rows=hot, hot_density=0.2)
    host = _run(pre, dtype, tile, cap)
    assert_packed_equal(host, pack(pre, dtype, tile, cap))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ovf_cap_delta", [0, -1])
def test_pack_list_spans_several_rounds(dtype, ovf_cap_delta):
    """More rows than one round of the overflow-list kernels (8192 rows): with
    room for every row the rows are listed over the flags in ovf_rows itself
    (several rounds of that in-place compaction); with one slot less the
    count scan builds the truncated list."""
    T, F = 2 * 8192 + 515, 256
    hot = tuple(range(3, T, 7))
    print(f"pack rounds {dtype} T={T} ovf_cap=T{ovf_cap_delta:+d}", flush=True)
    pre = pre_activations(T, F, dtype, seed=11, density=0.01, hot_rows=hot, hot_density=0.2)
    ref = pack(pre, dtype, 128, 2)
    assert ref.n_ovf > 2000
    ovf_cap = T + ovf_cap_delta
    host = _run(pre, dtype, 128, 2, ovf_cap=ovf_cap)
    assert host["ovf_rows"].shape[0] == min(ref.n_ovf, ovf_cap)
    assert_packed_equal(host, ref)
