"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before any HIP call (CPU only: no kernel is ever launched here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twell.h")

twell = pytest.importorskip("activation_sparse_transformer_bf16_amd")

FAKE = 0x100000  # a non-null, 256-byte aligned address that must never be dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_binding_exports():
    assert set(declared_functions()) == set(twell.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(twell.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert twell.twell_abi_version() == twell.ABI_VERSION == 3
    assert twell.twell_status_str(twell.TWELL_OK) == "ok"
    assert "workspace" in twell.twell_status_str(twell.TWELL_ERR_WORKSPACE)
    assert twell.twell_status_str(99) == "unknown status"


def _matrix(rows=8, cols=512, tile=256, cap=16, dtype=twell.TWELL_BF16, ovf_cap=None, **kw):
    m = twell.TwellMatrixC(rows, cols, tile, cap, dtype, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                           rows if ovf_cap is None else ovf_cap)
    for k, v in kw.items():
        setattr(m, k, v)
    return m


L = twell.lib()


@pytest.mark.parametrize("kw,status", [
    (dict(cols=500), twell.TWELL_ERR_INVALID_ARG),        # cols % tile != 0
    (dict(tile=64, cols=512), twell.TWELL_ERR_UNSUPPORTED),
    (dict(cap=0), twell.TWELL_ERR_INVALID_ARG),
    (dict(cap=65), twell.TWELL_ERR_UNSUPPORTED),
    (dict(dtype=7), twell.TWELL_ERR_INVALID_ARG),
    (dict(rows=-1), twell.TWELL_ERR_INVALID_ARG),
    (dict(ovf_cap=-2), twell.TWELL_ERR_INVALID_ARG),
    (dict(cnt=None), twell.TWELL_ERR_INVALID_ARG),
    (dict(n_ovf=None), twell.TWELL_ERR_INVALID_ARG),
    (dict(ovf_rows=None), twell.TWELL_ERR_INVALID_ARG),  # ovf_cap > 0
    (dict(dense=FAKE + 8), twell.TWELL_ERR_UNSUPPORTED),  # misaligned dense
])
def test_pack_validation(kw, status):
    m = _matrix(**kw)
    assert L.twell_pack(FAKE, ctypes.byref(m), None) == status
    assert twell.twell_last_error() != ""


def test_pack_null_pre_and_misaligned_pre():
    m = _matrix()
    assert L.twell_pack(None, ctypes.byref(m), None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_pack(FAKE + 2, ctypes.byref(m), None) == twell.TWELL_ERR_UNSUPPORTED
    assert L.twell_pack(FAKE, None, None) == twell.TWELL_ERR_INVALID_ARG


def _ffn(m, d=512, ws=FAKE, ws_bytes=1 << 40, x=FAKE, y=FAKE, bias=None):
    return L.twell_ffn_forward(x, FAKE, FAKE, FAKE, bias, y, d, ctypes.byref(m), ws, ws_bytes, None)


def test_ffn_forward_validation():
    assert _ffn(_matrix(), d=256) == twell.TWELL_ERR_UNSUPPORTED     # bf16 needs d % 512
    assert _ffn(_matrix(), d=0) == twell.TWELL_ERR_INVALID_ARG
    assert _ffn(_matrix(), d=16384) == twell.TWELL_ERR_UNSUPPORTED
    assert _ffn(_matrix(ovf_cap=4)) == twell.TWELL_ERR_INVALID_ARG   # ovf_cap < rows
    assert _ffn(_matrix(), x=None) == twell.TWELL_ERR_INVALID_ARG
    assert _ffn(_matrix(), y=FAKE + 4) == twell.TWELL_ERR_UNSUPPORTED
    assert _ffn(_matrix(), bias=FAKE + 2) == twell.TWELL_ERR_UNSUPPORTED
    assert _ffn(_matrix(), ws_bytes=16) == twell.TWELL_ERR_WORKSPACE
    assert _ffn(_matrix(), ws=None) == twell.TWELL_ERR_WORKSPACE
    assert _ffn(_matrix(), ws=FAKE + 16) == twell.TWELL_ERR_UNSUPPORTED
    # fp32 accepts d % 256 up to 4096
    assert _ffn(_matrix(dtype=twell.TWELL_F32), d=384) == twell.TWELL_ERR_UNSUPPORTED
    assert _ffn(_matrix(dtype=twell.TWELL_F32), d=4352) == twell.TWELL_ERR_UNSUPPORTED


def test_sparse_ffn_and_gate_pack_validation():
    m = _matrix(ovf_cap=1)
    assert L.twell_sparse_ffn(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, FAKE, 1 << 40,
                              None) == twell.TWELL_ERR_INVALID_ARG
    m = _matrix()
    assert L.twell_sparse_ffn(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, FAKE, 8,
                              None) == twell.TWELL_ERR_WORKSPACE
    assert L.twell_gate_pack(None, FAKE, None, 512, ctypes.byref(m), None, None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_gate_pack(FAKE, FAKE, None, 512, ctypes.byref(m), FAKE + 8,
                             None) == twell.TWELL_ERR_UNSUPPORTED


def test_saved_u_validation():
    """Only the forward saves u: the other producers of a TwELL matrix reject
    one, the hybrid conversion needs the TwELL u to fill the hybrid's, and a
    misaligned u is rejected (all before any launch)."""
    m = _matrix(u=FAKE)
    assert L.twell_pack(FAKE, ctypes.byref(m), None) == twell.TWELL_ERR_INVALID_ARG
    for f in (L.twell_sparse_ffn_fused, L.twell_sparse_ffn_grouped):
        assert f(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, FAKE, 1 << 40,
                 None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_sparse_ffn(ctypes.byref(_matrix(u=FAKE + 2)), FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, FAKE,
                              1 << 40, None) == twell.TWELL_ERR_UNSUPPORTED
    H = L.twell_to_hybrid
    assert H(ctypes.byref(_matrix(dense=FAKE)), ctypes.byref(_hybrid(u=FAKE)), None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(_matrix(dense=FAKE, u=FAKE)), ctypes.byref(_hybrid(u=FAKE + 2)),
             None) == twell.TWELL_ERR_UNSUPPORTED


def test_layout_validation():
    """The tile-major layout is written by twell_gate_pack and read by the
    overflow scan and the grouped fused kernel only; every other entry point
    rejects it, an unknown layout and a tile-major matrix with u are invalid
    (all before any launch)."""
    tiles = twell.TWELL_LAYOUT_TILES
    for bad in (2, -1):
        assert L.twell_overflow_scan(ctypes.byref(_matrix(layout=bad)), None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_overflow_scan(ctypes.byref(_matrix(layout=tiles, u=FAKE)), None) == twell.TWELL_ERR_INVALID_ARG
    m = _matrix(layout=tiles, dense=FAKE)
    U = twell.TWELL_ERR_UNSUPPORTED
    assert L.twell_pack(FAKE, ctypes.byref(m), None) == U
    for f in (L.twell_sparse_ffn, L.twell_sparse_ffn_fused):
        assert f(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, FAKE, 1 << 40, None) == U
    assert L.twell_ffn_forward(FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, ctypes.byref(m), FAKE, 1 << 40, None) == U
    assert L.twell_ffn_forward_noalloc(FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, ctypes.byref(m), None) == U
    assert L.twell_to_hybrid(ctypes.byref(m), ctypes.byref(_hybrid()), None) == U
    assert L.twell_l1_norm(ctypes.byref(m), FAKE, FAKE, 1 << 20, None) == U
    assert L.twell_l1_grad(ctypes.byref(m), ctypes.c_float(1.0), FAKE, None, None) == U
    # accepted by the grouped kernel's validation: it fails only at the
    # workspace check, after the layout has passed
    assert L.twell_sparse_ffn_grouped(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, FAKE, 10,
                                      None) == twell.TWELL_ERR_WORKSPACE


def test_dense_validation():
    D = L.dense_ffn_forward
    assert D(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 512, 500, 1, FAKE, 1 << 40, None) == twell.TWELL_ERR_UNSUPPORTED
    assert D(FAKE, FAKE, FAKE, FAKE, None, FAKE, -1, 512, 512, 1, FAKE, 1 << 40, None) == twell.TWELL_ERR_INVALID_ARG
    assert D(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 512, 512, 3, FAKE, 1 << 40, None) == twell.TWELL_ERR_INVALID_ARG
    assert D(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 512, 512, 1, FAKE, 10, None) == twell.TWELL_ERR_WORKSPACE


def test_workspace_sizes():
    ws = twell.twell_ffn_workspace_size
    import torch
    n = ws(8192, 2048, 8192, 256, 16, torch.bfloat16)
    # row flags + entry counts + the region the entry lists (8 bytes per TwELL
    # slot) and one fallback chunk of 4096 bf16 rows share + 128 partial tiles
    assert n >= 8192 + 8192 * 4 + max(8192 * 32 * 16 * 8, 4096 * 8192 * 2) + 128 * 256 * 256 * 4
    assert n % 256 == 0
    # smaller than the dense activation matrix [T][F] it stands in for, at the
    # 1.5B-class and the larger layer shapes
    assert n < 128 * 2 ** 20 and n < 8192 * 8192 * 2
    assert ws(16384, 4096, 14336, 256, 16, torch.bfloat16) < 16384 * 14336 * 2
    assert ws(8, 2048, 8192, 100, 16, torch.bfloat16) == 0
    assert ws(8, 300, 8192, 256, 16, torch.bfloat16) == 0
    assert ws(0, 512, 512, 256, 16, torch.bfloat16) >= 256
    assert twell.dense_ffn_workspace_size(64, 256, 1024, torch.float32) == 64 * 1024 * 4


def test_binding_keeps_its_own_argtypes():
    # Reconfiguring the public ctypes handle must not change how the binding
    # marshals pointers (without argtypes ctypes would pass 64-bit device
    # pointers as 32-bit ints).
    pub = twell.lib().twell_pack
    saved = pub.argtypes
    try:
        pub.argtypes = None
        assert twell._lib.twell_pack.argtypes is not None
        assert ctypes.c_void_p in twell._lib.twell_ffn_forward.argtypes
    finally:
        pub.argtypes = saved


def _hybrid(rows=8, cols=512, width=16, dtype=twell.TWELL_BF16, dense_cap=8, **kw):
    h = twell.TwellHybridC(rows, cols, width, dtype, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dense_cap)
    for k, v in kw.items():
        setattr(h, k, v)
    return h


def test_to_hybrid_validation():
    H = L.twell_to_hybrid
    m = _matrix(dense=FAKE)
    assert H(ctypes.byref(m), None, None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(m), ctypes.byref(_hybrid(rows=7)), None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(m), ctypes.byref(_hybrid(cols=256)), None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(m), ctypes.byref(_hybrid(dtype=twell.TWELL_F32)), None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(m), ctypes.byref(_hybrid(width=0)), None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(m), ctypes.byref(_hybrid(n_dense=None)), None) == twell.TWELL_ERR_INVALID_ARG
    assert H(ctypes.byref(m), ctypes.byref(_hybrid(val=FAKE + 1)), None) == twell.TWELL_ERR_UNSUPPORTED
    # the TwELL matrix must carry its dense backup rows, for every row
    m_nodense = _matrix()
    assert H(ctypes.byref(m_nodense), ctypes.byref(_hybrid()), None) == twell.TWELL_ERR_INVALID_ARG
    m_short = _matrix(dense=FAKE, ovf_cap=4)
    assert H(ctypes.byref(m_short), ctypes.byref(_hybrid()), None) == twell.TWELL_ERR_INVALID_ARG


def test_l1_validation():
    assert twell.twell_l1_workspace_size() >= 8
    m = _matrix(dense=FAKE)
    N = L.twell_l1_norm
    assert N(ctypes.byref(m), None, FAKE, 1 << 20, None) == twell.TWELL_ERR_INVALID_ARG
    assert N(ctypes.byref(m), FAKE, FAKE, 8, None) == twell.TWELL_ERR_WORKSPACE
    assert N(ctypes.byref(m), FAKE, None, 1 << 20, None) == twell.TWELL_ERR_WORKSPACE
    assert N(ctypes.byref(m), FAKE + 4, FAKE, 1 << 20, None) == twell.TWELL_ERR_UNSUPPORTED
    assert N(ctypes.byref(_matrix()), FAKE, FAKE, 1 << 20, None) == twell.TWELL_ERR_INVALID_ARG  # no dense rows
    G = L.twell_l1_grad
    assert G(ctypes.byref(m), ctypes.c_float(1.0), None, None, None) == twell.TWELL_ERR_INVALID_ARG
    assert G(ctypes.byref(_matrix()), ctypes.c_float(1.0), FAKE, FAKE, None) == twell.TWELL_ERR_INVALID_ARG
    assert G(ctypes.byref(m), ctypes.c_float(1.0), FAKE + 1, None, None) == twell.TWELL_ERR_UNSUPPORTED


def test_backward_validation_and_workspace():
    import torch
    ws = twell.twell_ffn_backward_workspace_size
    n = ws(8192, 2048, 8192, 256, 8192, torch.bfloat16)
    # per entry slot: (du, dpre) 8 B + position 4 B + column-major record 16 B;
    # F a multiple of 128: the dense rows go to the matrix-core kernels, which
    # need gathered x / dy rows (two bf16 copies each), du / dpre rows and a,
    # du, dpre transposed (high and low bf16 parts)
    slots = 8192 * 256
    dense = 2 * (2 * 8192 * 2048 * 2) + 2 * (8192 * 8192 * 2) + 3 * (8192 * 2 * 8192 * 2)
    assert n >= slots * 28 + dense and n % 256 == 0
    assert n < (slots + 8192 * 8192) * 28  # no entry slots for the dense rows
    # other hidden sizes: the dense rows' entries are walked like the others
    n2 = ws(8192, 2048, 8000, 256, 8192, torch.bfloat16)
    assert n2 >= (8192 * 256 + 8192 * 8000) * 28 and n2 % 256 == 0
    assert ws(8, 8192, 512, 16, 8, torch.bfloat16) == 0      # d above the backward's limit
    assert ws(8, 4096, 512, 16, 8, torch.float32) == 0       # fp32 d above 2048
    assert ws(8, 2048, 32768, 16, 8, torch.bfloat16) == 0    # F above 16384
    assert ws(8, 2048, 512, 0, 8, torch.bfloat16) == 0       # width 0
    assert ws(0, 512, 512, 16, 0, torch.bfloat16) > 0
    B = L.twell_ffn_backward
    h = _hybrid()

    def call(hy, d=512, x=FAKE, dy=FAKE, dx=FAKE, dwg=FAKE, wsb=1 << 40):
        return B(ctypes.byref(hy) if hy is not None else None, x, FAKE, FAKE, FAKE, dy, ctypes.c_float(0.0), d,
                 dx, dwg, FAKE, FAKE, FAKE, wsb, None)

    assert call(None) == twell.TWELL_ERR_INVALID_ARG
    assert call(h, d=300) == twell.TWELL_ERR_UNSUPPORTED
    assert call(h, d=8192) == twell.TWELL_ERR_UNSUPPORTED
    assert call(_hybrid(width=0)) == twell.TWELL_ERR_INVALID_ARG
    assert call(_hybrid(cols=20000)) == twell.TWELL_ERR_UNSUPPORTED
    assert call(_hybrid(n_dense=None)) == twell.TWELL_ERR_INVALID_ARG
    assert call(_hybrid(dense=None)) == twell.TWELL_ERR_INVALID_ARG        # dense_cap > 0 needs the rows
    assert call(_hybrid(dense=FAKE + 2)) == twell.TWELL_ERR_UNSUPPORTED    # matrix-core dense rows: 16-byte aligned
    assert call(_hybrid(col=FAKE + 2)) == twell.TWELL_ERR_UNSUPPORTED
    assert call(h, x=None) == twell.TWELL_ERR_INVALID_ARG
    assert call(h, dwg=None) == twell.TWELL_ERR_INVALID_ARG
    assert call(h, dx=FAKE + 8) == twell.TWELL_ERR_UNSUPPORTED
    assert call(h, wsb=100) == twell.TWELL_ERR_WORKSPACE


def test_stream_probe_validation():
    assert L.twell_stream_probe(FAKE, FAKE, 1024, 2, None) == twell.TWELL_ERR_INVALID_ARG   # mode
    assert L.twell_stream_probe(None, FAKE, 1024, 0, None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_stream_probe(FAKE, None, 1024, 1, None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_stream_probe(FAKE, FAKE, 1000, 1, None) == twell.TWELL_ERR_UNSUPPORTED  # bytes % 16
    assert L.twell_stream_probe(FAKE + 8, FAKE, 1024, 0, None) == twell.TWELL_ERR_UNSUPPORTED
    assert L.twell_stream_probe(FAKE, FAKE + 8, 1024, 1, None) == twell.TWELL_ERR_UNSUPPORTED
    assert L.twell_stream_probe(FAKE, FAKE + 2, 1024, 0, None) == twell.TWELL_ERR_UNSUPPORTED  # sink
    assert L.twell_stream_probe(None, None, 0, 0, None) == twell.TWELL_OK                    # nothing to do


def test_mfma_probe_validation():
    assert L.twell_mfma_probe(None, 10, 4, None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_mfma_probe(FAKE, 0, 4, None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_mfma_probe(FAKE, 10, 0, None) == twell.TWELL_ERR_INVALID_ARG
    assert L.twell_mfma_probe(FAKE + 2, 10, 4, None) == twell.TWELL_ERR_UNSUPPORTED


def test_noalloc_rejects_shapes_beyond_the_static_scratch():
    # 65536 tokens x 8192 units: the entry lists alone need 256 MiB, more than
    # the 64 MiB static scratch; rejected before any HIP call
    m = _matrix(rows=65536, cols=8192)
    st = L.twell_ffn_forward_noalloc(FAKE, FAKE, FAKE, FAKE, None, FAKE, 2048, ctypes.byref(m), None)
    assert st == twell.TWELL_ERR_WORKSPACE
    assert "static scratch" in twell.twell_last_error()
    assert twell.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert "((size_t)64 << 20)" in open(HEADER).read()
    # the validation of the allocating entry point applies as well
    bad = _matrix(rows=8, cols=500)
    assert L.twell_ffn_forward_noalloc(FAKE, FAKE, FAKE, FAKE, None, FAKE, 512, ctypes.byref(bad),
                                       None) == twell.TWELL_ERR_INVALID_ARG
