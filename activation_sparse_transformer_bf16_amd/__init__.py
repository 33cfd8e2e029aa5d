"""Python binding of libtwell.so, the MI355X TwELL sparse-FFN library.

Thin ctypes marshalling over the C ABI declared in ``include/twell.h``: torch
tensors supply device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  The functions carry the same
names as the C entry points.  Importing this package fails loudly when the
library has not been built (``python activation_sparse_transformer_bf16_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# TWELL_LIBRARY names another build of the same library (the host-sanitizer
# build of build.py); by default the in-tree libtwell.so.
LIB_PATH = os.environ.get("TWELL_LIBRARY") or os.path.join(_HERE, "libtwell.so")

TWELL_OK, TWELL_ERR_INVALID_ARG, TWELL_ERR_UNSUPPORTED, TWELL_ERR_WORKSPACE, TWELL_ERR_HIP = range(5)
ABI_VERSION = 3  # TWELL_ABI_VERSION of include/twell.h that these mirrors follow
TWELL_F32, TWELL_BF16 = 0, 1
TWELL_LAYOUT_ROWS, TWELL_LAYOUT_TILES = 0, 1


class TwellMatrixC(ctypes.Structure):
    """Mirror of ``twell_matrix`` (include/twell.h)."""

    _fields_ = [
        ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("tile", ctypes.c_int32),
        ("cap", ctypes.c_int32), ("dtype", ctypes.c_int), ("cnt", ctypes.c_void_p),
        ("val", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("ovf_rows", ctypes.c_void_p),
        ("n_ovf", ctypes.c_void_p), ("dense", ctypes.c_void_p), ("ovf_cap", ctypes.c_int32),
        ("u", ctypes.c_void_p), ("layout", ctypes.c_int),
    ]


LAYOUTS = {"rows": TWELL_LAYOUT_ROWS, "tiles": TWELL_LAYOUT_TILES}  # twell_layout: record (t, k) at t * nt + k, or at k * rows + t


class TwellHybridC(ctypes.Structure):
    """Mirror of ``twell_hybrid`` (include/twell.h)."""

    _fields_ = [
        ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("width", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("cnt", ctypes.c_void_p), ("val", ctypes.c_void_p),
        ("col", ctypes.c_void_p), ("dense_rows", ctypes.c_void_p), ("n_dense", ctypes.c_void_p),
        ("dense", ctypes.c_void_p), ("dense_cap", ctypes.c_int32), ("u", ctypes.c_void_p),
    ]


class TwellError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    # torch ships its own libamdhip64.so.7; importing it first makes libtwell.so
    # bind to that same HIP runtime instead of loading a second one.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python activation_sparse_transformer_bf16_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.twell_abi_version.restype = ctypes.c_int
    if lib.twell_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.twell_abi_version()}, this binding needs {ABI_VERSION}: "
                          "rebuild it")
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    M = ctypes.POINTER(TwellMatrixC)
    sig = {
        "twell_abi_version": (I, []),
        "twell_status_str": (ctypes.c_char_p, [I]),
        "twell_last_error": (ctypes.c_char_p, []),
        "twell_pack": (I, [P, M, P]),
        "twell_ffn_workspace_size": (Z, [I, I, I, I, I, I]),
        "twell_ffn_forward": (I, [P, P, P, P, P, P, I, M, P, Z, P]),
        "twell_ffn_forward_noalloc": (I, [P, P, P, P, P, P, I, M, P]),
        "twell_gate_pack": (I, [P, P, P, I, M, P, P]),
        "twell_overflow_scan": (I, [M, P]),
        "twell_sparse_ffn": (I, [M, P, P, P, P, P, P, I, P, Z, P]),
        "twell_sparse_ffn_fused": (I, [M, P, P, P, P, P, P, I, P, Z, P]),
        "twell_sparse_ffn_grouped": (I, [M, P, P, P, P, P, P, I, P, Z, P]),
        "twell_sparse_ffn_grouped_workspace_size": (Z, [I, I, I, I, I, I]),
        "dense_ffn_workspace_size": (Z, [I, I, I, I]),
        "dense_ffn_forward": (I, [P, P, P, P, P, P, I, I, I, I, P, Z, P]),
        "twell_to_hybrid": (I, [M, ctypes.POINTER(TwellHybridC), P]),
        "twell_l1_workspace_size": (Z, []),
        "twell_l1_norm": (I, [M, P, P, Z, P]),
        "twell_l1_grad": (I, [M, ctypes.c_float, P, P, P]),
        "twell_ffn_backward_workspace_size": (Z, [I, I, I, I, I, I]),
        "twell_stream_probe": (I, [P, P, Z, I, P]),
        "twell_mfma_probe": (I, [P, I, I, P]),
        "twell_ffn_backward": (I, [ctypes.POINTER(TwellHybridC), P, P, P, P, P, ctypes.c_float, I, P, P, P, P,
                                   P, Z, P]),
    }
    # Private function objects: changing argtypes on the public handle (lib())
    # cannot make this binding pass truncated pointers.
    fns = {}
    for name, (res, args) in sig.items():
        for fn in (lib._FuncPtr((name, lib)), getattr(lib, name)):
            fn.restype, fn.argtypes = res, args
        fns[name] = lib._FuncPtr((name, lib))
        fns[name].restype, fns[name].argtypes = res, args
    return lib, fns


class _Fns:
    def __init__(self, fns):
        self.__dict__.update(fns)


_public_lib, _private = _load()
_lib = _Fns(_private)

# Names every build of the library must export (checked by the CPU tests).
EXPORTS = ("twell_abi_version", "twell_status_str", "twell_last_error", "twell_pack",
           "twell_ffn_workspace_size", "twell_ffn_forward", "twell_gate_pack", "twell_overflow_scan",
           "twell_sparse_ffn",
           "dense_ffn_workspace_size", "dense_ffn_forward", "twell_to_hybrid",
           "twell_l1_workspace_size", "twell_l1_norm", "twell_l1_grad",
           "twell_ffn_backward_workspace_size", "twell_ffn_backward", "twell_sparse_ffn_fused",
           "twell_stream_probe", "twell_mfma_probe", "twell_ffn_forward_noalloc", "twell_sparse_ffn_grouped",
           "twell_sparse_ffn_grouped_workspace_size")

# Size of the static device scratch behind twell_ffn_forward_noalloc
# (TWELL_NOALLOC_SCRATCH_BYTES in include/twell.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def lib():
    """The ctypes handle of libtwell.so (its functions have argtypes set)."""
    return _public_lib


def twell_abi_version() -> int:
    return _lib.twell_abi_version()


def twell_status_str(status: int) -> str:
    return _lib.twell_status_str(status).decode()


def twell_last_error() -> str:
    return _lib.twell_last_error().decode()


def _check(status: int):
    if status != TWELL_OK:
        raise TwellError(status, f"{twell_status_str(status)}: {twell_last_error()}")


# --------------------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.float32:
        return TWELL_F32
    if t == torch.bfloat16:
        return TWELL_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, device, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class TwellMatrix:
    """Device buffers of one TwELL matrix (see ``twell_matrix`` in include/twell.h)."""

    rows: int
    cols: int
    tile: int
    cap: int
    dtype: object        # torch dtype of the values
    cnt: object          # int16 [rows, cols/tile] (uint16 bit patterns); tile-major: [cols/tile, rows]
    val: object          # dtype [rows, cols/tile, cap]; tile-major: [cols/tile, rows, cap]
    idx: object          # uint8 [rows, cols/tile, cap]; tile-major: [cols/tile, rows, cap]
    ovf_rows: object     # int32 [ovf_cap]
    n_ovf: object        # int32 [1]
    dense: object        # dtype [ovf_cap, cols] or None
    ovf_cap: int
    u: object = None     # float32 [rows, cols/tile, cap] (u saved by the forward) or None
    layout: str = "rows"  # "rows" (row-major records) or "tiles" (tile-major, see twell_matrix)

    @classmethod
    def empty(cls, rows: int, cols: int, tile: int, cap: int, dtype, device,
              ovf_cap: Optional[int] = None, dense: bool = True, u: bool = False,
              layout: str = "rows") -> "TwellMatrix":
        torch = _torch()
        nt = cols // tile
        ovf_cap = rows if ovf_cap is None else ovf_cap
        if layout not in LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(LAYOUTS)}, got {layout!r}")
        r2 = (rows, nt) if layout == "rows" else (nt, rows)
        return cls(rows, cols, tile, cap, dtype,
                   torch.empty(r2, dtype=torch.int16, device=device),
                   torch.empty(r2 + (cap,), dtype=dtype, device=device),
                   torch.empty(r2 + (cap,), dtype=torch.uint8, device=device),
                   torch.empty((max(ovf_cap, 1),), dtype=torch.int32, device=device),
                   torch.empty((1,), dtype=torch.int32, device=device),
                   torch.empty((max(ovf_cap, 1), cols), dtype=dtype, device=device) if dense else None,
                   ovf_cap,
                   torch.empty(r2 + (cap,), dtype=torch.float32, device=device) if u else None,
                   layout)

    def validate(self, device=None) -> None:
        """Check every buffer against the matrix's own fields (device, dtype,
        shape, contiguity) before its pointers reach the library."""
        torch = _torch()
        device = self.cnt.device if device is None else device
        _dtype_code(self.dtype)
        if self.rows < 0 or self.cols <= 0 or self.tile <= 0 or self.cap <= 0 or self.cols % self.tile:
            raise ValueError(f"bad TwELL shape rows={self.rows} cols={self.cols} tile={self.tile} cap={self.cap}")
        nt = self.cols // self.tile
        if self.layout not in LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(LAYOUTS)}, got {self.layout!r}")
        r2 = (self.rows, nt) if self.layout == "rows" else (nt, self.rows)
        _need(self.cnt, "cnt", device, torch.int16, r2)
        _need(self.val, "val", device, self.dtype, r2 + (self.cap,))
        _need(self.idx, "idx", device, torch.uint8, r2 + (self.cap,))
        _need(self.ovf_rows, "ovf_rows", device, torch.int32)
        if self.ovf_rows.numel() < max(self.ovf_cap, 1):
            raise ValueError(f"ovf_rows holds {self.ovf_rows.numel()} entries, ovf_cap is {self.ovf_cap}")
        _need(self.n_ovf, "n_ovf", device, torch.int32, (1,))
        if self.dense is not None:
            _need(self.dense, "dense", device, self.dtype)
            if self.dense.dim() != 2 or self.dense.shape[1] != self.cols or self.dense.shape[0] < self.ovf_cap:
                raise ValueError(f"dense must have shape (>= {self.ovf_cap}, {self.cols}), "
                                 f"got {tuple(self.dense.shape)}")
        if self.u is not None:
            _need(self.u, "u", device, torch.float32, r2 + (self.cap,))

    def c_struct(self) -> TwellMatrixC:
        return TwellMatrixC(self.rows, self.cols, self.tile, self.cap, _dtype_code(self.dtype),
                            _ptr(self.cnt), _ptr(self.val), _ptr(self.idx), _ptr(self.ovf_rows),
                            _ptr(self.n_ovf), _ptr(self.dense), self.ovf_cap, _ptr(self.u),
                            LAYOUTS.get(self.layout, -1))

    @property
    def device(self):
        return self.cnt.device


@dataclass
class TwellHybrid:
    """Device buffers of one hybrid matrix (see ``twell_hybrid`` in include/twell.h)."""

    rows: int
    cols: int
    width: int
    dtype: object        # torch dtype of the values
    cnt: object          # int32 [rows]
    val: object          # dtype [rows, width]
    col: object          # int32 [rows, width]
    dense_rows: object   # int32 [dense_cap]
    n_dense: object      # int32 [1]
    dense: object        # dtype [dense_cap, cols] or None
    dense_cap: int
    u: object = None     # float32 [rows, width] (saved u of the ELL slots) or None

    @classmethod
    def empty(cls, rows: int, cols: int, width: int, dtype, device, dense_cap: Optional[int] = None,
              dense: bool = True, u: bool = False) -> "TwellHybrid":
        torch = _torch()
        dense_cap = rows if dense_cap is None else dense_cap
        return cls(rows, cols, width, dtype,
                   torch.empty((rows,), dtype=torch.int32, device=device),
                   torch.empty((rows, width), dtype=dtype, device=device),
                   torch.empty((rows, width), dtype=torch.int32, device=device),
                   torch.empty((max(dense_cap, 1),), dtype=torch.int32, device=device),
                   torch.empty((1,), dtype=torch.int32, device=device),
                   torch.empty((max(dense_cap, 1), cols), dtype=dtype, device=device) if dense else None,
                   dense_cap,
                   torch.empty((rows, width), dtype=torch.float32, device=device) if u else None)

    def validate(self, device=None) -> None:
        """Check every buffer against the hybrid matrix's own fields."""
        torch = _torch()
        device = self.cnt.device if device is None else device
        _dtype_code(self.dtype)
        if self.rows < 0 or self.cols <= 0 or self.width < 1 or self.dense_cap < 0:
            raise ValueError(f"bad hybrid shape rows={self.rows} cols={self.cols} width={self.width}")
        _need(self.cnt, "cnt", device, torch.int32, (self.rows,))
        _need(self.val, "val", device, self.dtype, (self.rows, self.width))
        _need(self.col, "col", device, torch.int32, (self.rows, self.width))
        _need(self.dense_rows, "dense_rows", device, torch.int32)
        if self.dense_rows.numel() < max(self.dense_cap, 1):
            raise ValueError(f"dense_rows holds {self.dense_rows.numel()} entries, dense_cap is {self.dense_cap}")
        _need(self.n_dense, "n_dense", device, torch.int32, (1,))
        if self.dense is not None:
            _need(self.dense, "dense", device, self.dtype)
            if self.dense.dim() != 2 or self.dense.shape[1] != self.cols or self.dense.shape[0] < self.dense_cap:
                raise ValueError(f"dense must have shape (>= {self.dense_cap}, {self.cols}), "
                                 f"got {tuple(self.dense.shape)}")
        if self.u is not None:
            _need(self.u, "u", device, torch.float32, (self.rows, self.width))

    def c_struct(self) -> TwellHybridC:
        return TwellHybridC(self.rows, self.cols, self.width, _dtype_code(self.dtype), _ptr(self.cnt),
                            _ptr(self.val), _ptr(self.col), _ptr(self.dense_rows), _ptr(self.n_dense),
                            _ptr(self.dense), self.dense_cap, _ptr(self.u))


def twell_to_hybrid(packed: TwellMatrix, width: int, dense_cap: Optional[int] = None, dense: bool = True,
                    out: Optional[TwellHybrid] = None) -> TwellHybrid:
    """Convert a TwELL matrix (with its dense backup rows) to the hybrid format;
    a new ``out`` carries the saved u when the TwELL matrix has one."""
    packed.validate()
    if out is None:
        out = TwellHybrid.empty(packed.rows, packed.cols, width, packed.dtype, packed.device, dense_cap, dense,
                                u=packed.u is not None)
    out.validate(packed.device)
    if (out.rows, out.cols, out.width, out.dtype) != (packed.rows, packed.cols, width, packed.dtype):
        raise ValueError("out must be a hybrid matrix of the TwELL matrix's rows, cols and dtype at this width")
    m = packed.c_struct()
    h = out.c_struct()
    _check(_lib.twell_to_hybrid(ctypes.byref(m), ctypes.byref(h), _stream(packed.device)))
    return out


def twell_l1_workspace_size() -> int:
    return int(_lib.twell_l1_workspace_size())


def twell_l1_norm(packed: TwellMatrix, out=None, workspace=None):
    """||h||_1 of the activations a TwELL matrix describes, as a float64 device tensor [1]."""
    torch = _torch()
    device = packed.device
    packed.validate()
    if out is None:
        out = torch.empty((1,), dtype=torch.float64, device=device)
    _need(out, "out", device, torch.float64, (1,))
    ws = _workspace(twell_l1_workspace_size(), device, workspace)
    m = packed.c_struct()
    _check(_lib.twell_l1_norm(ctypes.byref(m), _ptr(out), _ptr(ws), ws.numel(), _stream(device)))
    return out


def twell_l1_grad(packed: TwellMatrix, lam: float, grad_val=None, grad_dense=None, dense: bool = True):
    """d(lam ||h||_1)/dh in the TwELL pattern: (grad_val, grad_dense or None)."""
    torch = _torch()
    device = packed.device
    packed.validate()
    if grad_val is None:
        grad_val = torch.empty_like(packed.val)
    if grad_dense is None and dense and packed.dense is not None:
        grad_dense = torch.empty_like(packed.dense)
    _need(grad_val, "grad_val", device, packed.dtype, tuple(packed.val.shape))
    if grad_dense is not None:
        if packed.dense is None:
            raise ValueError("grad_dense needs the TwELL matrix's dense backup rows")
        _need(grad_dense, "grad_dense", device, packed.dtype, tuple(packed.dense.shape))
    m = packed.c_struct()
    _check(_lib.twell_l1_grad(ctypes.byref(m), ctypes.c_float(lam), _ptr(grad_val), _ptr(grad_dense),
                              _stream(device)))
    return grad_val, grad_dense


def twell_ffn_backward_workspace_size(T: int, d: int, F: int, width: int, dense_cap: int, dtype) -> int:
    return int(_lib.twell_ffn_backward_workspace_size(T, d, F, width, dense_cap, _dtype_code(dtype)))


def twell_ffn_backward(hy: TwellHybrid, x, w_gate, w_up, w_down, dy, lam: float = 0.0, dx=None, dw_gate=None,
                       dw_up=None, dw_down=None, workspace=None):
    """Gradients of the FFN layer from its hybrid activations: (dx, dw_gate, dw_up, dw_down);
    dx in the activation dtype, the weight gradients fp32 [F, d]."""
    torch = _torch()
    device = x.device
    T, d = x.shape
    F = hy.cols
    hy.validate(device)
    _need(x, "x", device, hy.dtype, (hy.rows, d))
    _need(dy, "dy", device, hy.dtype, (T, d))
    for w, name in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _need(w, name, device, hy.dtype, (F, d))
    if dx is None:
        dx = torch.empty((T, d), dtype=hy.dtype, device=device)
    outs = []
    for g, name in ((dw_gate, "dw_gate"), (dw_up, "dw_up"), (dw_down, "dw_down")):
        if g is None:
            g = torch.empty((F, d), dtype=torch.float32, device=device)
        _need(g, name, device, torch.float32, (F, d))
        outs.append(g)
    _need(dx, "dx", device, hy.dtype, (T, d))
    ws = _workspace(twell_ffn_backward_workspace_size(T, d, F, hy.width, hy.dense_cap, hy.dtype), device,
                    workspace)
    h = hy.c_struct()
    _check(_lib.twell_ffn_backward(ctypes.byref(h), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dy),
                                   ctypes.c_float(lam), d, _ptr(dx), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                   _ptr(ws), ws.numel(), _stream(device)))
    return dx, outs[0], outs[1], outs[2]


def twell_pack(pre, tile: int, cap: int, ovf_cap: Optional[int] = None, dense: bool = True,
               out: Optional[TwellMatrix] = None) -> TwellMatrix:
    """Pack a pre-activation matrix [T, F] (fp32 or bf16, on the GPU) into TwELL."""
    device = pre.device
    _need(pre, "pre", device)
    _dtype_code(pre.dtype)
    if pre.dim() != 2:
        raise ValueError(f"pre must be 2-D [T, F], got shape {tuple(pre.shape)}")
    T, F = pre.shape
    if out is None:
        out = TwellMatrix.empty(T, F, tile, cap, pre.dtype, device, ovf_cap, dense)
    out.validate(device)
    if (out.rows, out.cols, out.tile, out.cap, out.dtype) != (T, F, tile, cap, pre.dtype):
        raise ValueError(f"out ({out.rows}x{out.cols}, tile {out.tile}, cap {out.cap}, {out.dtype}) does not "
                         f"match pre ({T}x{F}, {pre.dtype}) at tile {tile}, cap {cap}")
    m = out.c_struct()
    _check(_lib.twell_pack(_ptr(pre), ctypes.byref(m), _stream(device)))
    return out


def twell_ffn_workspace_size(T: int, d: int, F: int, tile: int, cap: int, dtype) -> int:
    return int(_lib.twell_ffn_workspace_size(T, d, F, tile, cap, _dtype_code(dtype)))


def dense_ffn_workspace_size(T: int, d: int, F: int, dtype) -> int:
    return int(_lib.dense_ffn_workspace_size(T, d, F, _dtype_code(dtype)))


def _ffn_checks(x, w_gate, w_up, w_down, gate_bias):
    torch = _torch()
    device = x.device
    if x.dim() != 2 or w_gate.dim() != 2:
        raise ValueError("x and the weights must be 2-D")
    T, d = x.shape
    F = w_gate.shape[0]
    _need(x, "x", device)
    _dtype_code(x.dtype)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(w, name, device, x.dtype, (F, d))
    if gate_bias is not None:
        _need(gate_bias, "gate_bias", device, torch.float32, (T,))
    return device, T, d, F


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        _need(workspace, "workspace", device, torch.uint8)
        if workspace.numel() >= nbytes:
            return workspace
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def _packed_for(packed: TwellMatrix, device, T: int, F: int, dtype) -> None:
    """A caller's TwELL matrix must describe exactly the activations of x."""
    packed.validate(device)
    if (packed.rows, packed.cols, packed.dtype) != (T, F, dtype):
        raise ValueError(f"packed ({packed.rows}x{packed.cols}, {packed.dtype}) does not match the layer "
                         f"({T} tokens x {F} units, {dtype})")


def twell_ffn_forward(x, w_gate, w_up, w_down, gate_bias=None, tile: int = 256, cap: int = 16,
                      packed: Optional[TwellMatrix] = None, y=None, workspace=None
                      ) -> Tuple[object, TwellMatrix]:
    """y = (ReLU(x W_g^T + beta) * (x W_u^T)) W_d through TwELL; returns (y, packed)."""
    torch = _torch()
    device, T, d, F = _ffn_checks(x, w_gate, w_up, w_down, gate_bias)
    if packed is None:
        packed = TwellMatrix.empty(T, F, tile, cap, x.dtype, device, T, dense=False)
    _packed_for(packed, device, T, F, x.dtype)
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=device)
    _need(y, "y", device, x.dtype, (T, d))
    ws = _workspace(twell_ffn_workspace_size(T, d, F, packed.tile, packed.cap, x.dtype), device, workspace)
    m = packed.c_struct()
    _check(_lib.twell_ffn_forward(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(gate_bias),
                                  _ptr(y), d, ctypes.byref(m), _ptr(ws),
                                  ws.numel(), _stream(device)))
    return y, packed


def twell_ffn_forward_noalloc(x, w_gate, w_up, w_down, packed: TwellMatrix, y, gate_bias=None):
    """twell_ffn_forward with its workspace in the library's static device
    scratch: the caller passes the outputs (packed, y) and nothing is
    allocated.  Calls that overlap on one GPU race (one scratch per GPU)."""
    device, T, d, F = _ffn_checks(x, w_gate, w_up, w_down, gate_bias)
    _packed_for(packed, device, T, F, x.dtype)
    _need(y, "y", device, x.dtype, (T, d))
    m = packed.c_struct()
    _check(_lib.twell_ffn_forward_noalloc(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(gate_bias),
                                          _ptr(y), d, ctypes.byref(m), _stream(device)))
    return y, packed


def twell_gate_pack(x, w_gate, gate_bias=None, tile: int = 256, cap: int = 16,
                    packed: Optional[TwellMatrix] = None, pre_out: bool = False, scan: bool = True):
    """Gate matmul + TwELL epilogue (one kernel), then, with ``scan``, the overflow
    scan; returns (packed, pre or None)."""
    torch = _torch()
    device = x.device
    if x.dim() != 2 or w_gate.dim() != 2:
        raise ValueError("x and w_gate must be 2-D")
    T, d = x.shape
    F = w_gate.shape[0]
    _need(x, "x", device)
    _dtype_code(x.dtype)
    _need(w_gate, "w_gate", device, x.dtype, (F, d))
    if gate_bias is not None:
        _need(gate_bias, "gate_bias", device, torch.float32, (T,))
    if packed is None:
        packed = TwellMatrix.empty(T, F, tile, cap, x.dtype, device, T, dense=False)
    _packed_for(packed, device, T, F, x.dtype)
    pre = torch.empty((T, F), dtype=x.dtype, device=device) if pre_out else None
    m = packed.c_struct()
    _check(_lib.twell_gate_pack(_ptr(x), _ptr(w_gate), _ptr(gate_bias), d, ctypes.byref(m),
                                _ptr(pre), _stream(device)))
    if scan:
        twell_overflow_scan(packed)
    return packed, pre


def twell_overflow_scan(packed: TwellMatrix) -> TwellMatrix:
    """List the overflowing rows of a packed matrix (fills ovf_rows and n_ovf)."""
    packed.validate()
    m = packed.c_struct()
    _check(_lib.twell_overflow_scan(ctypes.byref(m), _stream(packed.device)))
    return packed


def twell_sparse_ffn(packed: TwellMatrix, x, w_gate, w_up, w_down, gate_bias=None, y=None,
                     workspace=None):
    """Up / down projections over TwELL plus the dense fallback; returns y."""
    torch = _torch()
    device, T, d, F = _ffn_checks(x, w_gate, w_up, w_down, gate_bias)
    _packed_for(packed, device, T, F, x.dtype)
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=device)
    _need(y, "y", device, x.dtype, (T, d))
    ws = _workspace(twell_ffn_workspace_size(T, d, F, packed.tile, packed.cap, x.dtype), device, workspace)
    m = packed.c_struct()
    _check(_lib.twell_sparse_ffn(ctypes.byref(m), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                 _ptr(gate_bias), _ptr(y), d, _ptr(ws), ws.numel(),
                                 _stream(device)))
    return y


def twell_sparse_ffn_fused(packed: TwellMatrix, x, w_gate, w_up, w_down, gate_bias=None, y=None,
                           workspace=None):
    """twell_sparse_ffn with the up and down projections in one kernel; returns y."""
    torch = _torch()
    device, T, d, F = _ffn_checks(x, w_gate, w_up, w_down, gate_bias)
    _packed_for(packed, device, T, F, x.dtype)
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=device)
    _need(y, "y", device, x.dtype, (T, d))
    ws = _workspace(twell_ffn_workspace_size(T, d, F, packed.tile, packed.cap, x.dtype), device, workspace)
    m = packed.c_struct()
    _check(_lib.twell_sparse_ffn_fused(ctypes.byref(m), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                       _ptr(gate_bias), _ptr(y), d, _ptr(ws), ws.numel(), _stream(device)))
    return y


def twell_sparse_ffn_grouped_workspace_size(T: int, d: int, F: int, tile: int, cap: int, dtype) -> int:
    return int(_lib.twell_sparse_ffn_grouped_workspace_size(T, d, F, tile, cap, _dtype_code(dtype)))


def twell_sparse_ffn_grouped(packed: TwellMatrix, x, w_gate, w_up, w_down, gate_bias=None, y=None,
                             workspace=None):
    """twell_sparse_ffn with the fused up+down kernel in hidden-group-major order
    (fp32 partial output rows per group, added in group order); returns y."""
    torch = _torch()
    device, T, d, F = _ffn_checks(x, w_gate, w_up, w_down, gate_bias)
    _packed_for(packed, device, T, F, x.dtype)
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=device)
    _need(y, "y", device, x.dtype, (T, d))
    ws = _workspace(twell_sparse_ffn_grouped_workspace_size(T, d, F, packed.tile, packed.cap, x.dtype), device,
                    workspace)
    m = packed.c_struct()
    _check(_lib.twell_sparse_ffn_grouped(ctypes.byref(m), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                         _ptr(gate_bias), _ptr(y), d, _ptr(ws), ws.numel(), _stream(device)))
    return y


def dense_ffn_forward(x, w_gate, w_up, w_down, gate_bias=None, y=None, workspace=None):
    """The same layer computed densely on the matrix cores (baseline)."""
    torch = _torch()
    device, T, d, F = _ffn_checks(x, w_gate, w_up, w_down, gate_bias)
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=device)
    _need(y, "y", device, x.dtype, (T, d))
    ws = _workspace(dense_ffn_workspace_size(T, d, F, x.dtype), device, workspace)
    _check(_lib.dense_ffn_forward(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(gate_bias),
                                  _ptr(y), T, d, F, _dtype_code(x.dtype), _ptr(ws), ws.numel(),
                                  _stream(device)))
    return y


def twell_stream_probe(src, dst, mode: int) -> None:
    """Streaming HBM probe on the current stream: mode 0 reads src (dst is a
    device sink of at least 4 bytes), mode 1 copies src into dst."""
    device = src.device
    _need(src, "src", device)
    _need(dst, "dst", device)
    nbytes = src.numel() * src.element_size()
    if mode == 1 and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    if mode == 0 and dst.numel() * dst.element_size() < 4:
        raise ValueError("the sink needs 4 bytes")
    _check(_lib.twell_stream_probe(_ptr(src), _ptr(dst), nbytes, mode, _stream(device)))


def twell_mfma_probe(sink, iters: int, blocks: int) -> float:
    """Matrix-core probe on the current stream; returns the flops it performs
    (sink: a device tensor of at least 4 bytes)."""
    _need(sink, "sink", sink.device)
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("the sink needs 4 bytes")
    _check(_lib.twell_mfma_probe(_ptr(sink), iters, blocks, _stream(sink.device)))
    return 2.0 * 32 * 32 * 16 * 8 * iters * 8 * blocks
