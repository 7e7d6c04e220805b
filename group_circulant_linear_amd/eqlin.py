"""Thin Python binding of libeqlin.so (argument marshalling only).

Every step of the layer runs in the HIP library; this module checks tensor
shapes, dtypes, devices and contiguity, allocates outputs with PyTorch (device
memory plumbing) and passes raw pointers plus torch's current HIP stream to the
C ABI declared in include/eqlin.h and include/eqconv.h.  There is no fallback:
if the library is not built, every call raises.
"""
from __future__ import annotations

import collections
import ctypes
import functools
import os
import re
from typing import NamedTuple, Optional

import torch

from .build import LIB, INCLUDE

T_P4 = 4
EQLIN_P4M = 108         # group code of p4m (dihedral, order 8); 4 and 8 are the cyclic groups
GROUP_CODES = {"p4": 4, "c4": 4, "c8": 8, "p4m": EQLIN_P4M}


def group_code(group) -> int:
    """Group code for the C ABI's T argument from 4, 8, EQLIN_P4M or a name."""
    code = GROUP_CODES.get(group, group) if isinstance(group, str) else int(group)
    if code not in (4, 8, EQLIN_P4M):
        raise ValueError(f"unsupported group {group!r}; use 'p4' (4), 'c8' (8) or 'p4m'")
    return code


def group_order(code: int) -> int:
    return 8 if code == EQLIN_P4M else code
EQLIN_F32, EQLIN_F16 = 0, 1
STATUS = {0: "EQLIN_OK", 1: "EQLIN_EINVAL", 2: "EQLIN_ENOTSUP", 3: "EQLIN_EALIGN",
          4: "EQLIN_EWORKSPACE", 5: "EQLIN_EHIP"}
_DTYPES = {torch.float32: EQLIN_F32, torch.float16: EQLIN_F16}

_lib: Optional[ctypes.CDLL] = None


class EqlinError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


def header_symbols() -> list:
    """Names of every function the headers under include/ declare."""
    names = set()
    for name in sorted(os.listdir(INCLUDE)):
        if not name.endswith(".h"):
            continue
        with open(os.path.join(INCLUDE, name)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        names.update(re.findall(r"\b((?:eqlin|eqconv)_\w+)\s*\(", text))
    return sorted(names)


def load_library(path: str = LIB) -> ctypes.CDLL:
    """Load libeqlin.so and declare the C signatures (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                           "or python -m group_circulant_linear_amd.build")
    lib = ctypes.CDLL(path)
    c_int, c_i64, c_sz, c_vp, c_fp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    sigs = {
        "eqlin_version": (c_int, []),
        "eqlin_status_str": (ctypes.c_char_p, [c_int]),
        "eqlin_last_hip_error": (c_int, []),
        "eqlin_prepared_weight_bytes": (c_sz, [c_int, c_int, c_int, c_int]),
        "eqlin_prepared_transpose_offset": (c_sz, [c_int, c_int, c_int, c_int]),
        "eqlin_prepare_weights": (c_int, [c_vp, c_int, c_int, c_int, c_int, c_vp, c_sz, c_vp]),
        "eqlin_forward_plan": (c_int, [c_i64, c_int, c_int, c_int, c_int, ctypes.POINTER(c_int),
                                       ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
        "eqlin_forward": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_int, c_vp]),
        "eqlin_forward_ex": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_int, c_vp, c_int, c_vp]),
        "eqlin_forward_residual": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_int, c_vp, c_vp, c_int,
                                           c_vp]),
        "eqlin_forward_workspace_bytes": (c_sz, [c_i64, c_int, c_int, c_int, c_int, ctypes.POINTER(c_int)]),
        "eqlin_forward_ws": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_int, c_vp, c_vp, c_vp, c_sz,
                                     c_int, c_vp]),
        "eqlin_backward_workspace_bytes": (c_sz, [c_i64, c_int, c_int, c_int, c_int]),
        "eqlin_backward": (c_int, [c_vp, c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_fp, c_vp, c_sz,
                                   c_int, c_vp]),
        "eqlin_backward_dx": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_int, c_vp]),
        "eqlin_backward_dw": (c_int, [c_vp, c_vp, c_i64, c_int, c_int, c_int, c_fp, c_vp, c_sz, c_int, c_vp]),
        "eqlin_backward_noalloc": (c_int, [c_vp, c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_fp, c_int, c_vp]),
        "eqconv_prepared_weight_bytes": (c_sz, [c_int, c_int, c_int, c_int]),
        "eqconv_prepared_adjoint_offset": (c_sz, [c_int, c_int, c_int, c_int]),
        "eqconv_prepare_weights": (c_int, [c_vp, c_int, c_int, c_int, c_int, c_vp, c_sz, c_vp]),
        "eqconv_forward": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_int, c_vp,
                                   c_int, c_vp]),
        "eqconv_backward_workspace_bytes": (c_sz, [c_i64, c_int, c_int, c_int, c_int, c_int, c_int]),
        "eqconv_backward": (c_int, [c_vp, c_vp, c_i64, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_fp,
                                    c_vp, c_sz, c_int, c_vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.eqlin_status_str(status).decode()
        if status == 5:
            msg += f", hipError {lib.eqlin_last_hip_error()}"
        raise EqlinError(fn, status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or float16")
    return _DTYPES[t.dtype]


def _need_cuda(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype) -> None:
    """A caller-supplied output: the C ABI takes no output size, so a wrong
    shape or dtype would be written past the buffer; refuse it before any
    launch."""
    _need_cuda(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {list(shape)} of dtype {dtype}, got {list(t.shape)} of {t.dtype}")


def _stream(t: torch.Tensor) -> int:
    """torch's current HIP stream on t's device, as the raw hipStream_t (the
    same value torch.cuda.current_stream(dev).cuda_stream gives, without
    building a stream object on every call)."""
    return torch._C._cuda_getCurrentRawStream(t.device.index)


@functools.lru_cache(maxsize=256)
def _prepared_bytes(C: int, D: int, T: int, dt: int) -> int:
    return int(load_library().eqlin_prepared_weight_bytes(C, D, T, dt))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Prepared(NamedTuple):
    """Prepared weight spectra (opaque byte buffer) and the layer they belong to
    (T is the group code: 4, 8 or EQLIN_P4M)."""
    buf: torch.Tensor
    C: int
    D: int
    dtype: torch.dtype
    T: int = T_P4

    @property
    def order(self) -> int:
        return group_order(self.T)


def eqlin_prepared_weight_bytes(C: int, D: int, dtype: torch.dtype, T=T_P4) -> int:
    return int(load_library().eqlin_prepared_weight_bytes(C, D, group_code(T), _DTYPES[dtype]))


def eqlin_prepared_transpose_offset(C: int, D: int, dtype: torch.dtype, T=T_P4) -> int:
    return int(load_library().eqlin_prepared_transpose_offset(C, D, group_code(T), _DTYPES[dtype]))


def eqlin_prepare_weights(w: torch.Tensor, out: Optional[torch.Tensor] = None, group=None) -> Prepared:
    """w [D/n][C/n][n] -> prepared spectra for eqlin_forward / eqlin_backward.

    group: None for the cyclic group of order n = w.shape[2] (4 or 8), or
    'p4m' / EQLIN_P4M for the dihedral group (n = 8)."""
    lib = load_library()
    _need_cuda(w, "w")
    dt = _dtype_code(w)
    if w.dim() != 3:
        raise ValueError(f"w must have shape [D/n, C/n, n], got {tuple(w.shape)}")
    T = group_code(int(w.shape[2]) if group is None else group)
    if w.shape[2] != group_order(T):
        raise ValueError(f"w's last dimension {w.shape[2]} is not the group order {group_order(T)}")
    n = group_order(T)
    D, C = n * w.shape[0], n * w.shape[1]
    nbytes = _prepared_bytes(C, D, T, dt)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    _need_cuda(out, "out")
    _check("eqlin_prepare_weights",
           lib.eqlin_prepare_weights(_ptr(w), C, D, T, dt, _ptr(out), out.numel() * out.element_size(),
                                     _stream(w)))
    return Prepared(out, C, D, w.dtype, T)


def eqlin_forward_plan(N: int, C: int, D: int, dtype: torch.dtype, T=T_P4) -> dict:
    """The forward launch's tile code, tile count and whole-tile count for this shape (no device work)."""
    lib = load_library()
    tile, tiles, whole = ctypes.c_int(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check("eqlin_forward_plan", lib.eqlin_forward_plan(N, C, D, group_code(T), _DTYPES[dtype], ctypes.byref(tile),
                                                         ctypes.byref(tiles), ctypes.byref(whole)))
    return {"tile": tile.value, "tiles": tiles.value, "whole": whole.value}


def eqlin_forward_workspace_bytes(N: int, C: int, D: int, dtype: torch.dtype, T=T_P4) -> tuple:
    """(bytes, parts) of eqlin_forward_ws's K-split workspace for this shape ((0, 0): none needed)."""
    return _fwd_ws_bytes(N, C, D, group_code(T), _DTYPES[dtype], os.environ.get("EQLIN_FWD_TILE"),
                         os.environ.get("EQLIN_FWD_SPLIT"))


@functools.lru_cache(maxsize=256)
def _fwd_ws_bytes(N: int, C: int, D: int, T: int, dt: int, tile_env, split_env) -> tuple:
    # the plan depends on the shape and on the two environment overrides, which are part of the key
    parts = ctypes.c_int(0)
    nbytes = load_library().eqlin_forward_workspace_bytes(N, C, D, T, dt, ctypes.byref(parts))
    return int(nbytes), parts.value


# The forward's K-split workspaces, one per (device, stream): allocated
# zero-filled on that stream (its arrival counters must start at zero, and
# every launch leaves them zero), grown when a larger layer needs more.
# Launches on one stream run in order, so they can share one workspace.  At
# most _FWD_WS_MAX are kept (least recently used first out): a dropped one
# was allocated and used on its own stream only, so torch's allocator reuses
# its memory in that stream's order.
_FWD_WS: "collections.OrderedDict" = collections.OrderedDict()
_FWD_WS_MAX = 8


def _forward_workspace(X: torch.Tensor, N: int, W_hat: Prepared) -> Optional[torch.Tensor]:
    nbytes, _ = eqlin_forward_workspace_bytes(N, W_hat.C, W_hat.D, W_hat.dtype, W_hat.T)
    if nbytes == 0:
        return None
    key = (X.device.index, _stream(X))
    ws = _FWD_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=X.device)
        _FWD_WS[key] = ws
    _FWD_WS.move_to_end(key)
    while len(_FWD_WS) > _FWD_WS_MAX:
        _FWD_WS.popitem(last=False)
    return ws


def _check_workspace(ws: torch.Tensor, N: int, W_hat: Prepared) -> None:
    _need_cuda(ws, "workspace")
    if ws.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    nbytes, _ = eqlin_forward_workspace_bytes(N, W_hat.C, W_hat.D, W_hat.dtype, W_hat.T)
    if ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the layer needs {nbytes}")


def eqlin_forward(X: torch.Tensor, W_hat: Prepared, out: Optional[torch.Tensor] = None,
                  workspace="auto") -> torch.Tensor:
    """Y = X W^T for the group-circulant W, X [N][C] -> Y [N][D].

    workspace: "auto" (a zero-filled workspace kept per device and stream, so
    that float32 layers can split the k axis of their last round of tiles:
    eqlin_forward_ws), None (eqlin_forward: no K split), or a caller's uint8
    tensor of at least eqlin_forward_workspace_bytes bytes, zero-filled before
    its first use."""
    return eqlin_forward_ex(X, W_hat, out=out, workspace=workspace)


ACT = {"none": 0, "gelu": 1}


def eqlin_forward_ex(X: torch.Tensor, W_hat: Prepared, bias: Optional[torch.Tensor] = None, act: str = "none",
                     out: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
                     workspace="auto") -> torch.Tensor:
    """Y = act(X W^T + b) (+ residual) in one kernel; bias [D/n] (group-invariant, storage dtype) or None;
    residual [N][D] in X's dtype or None (it may be `out` itself: an in-place update); workspace as for
    eqlin_forward."""
    lib = load_library()
    _need_cuda(X, "X")
    dt = _dtype_code(X)
    if X.dtype != W_hat.dtype:
        raise TypeError("X and the prepared weights differ in dtype")
    if X.dim() != 2 or X.shape[1] != W_hat.C:
        raise ValueError(f"X must have shape [N, {W_hat.C}], got {tuple(X.shape)}")
    if act not in ACT:
        raise ValueError(f"act must be one of {sorted(ACT)}")
    if bias is not None:
        _need_cuda(bias, "bias")
        if bias.dtype != X.dtype or tuple(bias.shape) != (W_hat.D // W_hat.order,):
            raise ValueError(f"bias must be [{W_hat.D // W_hat.order}] of dtype {X.dtype}")
    N = X.shape[0]
    if residual is not None:
        _need_cuda(residual, "residual")
        if residual.dtype != X.dtype or tuple(residual.shape) != (N, W_hat.D):
            raise ValueError(f"residual must be [{N}, {W_hat.D}] of dtype {X.dtype}")
    if out is None:
        out = torch.empty((N, W_hat.D), dtype=X.dtype, device=X.device)
    _check_out(out, "out", (N, W_hat.D), X.dtype)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 device tensor')
        workspace = _forward_workspace(X, N, W_hat)
    elif workspace is not None:
        _check_workspace(workspace, N, W_hat)
    if workspace is not None:
        _check("eqlin_forward_ws",
               lib.eqlin_forward_ws(_ptr(X), N, W_hat.C, W_hat.D, W_hat.T, _ptr(W_hat.buf), _ptr(bias), ACT[act],
                                    _ptr(residual), _ptr(out), _ptr(workspace), workspace.numel(), dt, _stream(X)))
    elif residual is None and bias is None and act == "none":
        _check("eqlin_forward", lib.eqlin_forward(_ptr(X), N, W_hat.C, W_hat.D, W_hat.T, _ptr(W_hat.buf),
                                                  _ptr(out), dt, _stream(X)))
    elif residual is None:
        _check("eqlin_forward_ex", lib.eqlin_forward_ex(_ptr(X), N, W_hat.C, W_hat.D, W_hat.T, _ptr(W_hat.buf),
                                                        _ptr(bias), ACT[act], _ptr(out), dt, _stream(X)))
    else:
        _check("eqlin_forward_residual",
               lib.eqlin_forward_residual(_ptr(X), N, W_hat.C, W_hat.D, W_hat.T, _ptr(W_hat.buf), _ptr(bias),
                                          ACT[act], _ptr(residual), _ptr(out), dt, _stream(X)))
    return out


def eqlin_backward_workspace_bytes(N: int, C: int, D: int, dtype: torch.dtype, T=T_P4) -> int:
    return int(load_library().eqlin_backward_workspace_bytes(N, C, D, group_code(T), _DTYPES[dtype]))


def eqlin_backward(dY: torch.Tensor, X: Optional[torch.Tensor], W_hat: Prepared, need_dx: bool = True,
                   need_dw: bool = True, workspace: Optional[torch.Tensor] = None,
                   dX_out: Optional[torch.Tensor] = None, dw_out: Optional[torch.Tensor] = None):
    """(dX [N][C] or None, dw [D/n][C/n][n] float32 or None) for upstream gradient dY [N][D]."""
    lib = load_library()
    _need_cuda(dY, "dY")
    dt = _dtype_code(dY)
    if dY.dtype != W_hat.dtype:
        raise TypeError("dY and the prepared weights differ in dtype")
    C, D, T, n = W_hat.C, W_hat.D, W_hat.T, W_hat.order
    if dY.dim() != 2 or dY.shape[1] != D:
        raise ValueError(f"dY must have shape [N, {D}], got {tuple(dY.shape)}")
    N = dY.shape[0]
    if not (need_dx or need_dw):
        raise ValueError("nothing to compute")
    dX = dw = None
    if need_dx:
        dX = dX_out if dX_out is not None else torch.empty((N, C), dtype=dY.dtype, device=dY.device)
        _check_out(dX, "dX_out", (N, C), dY.dtype)
    ws_bytes = 0
    if need_dw:
        if X is None:
            raise ValueError("dw needs X")
        _need_cuda(X, "X")
        if X.dtype != dY.dtype or tuple(X.shape) != (N, C):
            raise ValueError(f"X must be [N, {C}] of dtype {dY.dtype}")
        dw = dw_out if dw_out is not None else torch.empty((D // n, C // n, n), dtype=torch.float32,
                                                           device=dY.device)
        _check_out(dw, "dw_out", (D // n, C // n, n), torch.float32)
        ws_bytes = int(lib.eqlin_backward_workspace_bytes(N, C, D, T, dt))
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dY.device)
        _need_cuda(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("eqlin_backward",
           lib.eqlin_backward(_ptr(dY), _ptr(X) if need_dw else None, N, C, D, T, _ptr(W_hat.buf),
                              _ptr(dX), _ptr(dw), _ptr(workspace) if need_dw else None, ws_bytes, dt,
                              _stream(dY)))
    return dX, dw


NOALLOC_SCRATCH_BYTES = 32 << 20   # EQLIN_NOALLOC_SCRATCH_BYTES


def eqlin_backward_noalloc(dY: torch.Tensor, X: Optional[torch.Tensor], W_hat: Prepared,
                           dX_out: Optional[torch.Tensor], dw_out: Optional[torch.Tensor] = None) -> None:
    """eqlin_backward without a workspace, into caller-allocated outputs: the dw
    split partials use the library's per-device static scratch (calls on one
    device must not overlap).  dX_out [N][C] (storage dtype) or None, dw_out
    [D/n][C/n][n] float32 or None.  The binding allocates nothing either."""
    lib = load_library()
    _need_cuda(dY, "dY")
    dt = _dtype_code(dY)
    if dY.dtype != W_hat.dtype:
        raise TypeError("dY and the prepared weights differ in dtype")
    C, D, T, n = W_hat.C, W_hat.D, W_hat.T, W_hat.order
    if dY.dim() != 2 or dY.shape[1] != D:
        raise ValueError(f"dY must have shape [N, {D}], got {tuple(dY.shape)}")
    N = dY.shape[0]
    if dX_out is None and dw_out is None:
        raise ValueError("nothing to compute")
    if dX_out is not None:
        _check_out(dX_out, "dX_out", (N, C), dY.dtype)
    if dw_out is not None:
        if X is None:
            raise ValueError("dw needs X")
        _need_cuda(X, "X")
        if X.dtype != dY.dtype or tuple(X.shape) != (N, C):
            raise ValueError(f"X must be [N, {C}] of dtype {dY.dtype}")
        _check_out(dw_out, "dw_out", (D // n, C // n, n), torch.float32)
    _check("eqlin_backward_noalloc",
           lib.eqlin_backward_noalloc(_ptr(dY), _ptr(X) if dw_out is not None else None, N, C, D, T,
                                      _ptr(W_hat.buf), _ptr(dX_out), _ptr(dw_out), dt, _stream(dY)))


def eqlin_backward_dx(dY: torch.Tensor, W_hat: Prepared, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX = dY W, dY [N][D] -> dX [N][C]."""
    lib = load_library()
    _need_cuda(dY, "dY")
    dt = _dtype_code(dY)
    C, D = W_hat.C, W_hat.D
    if dY.dtype != W_hat.dtype or dY.dim() != 2 or dY.shape[1] != D:
        raise ValueError(f"dY must be [N, {D}] of dtype {W_hat.dtype}")
    N = dY.shape[0]
    if out is None:
        out = torch.empty((N, C), dtype=dY.dtype, device=dY.device)
    _check_out(out, "out", (N, C), dY.dtype)
    _check("eqlin_backward_dx", lib.eqlin_backward_dx(_ptr(dY), N, C, D, W_hat.T, _ptr(W_hat.buf), _ptr(out), dt,
                                                      _stream(dY)))
    return out


def eqlin_backward_dw(dY: torch.Tensor, X: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, T=T_P4) -> torch.Tensor:
    """dw [D/n][C/n][n] (float32) from dY [N][D] and X [N][C]; T = group (4, 8, 'p4m')."""
    lib = load_library()
    _need_cuda(dY, "dY")
    _need_cuda(X, "X")
    dt = _dtype_code(dY)
    if X.dtype != dY.dtype or X.dim() != 2 or dY.dim() != 2 or X.shape[0] != dY.shape[0]:
        raise ValueError("dY [N, D] and X [N, C] must share N and dtype")
    N, C, D = X.shape[0], X.shape[1], dY.shape[1]
    T = group_code(T)
    n = group_order(T)
    if out is None:
        out = torch.empty((D // n, C // n, n), dtype=torch.float32, device=dY.device)
    _check_out(out, "out", (D // n, C // n, n), torch.float32)
    ws_bytes = int(lib.eqlin_backward_workspace_bytes(N, C, D, T, dt))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dY.device)
    _need_cuda(workspace, "workspace")
    _check("eqlin_backward_dw",
           lib.eqlin_backward_dw(_ptr(dY), _ptr(X), N, C, D, T, _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), dt, _stream(dY)))
    return out


# ------------------------------------------------------------ p4 group convolution

class ConvPrepared(NamedTuple):
    """Prepared filter spectra of a p4 group convolution (opaque byte buffer)."""
    buf: torch.Tensor
    C: int
    D: int
    K: int
    dtype: torch.dtype


def eqconv_prepared_weight_bytes(C: int, D: int, K: int, dtype: torch.dtype) -> int:
    return int(load_library().eqconv_prepared_weight_bytes(C, D, K, _DTYPES[dtype]))


def eqconv_prepare_weights(psi: torch.Tensor, out: Optional[torch.Tensor] = None) -> ConvPrepared:
    """psi [D/4][C/4][K][K][4] -> prepared spectra for eqconv_forward / eqconv_backward."""
    lib = load_library()
    _need_cuda(psi, "psi")
    dt = _dtype_code(psi)
    if psi.dim() != 5 or psi.shape[2] != psi.shape[3] or psi.shape[4] != 4:
        raise ValueError(f"psi must have shape [D/4, C/4, K, K, 4], got {tuple(psi.shape)}")
    D, C, K = 4 * psi.shape[0], 4 * psi.shape[1], int(psi.shape[2])
    nbytes = int(lib.eqconv_prepared_weight_bytes(C, D, K, dt))
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=psi.device)
    _need_cuda(out, "out")
    _check("eqconv_prepare_weights",
           lib.eqconv_prepare_weights(_ptr(psi), C, D, K, dt, _ptr(out), out.numel() * out.element_size(),
                                      _stream(psi)))
    return ConvPrepared(out, C, D, K, psi.dtype)


def eqconv_forward(X: torch.Tensor, P: ConvPrepared, bias: Optional[torch.Tensor] = None, act: str = "none",
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = act(conv(X, psi) + b), X [N][H][W][C] -> Y [N][H][W][D] (channels last, rotation fastest)."""
    lib = load_library()
    _need_cuda(X, "X")
    dt = _dtype_code(X)
    if X.dtype != P.dtype:
        raise TypeError("X and the prepared filter differ in dtype")
    if X.dim() != 4 or X.shape[3] != P.C:
        raise ValueError(f"X must have shape [N, H, W, {P.C}], got {tuple(X.shape)}")
    if act not in ACT:
        raise ValueError(f"act must be one of {sorted(ACT)}")
    if bias is not None:
        _need_cuda(bias, "bias")
        if bias.dtype != X.dtype or tuple(bias.shape) != (P.D // 4,):
            raise ValueError(f"bias must be [{P.D // 4}] of dtype {X.dtype}")
    N, H, W = X.shape[:3]
    if out is None:
        out = torch.empty((N, H, W, P.D), dtype=X.dtype, device=X.device)
    _check_out(out, "out", (N, H, W, P.D), X.dtype)
    _check("eqconv_forward", lib.eqconv_forward(_ptr(X), N, H, W, P.C, P.D, P.K, _ptr(P.buf), _ptr(bias), ACT[act],
                                                _ptr(out), dt, _stream(X)))
    return out


def eqconv_backward_workspace_bytes(N: int, H: int, W: int, C: int, D: int, K: int, dtype: torch.dtype) -> int:
    return int(load_library().eqconv_backward_workspace_bytes(N, H, W, C, D, K, _DTYPES[dtype]))


def eqconv_backward(dY: torch.Tensor, X: Optional[torch.Tensor], P: ConvPrepared, need_dx: bool = True,
                    need_dpsi: bool = True, workspace: Optional[torch.Tensor] = None):
    """(dX [N][H][W][C] or None, dpsi [D/4][C/4][K][K][4] float32 or None) for dY [N][H][W][D]."""
    lib = load_library()
    _need_cuda(dY, "dY")
    dt = _dtype_code(dY)
    if dY.dtype != P.dtype:
        raise TypeError("dY and the prepared filter differ in dtype")
    if dY.dim() != 4 or dY.shape[3] != P.D:
        raise ValueError(f"dY must have shape [N, H, W, {P.D}], got {tuple(dY.shape)}")
    if not (need_dx or need_dpsi):
        raise ValueError("nothing to compute")
    N, H, W = dY.shape[:3]
    dX = dpsi = None
    ws_bytes = 0
    if need_dx:
        dX = torch.empty((N, H, W, P.C), dtype=dY.dtype, device=dY.device)
    if need_dpsi:
        if X is None:
            raise ValueError("dpsi needs X")
        _need_cuda(X, "X")
        if X.dtype != dY.dtype or tuple(X.shape) != (N, H, W, P.C):
            raise ValueError(f"X must be [N, H, W, {P.C}] of dtype {dY.dtype}")
        dpsi = torch.empty((P.D // 4, P.C // 4, P.K, P.K, 4), dtype=torch.float32, device=dY.device)
        ws_bytes = int(lib.eqconv_backward_workspace_bytes(N, H, W, P.C, P.D, P.K, dt))
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dY.device)
        _need_cuda(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("eqconv_backward",
           lib.eqconv_backward(_ptr(dY), _ptr(X) if need_dpsi else None, N, H, W, P.C, P.D, P.K, _ptr(P.buf),
                               _ptr(dX), _ptr(dpsi), _ptr(workspace) if need_dpsi else None, ws_bytes, dt,
                               _stream(dY)))
    return dX, dpsi
