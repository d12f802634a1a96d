"""MI355X (gfx950) SwiGLU MLP training step: Python binding of libswiglu_mlp.so.

Every function here only marshals arguments (torch tensors -> device
pointers, the current HIP stream) and calls the C ABI declared in
``include/swiglu_mlp.h``; all arithmetic runs in the HIP kernels.  There is
no CPU fallback: importing fails loudly when the library is not built, and
calls fail loudly on tensors that are not bf16 on a GPU.

Layouts (the note "SwiGLU MLP forward principle, backward chain and
optimisation", section 1): x [M,D], W1 [D,2I] with columns [0,I) the
un-gated "left" branch and [I,2I) the gate, W_down [I,Dout].
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
import re

import torch

__all__ = [
    "SwiGLUError", "lib", "LIB_PATH", "HEADER_PATH", "exported_names",
    "swiglu_mlp_fwd", "swiglu_mlp_bwd", "swiglu_mlp_bwd_unfused",
    "swiglu_mlp_fwd_noalloc", "swiglu_mlp_fwd_noalloc_limit",
    "swiglu_mlp_fwd_workspace", "swiglu_mlp_bwd_workspace", "swiglu_mlp_bwd_unfused_workspace",
    "swiglu_fwd_gemm1", "swiglu_fwd_down", "swiglu_bwd_dgrad_fused", "swiglu_bwd_dgrad_plain",
    "swiglu_bwd_elementwise", "swiglu_bwd_dw_down", "swiglu_bwd_dx", "swiglu_bwd_dw1",
    "swiglu_act_eval", "SwiGLUMLPFunction", "swiglu_mlp",
    "swiglu_mlp_fwd_save_h", "swiglu_mlp_bwd_saved_h_workspace", "swiglu_mlp_bwd_saved_h",
    "swiglu_bwd_dgrad_fused_gp", "SwiGLUMLPSaveHFunction", "swiglu_mlp_save_h",
    "swiglu_mlp_fwd_residual", "swiglu_mlp_bwd_residual", "swiglu_fwd_down_residual",
    "swiglu_bwd_dx_residual", "SwiGLUResidualMLPFunction", "swiglu_mlp_residual",
    "swiglu_mlp_stack",
    "swiglu_moe_fwd_workspace", "swiglu_moe_bwd_workspace", "swiglu_moe_fwd", "swiglu_moe_bwd",
    "swiglu_moe_bwd_dgrad_fused", "SwiGLUMoEFunction", "swiglu_moe",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswiglu_mlp.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "swiglu_mlp.h")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "swiglu_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "swiglu_abi_version": (ctypes.c_int, []),
    "swiglu_mlp_fwd_workspace": (_SZ, [_I64] * 4),
    "swiglu_mlp_bwd_workspace": (_SZ, [_I64] * 4),
    "swiglu_mlp_bwd_unfused_workspace": (_SZ, [_I64] * 4),
    "swiglu_mlp_fwd": (ctypes.c_int, [_P] * 5 + [_P, _SZ] + [_I64] * 4 + [_P]),
    "swiglu_mlp_fwd_noalloc_limit": (_SZ, []),
    "swiglu_mlp_fwd_noalloc": (ctypes.c_int, [_P] * 5 + [_I64] * 4 + [_P]),
    "swiglu_mlp_bwd": (ctypes.c_int, [_P] * 8 + [_P, _SZ] + [_I64] * 4 + [_P]),
    "swiglu_mlp_bwd_unfused": (ctypes.c_int, [_P] * 8 + [_P, _SZ] + [_I64] * 4 + [_P]),
    "swiglu_fwd_gemm1": (ctypes.c_int, [_P] * 4 + [_I64] * 3 + [_P]),
    "swiglu_fwd_down": (ctypes.c_int, [_P] * 3 + [_I64] * 3 + [_P]),
    "swiglu_bwd_dgrad_fused": (ctypes.c_int, [_P] * 5 + [_I64] * 3 + [_P]),
    "swiglu_bwd_dgrad_plain": (ctypes.c_int, [_P] * 3 + [_I64] * 3 + [_P]),
    "swiglu_bwd_elementwise": (ctypes.c_int, [_P] * 4 + [_I64] * 2 + [_P]),
    "swiglu_bwd_dw_down": (ctypes.c_int, [_P] * 3 + [_I64] * 3 + [_P]),
    "swiglu_bwd_dx": (ctypes.c_int, [_P] * 3 + [_I64] * 3 + [_P]),
    "swiglu_bwd_dw1": (ctypes.c_int, [_P] * 3 + [_I64] * 3 + [_P]),
    "swiglu_act_eval": (ctypes.c_int, [_P] * 4 + [_I64] + [_P]),
    "swiglu_mlp_fwd_save_h": (ctypes.c_int, [_P] * 6 + [_I64] * 4 + [_P]),
    "swiglu_mlp_bwd_saved_h_workspace": (_SZ, [_I64] * 4),
    "swiglu_mlp_bwd_saved_h": (ctypes.c_int, [_P] * 9 + [_P, _SZ] + [_I64] * 4 + [_P]),
    "swiglu_bwd_dgrad_fused_gp": (ctypes.c_int, [_P] * 4 + [_I64] * 3 + [_P]),
    "swiglu_mlp_fwd_residual": (ctypes.c_int, [_P] * 5 + [_P, _SZ] + [_I64] * 4 + [_P]),
    "swiglu_mlp_bwd_residual": (ctypes.c_int, [_P] * 8 + [_P, _SZ] + [_I64] * 4 + [_P]),
    "swiglu_fwd_down_residual": (ctypes.c_int, [_P] * 4 + [_I64] * 3 + [_P]),
    "swiglu_bwd_dx_residual": (ctypes.c_int, [_P] * 4 + [_I64] * 3 + [_P]),
    "swiglu_moe_fwd_workspace": (_SZ, [_I64] * 5),
    "swiglu_moe_bwd_workspace": (_SZ, [_I64] * 5),
    "swiglu_moe_fwd": (ctypes.c_int, [_P] * 6 + [_P, _SZ] + [_I64] * 5 + [_P]),
    "swiglu_moe_bwd": (ctypes.c_int, [_P] * 9 + [_P, _SZ] + [_I64] * 5 + [_P]),
    "swiglu_moe_bwd_dgrad_fused": (ctypes.c_int, [_P] * 6 + [_I64] * 4 + [_P]),
}


class SwiGLUError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().swiglu_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m bwd_gemm_epilogue_amd.build` "
                "(there is no CPU fallback)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def exported_names():
    """Function names declared in include/swiglu_mlp.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swiglu_[a-z0-9_]+)\s*\(", text)))


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _check(fn: str, status: int):
    if status != 0:
        raise SwiGLUError(fn, status)


def _on_device(t: torch.Tensor, name: str):
    """t must be a contiguous tensor on the GPU the call launches on (the
    current device inside a call, set from its first tensor)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (no CPU path)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, the call runs on cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _dev(t: torch.Tensor, name: str, shape=None) -> int:
    _on_device(t, name)
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    """The HIP stream handle of a call (inside a _launches call `stream` is
    already the torch stream the call runs on)."""
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _launches(fn):
    """Run a launching call with its first tensor's device current and the
    launch stream as torch's current stream.  Every tensor the call
    allocates (outputs, a temporary workspace) then belongs to that stream in
    the caching allocator, so a temporary freed on return is not handed to
    other work before the launched kernels are done with it.  `stream` may
    be a torch stream or a raw HIP stream handle (wrapped as an external
    stream)."""
    params = list(inspect.signature(fn).parameters)
    at = params.index("stream")

    @functools.wraps(fn)
    def call(*args, **kw):
        if len(args) > at:
            kw["stream"] = args[at]
            args = args[:at]
        like = args[0] if args else None
        if not isinstance(like, torch.Tensor) or not like.is_cuda:
            raise ValueError(f"{fn.__name__}: the first argument must be a tensor on a GPU (no CPU path)")
        stream = kw.get("stream")
        if stream is None:
            st = torch.cuda.current_stream(like.device)
        elif isinstance(stream, torch.cuda.Stream):
            st = stream
        else:
            st = torch.cuda.ExternalStream(int(stream), device=like.device)
        if st.device != like.device:
            raise ValueError(f"{fn.__name__}: the stream is on {st.device}, the tensors on {like.device}")
        kw["stream"] = st
        with torch.cuda.device(like.device), torch.cuda.stream(st):
            return fn(*args, **kw)

    return call


def _empty(shape, like: torch.Tensor):
    return torch.empty(shape, dtype=torch.bfloat16, device=like.device)


def _ws(nbytes: int, like: torch.Tensor, ws):
    if ws is None:
        ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)
    _on_device(ws, "workspace")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel() * ws.element_size()} < {nbytes}")
    return ws


def _dims_fwd(x, W1, W_down):
    M, D = x.shape
    D2, I2 = W1.shape
    I, Dout = W_down.shape
    if D2 != D or I2 != 2 * I:
        raise ValueError(f"inconsistent shapes x{tuple(x.shape)} W1{tuple(W1.shape)} W_down{tuple(W_down.shape)}")
    return M, D, I, Dout


@_launches
def swiglu_mlp_fwd_save_h(x, W1, W_down, preact=None, h=None, y=None, stream=None):
    """Save-h forward: returns (preact [M,2I], h [M,I], y [M,Dout]); h is kept."""
    M, D, I, Dout = _dims_fwd(x, W1, W_down)
    preact = _empty((M, 2 * I), x) if preact is None else preact
    h = _empty((M, I), x) if h is None else h
    y = _empty((M, Dout), x) if y is None else y
    _check("swiglu_mlp_fwd_save_h", lib().swiglu_mlp_fwd_save_h(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"), _dev(preact, "preact", (M, 2 * I)),
        _dev(h, "h", (M, I)), _dev(y, "y", (M, Dout)), M, D, I, Dout, _stream(x, stream)))
    return preact, h, y


def swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout) -> int:
    return lib().swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout)


@_launches
def swiglu_mlp_bwd_saved_h(x, W1, W_down, preact, h, dy, dx=None, dW1=None, dW_down=None, ws=None,
                           stream=None):
    """Backward from the save-h saved set {x, W1, W_down, preact, h}: (dx, dW1, dW_down)."""
    M, D, I, Dout = _dims_fwd(x, W1, W_down)
    dx = _empty((M, D), x) if dx is None else dx
    dW1 = _empty((D, 2 * I), x) if dW1 is None else dW1
    dW_down = _empty((I, Dout), x) if dW_down is None else dW_down
    ws = _ws(swiglu_mlp_bwd_saved_h_workspace(M, D, I, Dout), x, ws)
    _check("swiglu_mlp_bwd_saved_h", lib().swiglu_mlp_bwd_saved_h(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"), _dev(preact, "preact", (M, 2 * I)),
        _dev(h, "h", (M, I)), _dev(dy, "dy", (M, Dout)), _dev(dx, "dx", (M, D)), _dev(dW1, "dW1", (D, 2 * I)),
        _dev(dW_down, "dW_down", (I, Dout)), ws.data_ptr(), ws.numel() * ws.element_size(),
        M, D, I, Dout, _stream(x, stream)))
    return dx, dW1, dW_down


# --------------------------------------------------------------------------
# whole step
# --------------------------------------------------------------------------

def swiglu_mlp_fwd_workspace(M, D, I, Dout) -> int:
    return lib().swiglu_mlp_fwd_workspace(M, D, I, Dout)


def swiglu_mlp_bwd_workspace(M, D, I, Dout) -> int:
    return lib().swiglu_mlp_bwd_workspace(M, D, I, Dout)


def swiglu_mlp_bwd_unfused_workspace(M, D, I, Dout) -> int:
    return lib().swiglu_mlp_bwd_unfused_workspace(M, D, I, Dout)


def _fwd(fn, x, W1, W_down, preact, y, ws, stream):
    M, D, I, Dout = _dims_fwd(x, W1, W_down)
    preact = _empty((M, 2 * I), x) if preact is None else preact
    y = _empty((M, Dout), x) if y is None else y
    ws = _ws(swiglu_mlp_fwd_workspace(M, D, I, Dout), x, ws)
    _check(fn, getattr(lib(), fn)(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"),
        _dev(preact, "preact", (M, 2 * I)), _dev(y, "y", (M, Dout)),
        ws.data_ptr(), ws.numel() * ws.element_size(), M, D, I, Dout, _stream(x, stream)))
    return preact, y


@_launches
def swiglu_mlp_fwd(x, W1, W_down, preact=None, y=None, ws=None, stream=None):
    """Returns (preact [M,2I], y [M,Dout]); h lives only in the workspace."""
    return _fwd("swiglu_mlp_fwd", x, W1, W_down, preact, y, ws, stream)


def swiglu_mlp_fwd_noalloc_limit() -> int:
    """Bytes of the library's static workspace used by swiglu_mlp_fwd_noalloc."""
    return lib().swiglu_mlp_fwd_noalloc_limit()


@_launches
def swiglu_mlp_fwd_noalloc(x, W1, W_down, preact=None, y=None, stream=None):
    """swiglu_mlp_fwd without a workspace argument: the library's own static
    device array holds h and the partial sums, so the C call allocates
    nothing (outputs are allocated here only when not given).  Refuses
    shapes whose workspace exceeds swiglu_mlp_fwd_noalloc_limit()."""
    M, D, I, Dout = _dims_fwd(x, W1, W_down)
    preact = _empty((M, 2 * I), x) if preact is None else preact
    y = _empty((M, Dout), x) if y is None else y
    _check("swiglu_mlp_fwd_noalloc", lib().swiglu_mlp_fwd_noalloc(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"),
        _dev(preact, "preact", (M, 2 * I)), _dev(y, "y", (M, Dout)), M, D, I, Dout, _stream(x, stream)))
    return preact, y


@_launches
def swiglu_mlp_fwd_residual(x, W1, W_down, preact=None, y=None, ws=None, stream=None):
    """Residual block: returns (preact [M,2I], y = x + MLP(x) [M,D]); needs Dout == D."""
    return _fwd("swiglu_mlp_fwd_residual", x, W1, W_down, preact, y, ws, stream)


def _bwd(fn, wsfn, x, W1, W_down, preact, dy, dx, dW1, dW_down, ws, stream):
    M, D, I, Dout = _dims_fwd(x, W1, W_down)
    dx = _empty((M, D), x) if dx is None else dx
    dW1 = _empty((D, 2 * I), x) if dW1 is None else dW1
    dW_down = _empty((I, Dout), x) if dW_down is None else dW_down
    ws = _ws(wsfn(M, D, I, Dout), x, ws)
    _check(fn, getattr(lib(), fn)(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"), _dev(preact, "preact", (M, 2 * I)),
        _dev(dy, "dy", (M, Dout)), _dev(dx, "dx", (M, D)), _dev(dW1, "dW1", (D, 2 * I)),
        _dev(dW_down, "dW_down", (I, Dout)), ws.data_ptr(), ws.numel() * ws.element_size(),
        M, D, I, Dout, _stream(x, stream)))
    return dx, dW1, dW_down


@_launches
def swiglu_mlp_bwd(x, W1, W_down, preact, dy, dx=None, dW1=None, dW_down=None, ws=None, stream=None):
    """Fused backward from the saved set {x, W1, W_down, preact}: (dx, dW1, dW_down)."""
    return _bwd("swiglu_mlp_bwd", swiglu_mlp_bwd_workspace, x, W1, W_down, preact, dy,
                dx, dW1, dW_down, ws, stream)


@_launches
def swiglu_mlp_bwd_residual(x, W1, W_down, preact, dy, dx=None, dW1=None, dW_down=None, ws=None,
                            stream=None):
    """Backward of the residual block: dx includes dy; dW1, dW_down as swiglu_mlp_bwd."""
    return _bwd("swiglu_mlp_bwd_residual", swiglu_mlp_bwd_workspace, x, W1, W_down, preact, dy,
                dx, dW1, dW_down, ws, stream)


@_launches
def swiglu_mlp_bwd_unfused(x, W1, W_down, preact, dy, dx=None, dW1=None, dW_down=None, ws=None,
                           stream=None):
    """Unfused baseline backward (dout materialised): (dx, dW1, dW_down)."""
    return _bwd("swiglu_mlp_bwd_unfused", swiglu_mlp_bwd_unfused_workspace, x, W1, W_down, preact, dy,
                dx, dW1, dW_down, ws, stream)


# --------------------------------------------------------------------------
# single steps
# --------------------------------------------------------------------------

@_launches
def swiglu_fwd_gemm1(x, W1, preact=None, h=None, stream=None):
    M, D = x.shape
    I = W1.shape[1] // 2
    preact = _empty((M, 2 * I), x) if preact is None else preact
    h = _empty((M, I), x) if h is None else h
    _check("swiglu_fwd_gemm1", lib().swiglu_fwd_gemm1(
        _dev(x, "x"), _dev(W1, "W1", (D, 2 * I)), _dev(preact, "preact", (M, 2 * I)),
        _dev(h, "h", (M, I)), M, D, I, _stream(x, stream)))
    return preact, h


@_launches
def swiglu_fwd_down(h, W_down, y=None, stream=None):
    M, I = h.shape
    Dout = W_down.shape[1]
    y = _empty((M, Dout), h) if y is None else y
    _check("swiglu_fwd_down", lib().swiglu_fwd_down(
        _dev(h, "h"), _dev(W_down, "W_down", (I, Dout)), _dev(y, "y", (M, Dout)), M, I, Dout,
        _stream(h, stream)))
    return y


@_launches
def swiglu_fwd_down_residual(h, W_down, x, y=None, stream=None):
    """y = h.W_down + x with the add in the GEMM epilogue."""
    M, I = h.shape
    D = W_down.shape[1]
    y = _empty((M, D), h) if y is None else y
    _check("swiglu_fwd_down_residual", lib().swiglu_fwd_down_residual(
        _dev(h, "h"), _dev(W_down, "W_down", (I, D)), _dev(x, "x", (M, D)), _dev(y, "y", (M, D)), M, I, D,
        _stream(h, stream)))
    return y


@_launches
def swiglu_bwd_dgrad_fused(dy, W_down, preact, grad_preact=None, h=None, stream=None):
    M, Dout = dy.shape
    I = W_down.shape[0]
    grad_preact = _empty((M, 2 * I), dy) if grad_preact is None else grad_preact
    h = _empty((M, I), dy) if h is None else h
    _check("swiglu_bwd_dgrad_fused", lib().swiglu_bwd_dgrad_fused(
        _dev(dy, "dy"), _dev(W_down, "W_down", (I, Dout)), _dev(preact, "preact", (M, 2 * I)),
        _dev(grad_preact, "grad_preact", (M, 2 * I)), _dev(h, "h", (M, I)), M, I, Dout,
        _stream(dy, stream)))
    return grad_preact, h


@_launches
def swiglu_bwd_dgrad_fused_gp(dy, W_down, preact, grad_preact=None, stream=None):
    """The save-h path's fused dgrad: grad_preact only."""
    M, Dout = dy.shape
    I = W_down.shape[0]
    grad_preact = _empty((M, 2 * I), dy) if grad_preact is None else grad_preact
    _check("swiglu_bwd_dgrad_fused_gp", lib().swiglu_bwd_dgrad_fused_gp(
        _dev(dy, "dy"), _dev(W_down, "W_down", (I, Dout)), _dev(preact, "preact", (M, 2 * I)),
        _dev(grad_preact, "grad_preact", (M, 2 * I)), M, I, Dout, _stream(dy, stream)))
    return grad_preact


@_launches
def swiglu_bwd_dgrad_plain(dy, W_down, dout=None, stream=None):
    M, Dout = dy.shape
    I = W_down.shape[0]
    dout = _empty((M, I), dy) if dout is None else dout
    _check("swiglu_bwd_dgrad_plain", lib().swiglu_bwd_dgrad_plain(
        _dev(dy, "dy"), _dev(W_down, "W_down", (I, Dout)), _dev(dout, "dout", (M, I)), M, I, Dout,
        _stream(dy, stream)))
    return dout


@_launches
def swiglu_bwd_elementwise(preact, dout, grad_preact=None, h=None, stream=None):
    M, I = dout.shape
    grad_preact = _empty((M, 2 * I), dout) if grad_preact is None else grad_preact
    h = _empty((M, I), dout) if h is None else h
    _check("swiglu_bwd_elementwise", lib().swiglu_bwd_elementwise(
        _dev(preact, "preact", (M, 2 * I)), _dev(dout, "dout"), _dev(grad_preact, "grad_preact", (M, 2 * I)),
        _dev(h, "h", (M, I)), M, I, _stream(dout, stream)))
    return grad_preact, h


@_launches
def swiglu_bwd_dw_down(h, dy, dW_down=None, stream=None):
    M, I = h.shape
    Dout = dy.shape[1]
    dW_down = _empty((I, Dout), h) if dW_down is None else dW_down
    _check("swiglu_bwd_dw_down", lib().swiglu_bwd_dw_down(
        _dev(h, "h"), _dev(dy, "dy", (M, Dout)), _dev(dW_down, "dW_down", (I, Dout)), M, I, Dout,
        _stream(h, stream)))
    return dW_down


@_launches
def swiglu_bwd_dx(grad_preact, W1, dx=None, stream=None):
    M, I2 = grad_preact.shape
    D = W1.shape[0]
    dx = _empty((M, D), grad_preact) if dx is None else dx
    _check("swiglu_bwd_dx", lib().swiglu_bwd_dx(
        _dev(grad_preact, "grad_preact"), _dev(W1, "W1", (D, I2)), _dev(dx, "dx", (M, D)), M, D, I2 // 2,
        _stream(grad_preact, stream)))
    return dx


@_launches
def swiglu_bwd_dx_residual(grad_preact, W1, dy, dx=None, stream=None):
    """dx = grad_preact.W1^T + dy with the add in the GEMM epilogue."""
    M, I2 = grad_preact.shape
    D = W1.shape[0]
    dx = _empty((M, D), grad_preact) if dx is None else dx
    _check("swiglu_bwd_dx_residual", lib().swiglu_bwd_dx_residual(
        _dev(grad_preact, "grad_preact"), _dev(W1, "W1", (D, I2)), _dev(dy, "dy", (M, D)),
        _dev(dx, "dx", (M, D)), M, D, I2 // 2, _stream(grad_preact, stream)))
    return dx


@_launches
def swiglu_bwd_dw1(x, grad_preact, dW1=None, stream=None):
    M, D = x.shape
    I2 = grad_preact.shape[1]
    dW1 = _empty((D, I2), x) if dW1 is None else dW1
    _check("swiglu_bwd_dw1", lib().swiglu_bwd_dw1(
        _dev(x, "x"), _dev(grad_preact, "grad_preact", (M, I2)), _dev(dW1, "dW1", (D, I2)), M, D, I2 // 2,
        _stream(x, stream)))
    return dW1


@_launches
def swiglu_act_eval(g, stream=None):
    """sigma, silu, silu' of bf16 g (any shape) as float32 tensors."""
    g = g.contiguous()
    _dev(g, "g")
    n = g.numel()
    outs = [torch.empty(g.shape, dtype=torch.float32, device=g.device) for _ in range(3)]
    _check("swiglu_act_eval", lib().swiglu_act_eval(
        g.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), n, _stream(g, stream)))
    return tuple(outs)


# --------------------------------------------------------------------------
# autograd
# --------------------------------------------------------------------------

class SwiGLUMLPFunction(torch.autograd.Function):
    """y = (left * silu(gate)) @ W_down with [left | gate] = x @ W1.

    Saves exactly {x, W1, W_down, preact} (the drop-h report's saved set);
    h is recomputed in the backward's fused dgrad epilogue."""

    @staticmethod
    def forward(ctx, x, W1, W_down):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        preact, y = swiglu_mlp_fwd(x2, W1.contiguous(), W_down.contiguous())
        ctx.save_for_backward(x2, W1, W_down, preact)
        ctx.lead = lead
        return y.reshape(*lead, y.shape[-1])

    @staticmethod
    def backward(ctx, grad_y):
        x2, W1, W_down, preact = ctx.saved_tensors
        dy = grad_y.reshape(-1, grad_y.shape[-1]).contiguous()
        dx, dW1, dW_down = swiglu_mlp_bwd(x2, W1.contiguous(), W_down.contiguous(), preact, dy)
        return dx.reshape(*ctx.lead, dx.shape[-1]), dW1, dW_down


def swiglu_mlp(x, W1, W_down):
    return SwiGLUMLPFunction.apply(x, W1, W_down)


class SwiGLUMLPSaveHFunction(torch.autograd.Function):
    """The drop-h report's fallback path (normal MLPBlock): the same y, but
    the saved set is {x, W1, W_down, preact, h} and the backward does not
    recompute h."""

    @staticmethod
    def forward(ctx, x, W1, W_down):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        preact, h, y = swiglu_mlp_fwd_save_h(x2, W1.contiguous(), W_down.contiguous())
        ctx.save_for_backward(x2, W1, W_down, preact, h)
        ctx.lead = lead
        return y.reshape(*lead, y.shape[-1])

    @staticmethod
    def backward(ctx, grad_y):
        x2, W1, W_down, preact, h = ctx.saved_tensors
        dy = grad_y.reshape(-1, grad_y.shape[-1]).contiguous()
        dx, dW1, dW_down = swiglu_mlp_bwd_saved_h(x2, W1.contiguous(), W_down.contiguous(), preact, h, dy)
        return dx.reshape(*ctx.lead, dx.shape[-1]), dW1, dW_down


def swiglu_mlp_save_h(x, W1, W_down):
    return SwiGLUMLPSaveHFunction.apply(x, W1, W_down)


class SwiGLUResidualMLPFunction(torch.autograd.Function):
    """Residual block y = x + (left * silu(gate)) @ W_down (Lesson 24,
    section 24): the add is fused into the down GEMM's epilogue and, in the
    backward, dy joins dx in the dx GEMM's epilogue.  Saved set as
    SwiGLUMLPFunction."""

    @staticmethod
    def forward(ctx, x, W1, W_down):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        preact, y = swiglu_mlp_fwd_residual(x2, W1.contiguous(), W_down.contiguous())
        ctx.save_for_backward(x2, W1, W_down, preact)
        ctx.lead = lead
        return y.reshape(*lead, y.shape[-1])

    @staticmethod
    def backward(ctx, grad_y):
        x2, W1, W_down, preact = ctx.saved_tensors
        dy = grad_y.reshape(-1, grad_y.shape[-1]).contiguous()
        dx, dW1, dW_down = swiglu_mlp_bwd_residual(x2, W1.contiguous(), W_down.contiguous(), preact, dy)
        return dx.reshape(*ctx.lead, dx.shape[-1]), dW1, dW_down


def swiglu_mlp_residual(x, W1, W_down):
    return SwiGLUResidualMLPFunction.apply(x, W1, W_down)


def swiglu_mlp_stack(x, layers, save_h=False):
    """A stack of MLP blocks applied in order (the drop-h report's 4-layer
    stack): x_{l+1} = MLP_l(x_l) for layers = [(W1_l, W_down_l), ...], each
    with Dout == D.  Every block is its own autograd node, so each keeps its
    own saved set: {x_l, W1_l, W_down_l, preact_l}, plus h_l with save_h."""
    fn = swiglu_mlp_save_h if save_h else swiglu_mlp
    for W1, W_down in layers:
        if W_down.shape[1] != x.shape[-1]:
            raise ValueError("a stack of blocks needs Dout == D in every layer")
        x = fn(x, W1, W_down)
    return x


# --------------------------------------------------------------------------
# mixture-of-experts blocks (grouped GEMMs over expert-packed rows)
# --------------------------------------------------------------------------

def _offsets(off, E: int) -> int:
    _on_device(off, "group_offsets")
    if off.dtype != torch.int32:
        raise ValueError("group_offsets must be a contiguous int32 tensor on the GPU")
    if tuple(off.shape) != (E + 1,):
        raise ValueError(f"group_offsets has shape {tuple(off.shape)}, expected ({E + 1},)")
    return off.data_ptr()


def _dims_moe(x, W1, W_down):
    M, D = x.shape
    E, D2, I2 = W1.shape
    E2, I, Dout = W_down.shape
    if D2 != D or I2 != 2 * I or E2 != E:
        raise ValueError(f"inconsistent shapes x{tuple(x.shape)} W1{tuple(W1.shape)} W_down{tuple(W_down.shape)}")
    return M, D, I, Dout, E


def swiglu_moe_fwd_workspace(M, D, I, Dout, E) -> int:
    return lib().swiglu_moe_fwd_workspace(M, D, I, Dout, E)


def swiglu_moe_bwd_workspace(M, D, I, Dout, E) -> int:
    return lib().swiglu_moe_bwd_workspace(M, D, I, Dout, E)


@_launches
def swiglu_moe_fwd(x, W1, W_down, group_offsets, preact=None, y=None, ws=None, stream=None):
    """Expert MLPs over expert-packed rows: x [M,D], W1 [E,D,2I], W_down
    [E,I,Dout], group_offsets int32 [E+1] on the GPU.  Returns (preact, y)."""
    M, D, I, Dout, E = _dims_moe(x, W1, W_down)
    preact = _empty((M, 2 * I), x) if preact is None else preact
    y = _empty((M, Dout), x) if y is None else y
    ws = _ws(swiglu_moe_fwd_workspace(M, D, I, Dout, E), x, ws)
    _check("swiglu_moe_fwd", lib().swiglu_moe_fwd(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"), _offsets(group_offsets, E),
        _dev(preact, "preact", (M, 2 * I)), _dev(y, "y", (M, Dout)),
        ws.data_ptr(), ws.numel() * ws.element_size(), M, D, I, Dout, E, _stream(x, stream)))
    return preact, y


@_launches
def swiglu_moe_bwd(x, W1, W_down, group_offsets, preact, dy, dx=None, dW1=None, dW_down=None, ws=None,
                   stream=None):
    """Backward of swiglu_moe_fwd: (dx [M,D], dW1 [E,D,2I], dW_down [E,I,Dout])."""
    M, D, I, Dout, E = _dims_moe(x, W1, W_down)
    dx = _empty((M, D), x) if dx is None else dx
    dW1 = _empty((E, D, 2 * I), x) if dW1 is None else dW1
    dW_down = _empty((E, I, Dout), x) if dW_down is None else dW_down
    ws = _ws(swiglu_moe_bwd_workspace(M, D, I, Dout, E), x, ws)
    _check("swiglu_moe_bwd", lib().swiglu_moe_bwd(
        _dev(x, "x"), _dev(W1, "W1"), _dev(W_down, "W_down"), _offsets(group_offsets, E),
        _dev(preact, "preact", (M, 2 * I)), _dev(dy, "dy", (M, Dout)), _dev(dx, "dx", (M, D)),
        _dev(dW1, "dW1", (E, D, 2 * I)), _dev(dW_down, "dW_down", (E, I, Dout)),
        ws.data_ptr(), ws.numel() * ws.element_size(), M, D, I, Dout, E, _stream(x, stream)))
    return dx, dW1, dW_down


@_launches
def swiglu_moe_bwd_dgrad_fused(dy, W_down, group_offsets, preact, grad_preact=None, h=None, stream=None):
    """The grouped fused dgrad step alone: (grad_preact [M,2I], h [M,I])."""
    M, Dout = dy.shape
    E, I, _ = W_down.shape
    grad_preact = _empty((M, 2 * I), dy) if grad_preact is None else grad_preact
    h = _empty((M, I), dy) if h is None else h
    _check("swiglu_moe_bwd_dgrad_fused", lib().swiglu_moe_bwd_dgrad_fused(
        _dev(dy, "dy"), _dev(W_down, "W_down", (E, I, Dout)), _offsets(group_offsets, E),
        _dev(preact, "preact", (M, 2 * I)), _dev(grad_preact, "grad_preact", (M, 2 * I)), _dev(h, "h", (M, I)),
        M, I, Dout, E, _stream(dy, stream)))
    return grad_preact, h


class SwiGLUMoEFunction(torch.autograd.Function):
    """Expert SwiGLU MLPs over expert-packed rows (Lesson 24, sections
    41-42).  Saves {x, W1, W_down, group_offsets, preact}; h is recomputed in
    the grouped fused dgrad's epilogue."""

    @staticmethod
    def forward(ctx, x, W1, W_down, group_offsets):
        preact, y = swiglu_moe_fwd(x.contiguous(), W1.contiguous(), W_down.contiguous(), group_offsets)
        ctx.save_for_backward(x, W1, W_down, group_offsets, preact)
        return y

    @staticmethod
    def backward(ctx, grad_y):
        x, W1, W_down, off, preact = ctx.saved_tensors
        dx, dW1, dW_down = swiglu_moe_bwd(x.contiguous(), W1.contiguous(), W_down.contiguous(), off, preact,
                                          grad_y.contiguous())
        return dx, dW1, dW_down, None


def swiglu_moe(x, W1, W_down, group_offsets):
    return SwiGLUMoEFunction.apply(x, W1, W_down, group_offsets)
