"""ctypes binding of libxfa.so.

Argument marshalling only: every step of the attention runs in the HIP
kernels of the library.  PyTorch supplies device memory and the current
stream.  If the library is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxfa.so")

XFA_DTYPE_F32 = 0
XFA_DTYPE_BF16 = 1
XFA_OK = 0
XFA_ERR_INVALID_ARGUMENT = 1
XFA_ERR_UNSUPPORTED = 2
XFA_ERR_HIP = 3

# exported symbols and their C signatures (mirrors include/xfa.h)
_c_void_p, _i64, _f32, _int, _u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_uint64
_SIGS = {
    "xfa_fwd": (_int, [_c_void_p] * 5 + [_i64] * 4 + [_f32, _int, _int, _c_void_p]),
    "xfa_bwd_preprocess": (_int, [_c_void_p] * 3 + [_i64] * 4 + [_f32, _int, _int, _c_void_p]),
    "xfa_bwd": (_int, [_c_void_p] * 10 + [_i64] * 4 + [_f32, _int, _int, _c_void_p]),
    "xfa_fwd_dropout": (_int, [_c_void_p] * 5 + [_i64] * 4 + [_f32, _int, _f32, _u64, _int, _c_void_p]),
    "xfa_bwd_dropout": (_int, [_c_void_p] * 10 + [_i64] * 4 + [_f32, _int, _f32, _u64, _int, _c_void_p]),
    "xfa_bwd_workspace_bytes": (ctypes.c_size_t, [_i64] * 4 + [_int]),
    "xfa_status_string": (ctypes.c_char_p, [_int]),
}

_lib = None


class XfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {xfa_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libxfa.so not built ({LIB_PATH}); run "
                               "`python -m transformer_attention_xfa_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def xfa_status_string(status: int) -> str:
    return lib().xfa_status_string(int(status)).decode()


# ---------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return XFA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return XFA_DTYPE_BF16
    raise TypeError(f"xfa supports float32 and bfloat16 tensors, got {t.dtype}")


def _check_same(ref, *ts, shape=None, dtype=None, names=()):
    for t, n in zip(ts, names):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if t.device != ref.device:
            raise ValueError(f"{n} is on {t.device}, expected {ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{n} has dtype {t.dtype}, expected {dtype}")


def _stream_handle(stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _scale(scale, hd) -> float:
    return 1.0 / math.sqrt(hd) if scale is None else float(scale)


def _seed(seed) -> int:
    return int(seed) & 0xFFFFFFFFFFFFFFFF


def _raise(st: int, where: str):
    if st != XFA_OK:
        raise XfaError(st, where)


def xfa_bwd_workspace_bytes(B: int, H: int, S: int, hd: int, dtype_code: int) -> int:
    """Bytes of device workspace the backward needs for this shape (0 in this build)."""
    return int(lib().xfa_bwd_workspace_bytes(B, H, S, hd, int(dtype_code)))


def _workspace_ptr(q, workspace, where: str):
    """Device address of the caller's workspace, checked against the size the
    library asks for; None (NULL) when it asks for none."""
    B, H, S, hd = q.shape
    need = xfa_bwd_workspace_bytes(B, H, S, hd, _dtype_code(q))
    if need == 0:
        return None
    if workspace is None:
        raise ValueError(f"{where}: needs a device workspace of {need} bytes (xfa_bwd_workspace_bytes)")
    if not workspace.is_cuda or workspace.device != q.device:
        raise ValueError(f"{where}: workspace must be on {q.device}")
    if workspace.numel() * workspace.element_size() < need or workspace.data_ptr() % 256:
        raise ValueError(f"{where}: workspace must hold {need} bytes, 256-byte aligned")
    return workspace.data_ptr()


# ------------------------------------------------------ C-ABI entry points
def xfa_fwd(q, k, v, out, lse, scale=None, causal=True, stream=None) -> None:
    """q, k, v, out: [B,H,S,hd] (float32 or bfloat16); lse: [B,H,S] float32."""
    torch = _torch()
    B, H, S, hd = q.shape
    _check_same(q, q, k, v, out, shape=q.shape, dtype=q.dtype, names=("q", "k", "v", "out"))
    _check_same(q, lse, shape=(B, H, S), dtype=torch.float32, names=("lse",))
    st = lib().xfa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, H, S, hd, _scale(scale, hd), int(bool(causal)), _dtype_code(q),
                       _stream_handle(stream))
    _raise(st, "xfa_fwd")


def xfa_bwd_preprocess(out, dout, delta, scale=None, causal=True, stream=None) -> None:
    """delta [B,H,S] float32 <- rowsum(dout * out)."""
    torch = _torch()
    B, H, S, hd = out.shape
    _check_same(out, out, dout, shape=out.shape, dtype=out.dtype, names=("out", "dout"))
    _check_same(out, delta, shape=(B, H, S), dtype=torch.float32, names=("delta",))
    st = lib().xfa_bwd_preprocess(out.data_ptr(), dout.data_ptr(), delta.data_ptr(), B, H, S, hd,
                                  _scale(scale, hd), int(bool(causal)), _dtype_code(out),
                                  _stream_handle(stream))
    _raise(st, "xfa_bwd_preprocess")


def xfa_bwd(q, k, v, dout, lse, delta, dq, dk, dv, scale=None, causal=True, stream=None,
            workspace=None) -> None:
    """dq, dk, dv <- gradients of sum(dout * out).  workspace: a device tensor
    of at least xfa_bwd_workspace_bytes(...) bytes, or None when that is 0."""
    torch = _torch()
    B, H, S, hd = q.shape
    _check_same(q, q, k, v, dout, dq, dk, dv, shape=q.shape, dtype=q.dtype,
                names=("q", "k", "v", "dout", "dq", "dk", "dv"))
    _check_same(q, lse, delta, shape=(B, H, S), dtype=torch.float32, names=("lse", "delta"))
    ws = _workspace_ptr(q, workspace, "xfa_bwd")
    st = lib().xfa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws,
                       B, H, S, hd, _scale(scale, hd), int(bool(causal)), _dtype_code(q),
                       _stream_handle(stream))
    _raise(st, "xfa_bwd")


def xfa_fwd_dropout(q, k, v, out, lse, scale=None, causal=True, dropout_p=0.0, seed=0, stream=None) -> None:
    """xfa_fwd with dropout on the attention probabilities (keep decisions
    from (seed, element index), kept weights scaled by 1/(1-p))."""
    torch = _torch()
    B, H, S, hd = q.shape
    _check_same(q, q, k, v, out, shape=q.shape, dtype=q.dtype, names=("q", "k", "v", "out"))
    _check_same(q, lse, shape=(B, H, S), dtype=torch.float32, names=("lse",))
    st = lib().xfa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, S, hd, _scale(scale, hd), int(bool(causal)), float(dropout_p),
                               _seed(seed), _dtype_code(q), _stream_handle(stream))
    _raise(st, "xfa_fwd_dropout")


def xfa_bwd_dropout(q, k, v, dout, lse, delta, dq, dk, dv, scale=None, causal=True, dropout_p=0.0, seed=0,
                    stream=None, workspace=None) -> None:
    """xfa_bwd of the forward that xfa_fwd_dropout ran with the same p and seed."""
    torch = _torch()
    B, H, S, hd = q.shape
    _check_same(q, q, k, v, dout, dq, dk, dv, shape=q.shape, dtype=q.dtype,
                names=("q", "k", "v", "dout", "dq", "dk", "dv"))
    _check_same(q, lse, delta, shape=(B, H, S), dtype=torch.float32, names=("lse", "delta"))
    ws = _workspace_ptr(q, workspace, "xfa_bwd_dropout")
    st = lib().xfa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                               delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws,
                               B, H, S, hd, _scale(scale, hd), int(bool(causal)), float(dropout_p),
                               _seed(seed), _dtype_code(q), _stream_handle(stream))
    _raise(st, "xfa_bwd_dropout")


# ------------------------------------------------------------ conveniences
def forward(q, k, v, scale=None, causal=True, stream=None, dropout_p=0.0, seed=0):
    """Allocate and return (out, lse).  dropout_p > 0 calls xfa_fwd_dropout."""
    torch = _torch()
    B, H, S, hd = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if dropout_p:
        xfa_fwd_dropout(q, k, v, out, lse, scale, causal, dropout_p, seed, stream)
    else:
        xfa_fwd(q, k, v, out, lse, scale, causal, stream)
    return out, lse


def backward(q, k, v, out, dout, lse, scale=None, causal=True, stream=None, dropout_p=0.0, seed=0):
    """Run the preprocess and the backward; allocate and return (dq, dk, dv).
    dropout_p > 0 calls xfa_bwd_dropout (same p and seed as the forward)."""
    torch = _torch()
    B, H, S, hd = q.shape
    delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    xfa_bwd_preprocess(out, dout, delta, scale, causal, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = xfa_bwd_workspace_bytes(B, H, S, hd, _dtype_code(q))
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    if dropout_p:
        xfa_bwd_dropout(q, k, v, dout, lse, delta, dq, dk, dv, scale, causal, dropout_p, seed, stream, ws)
    else:
        xfa_bwd(q, k, v, dout, lse, delta, dq, dk, dv, scale, causal, stream, ws)
    return dq, dk, dv
