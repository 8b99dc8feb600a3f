"""Python binding of libvggt_attn (MI355X / gfx950 alternating attention).

Thin argument marshalling over the C ABI declared in include/vggt_attn.h:
every function checks dtype, shape, contiguity and device of torch tensors,
passes raw device pointers and the current HIP stream, and raises on a
non-OK status.  All computation happens in the library's HIP kernels; torch
only provides device memory and streams.  There is no fallback: if the
library is missing or fails to load, every call raises.

Streams: a call launches on `stream` (default: torch's current stream) and,
when one is given, runs with it as torch's current stream, so its workspace
and default-allocated outputs belong to that stream.  Buffers the caller
allocated elsewhere stay the caller's to order (Tensor.record_stream).
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvggt_attn.so")

BF16, F32 = 0, 1
HEAD_DIM = 64

STATUS = {
    0: "VGGT_OK", 1: "VGGT_ERR_NULL", 2: "VGGT_ERR_SHAPE", 3: "VGGT_ERR_UNSUPPORTED", 4: "VGGT_ERR_ALIGN",
    5: "VGGT_ERR_ALIAS", 6: "VGGT_ERR_WORKSPACE", 7: "VGGT_ERR_DEVICE",
}

PRE_ROPE, PRE_QKNORM = 1, 2


class QkNorm(ctypes.Structure):
    """vggt_qk_norm: device pointers of the [64] float32 LayerNorm parameters and eps."""
    _fields_ = [("q_gamma", ctypes.c_void_p), ("q_beta", ctypes.c_void_p), ("k_gamma", ctypes.c_void_p),
                ("k_beta", ctypes.c_void_p), ("eps", ctypes.c_float)]


# name -> (restype, argtypes); pointers are passed as c_void_p
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_np = ctypes.POINTER(QkNorm)
SIGNATURES = {
    "vggt_abi_version": (_i, []),
    "vggt_status_str": (ctypes.c_char_p, [_i]),
    "vggt_last_error": (ctypes.c_char_p, []),
    "vggt_attn_rope": (_i, [_vp, _i, _i, _i, _i, _vp, _f, _vp]),
    "vggt_frame_attn_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "vggt_frame_attn": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _vp, _sz, _vp]),
    "vggt_frame_attn_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _vp]),
    "vggt_global_attn_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "vggt_global_attn": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _i, _vp, _sz, _vp]),
    "vggt_frame_attn_qknorm": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _np, _vp, _sz, _vp]),
    "vggt_global_attn_qknorm": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _i, _np, _vp, _sz, _vp]),
    "vggt_descriptor_count": (_i, [_i, _i, _i, _i, _i]),
    "vggt_descriptor_pool": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "vggt_descriptor_xattn_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "vggt_descriptor_xattn": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "vggt_descriptor_cache_bytes": (_sz, [_i, _i, _i]),
    "vggt_descriptor_cache_append": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _i, _vp]),
    "vggt_descriptor_cache_attn_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "vggt_descriptor_cache_attn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "vggt_descriptor_chunked_xattn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "vggt_frame_attn_ex_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "vggt_frame_attn_ex": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _f, _f, _np, _vp, _sz, _vp]),
    "vggt_global_attn_ex_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "vggt_global_attn_ex": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _f, _f, _i,
                                 _np, _vp, _sz, _vp]),
    "vggt_frame_attn_train": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _vp, _sz, _vp]),
    "vggt_global_attn_train": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _f, _f, _i, _vp, _sz, _vp]),
    "vggt_attn_backward_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "vggt_frame_attn_backward": (_i, [_vp] * 9 + [_i, _i, _i, _i, _vp, _f, _f, _vp, _sz, _vp]),
    "vggt_global_attn_backward": (_i, [_vp] * 9 + [_i, _i, _i, _i, _vp, _f, _f, _vp, _sz, _vp]),
    "vggt_timer_start": (_i, [_i]),
    "vggt_timer_stop": (_i, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_i), _i, ctypes.POINTER(_i)]),
}

TIMER_KINDS = {1: "frame", 2: "global", 3: "xattn", 4: "cache", 5: "chunked", 6: "bwd_dq", 7: "bwd_dkdv"}

_lib = None


class VggtError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m feed_forward_view_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise VggtError(fn, status, lib().vggt_last_error().decode(errors="replace"))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _tok(t: torch.Tensor, name: str) -> tuple[int, int, int]:
    if t.dim() != 4 or t.shape[-1] != HEAD_DIM:
        raise ValueError(f"{name} must be [S, T, H, {HEAD_DIM}], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    return int(t.shape[0]), int(t.shape[1]), int(t.shape[2])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _pos(pos_yx, T: int):
    if pos_yx is None:
        return None
    if pos_yx.dtype != torch.int32 or tuple(pos_yx.shape) != (T, 2) or not pos_yx.is_contiguous():
        raise ValueError(f"pos_yx must be contiguous int32 [{T}, 2]")
    return ctypes.c_void_p(pos_yx.data_ptr())


def _on_stream(fn):
    """Run a call with the caller's `stream` as torch's current stream, so that the
    workspace and any default-allocated outputs come from that stream's pool: the
    caching allocator then hands a block freed after the call (the workspace) only
    to later work of the same stream, never to another stream while the kernels
    still read it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        s = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if s is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(s):
            return fn(*args, **kwargs)

    return wrapper


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace, workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# the five calls (names as in the C ABI)
# ---------------------------------------------------------------------------

@_on_stream
def vggt_attn_rope(x: torch.Tensor, pos_yx: torch.Tensor, rope_base: float = 100.0, stream=None) -> torch.Tensor:
    """Rotate x [S, T, H, 64] in place by 2D RoPE; returns x."""
    S, T, H = _tok(x, "x")
    _check("vggt_attn_rope",
           lib().vggt_attn_rope(_ptr(x), _dtype_code(x), S, T, H, _pos(pos_yx, T), rope_base, _stream(stream)))
    return x


def vggt_frame_attn_workspace(S, T, H, rope_on, dtype=torch.bfloat16) -> int:
    """rope_on: bool, or PRE_ROPE | PRE_QKNORM flags."""
    return int(lib().vggt_frame_attn_workspace(S, T, H, int(rope_on), BF16 if dtype == torch.bfloat16 else F32))


@_on_stream
def vggt_frame_attn(q, k, v, out=None, pos_yx=None, rope_base=100.0, scale=0.0, workspace=None, stream=None):
    """Frame-wise attention over [S, T, H, 64]; returns out."""
    S, T, H = _tok(q, "q")
    for n, t in (("k", k), ("v", v)):
        if _tok(t, n) != (S, T, H) or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q")
    out = torch.empty_like(q) if out is None else out
    if _tok(out, "out") != (S, T, H) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = vggt_frame_attn_workspace(S, T, H, pos_yx is not None, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_frame_attn",
           lib().vggt_frame_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, H, _pos(pos_yx, T),
                                 rope_base, scale, _ptr(ws), nbytes, _stream(stream)))
    return out


def vggt_global_attn_workspace(S, T, H, kv_splits, rope_on, dtype=torch.bfloat16) -> int:
    """rope_on: bool, or PRE_ROPE | PRE_QKNORM flags."""
    return int(lib().vggt_global_attn_workspace(S, T, H, kv_splits, int(rope_on),
                                                BF16 if dtype == torch.bfloat16 else F32))


@_on_stream
def vggt_frame_attn_noalloc(q, k, v, out=None, pos_yx=None, rope_base=100.0, scale=0.0, stream=None):
    """vggt_frame_attn whose workspace is the library's own device array (the C call
    allocates nothing; pass `out` to allocate nothing here either); returns out."""
    S, T, H, out = _check_qkv(q, k, v, out)
    _check("vggt_frame_attn_noalloc",
           lib().vggt_frame_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, H,
                                         _pos(pos_yx, T), rope_base, scale, _stream(stream)))
    return out


@_on_stream
def vggt_global_attn(q, k, v, out=None, pos_yx=None, rope_base=100.0, scale=0.0, kv_splits=0, workspace=None,
                     stream=None):
    """Global attention over all S*T tokens; returns out."""
    S, T, H = _tok(q, "q")
    for n, t in (("k", k), ("v", v)):
        if _tok(t, n) != (S, T, H) or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q")
    out = torch.empty_like(q) if out is None else out
    if _tok(out, "out") != (S, T, H) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = vggt_global_attn_workspace(S, T, H, kv_splits, pos_yx is not None, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_global_attn",
           lib().vggt_global_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, H, _pos(pos_yx, T),
                                  rope_base, scale, kv_splits, _ptr(ws), nbytes, _stream(stream)))
    return out


def _qk_norm(q_norm, k_norm, eps: float, H: int):
    """QkNorm from (gamma, beta) pairs of float32 [64] GPU tensors."""
    ptrs = []
    for name, pair in (("q_norm", q_norm), ("k_norm", k_norm)):
        for t in pair:
            if t.dtype != torch.float32 or t.numel() != HEAD_DIM or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"{name} gamma/beta must be contiguous float32 GPU tensors of {HEAD_DIM}")
            ptrs.append(t.data_ptr())
    return QkNorm(ptrs[0], ptrs[1], ptrs[2], ptrs[3], eps)


def _check_qkv(q, k, v, out):
    S, T, H = _tok(q, "q")
    for n, t in (("k", k), ("v", v)):
        if _tok(t, n) != (S, T, H) or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q")
    out = torch.empty_like(q) if out is None else out
    if _tok(out, "out") != (S, T, H) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    return S, T, H, out


@_on_stream
def vggt_frame_attn_qknorm(q, k, v, q_norm, k_norm, eps=1e-5, out=None, pos_yx=None, rope_base=100.0, scale=0.0,
                           workspace=None, stream=None):
    """Frame-wise attention with per-head LayerNorm of q and k (gamma, beta pairs) before RoPE."""
    S, T, H, out = _check_qkv(q, k, v, out)
    norm = _qk_norm(q_norm, k_norm, eps, H)
    flags = PRE_QKNORM | (PRE_ROPE if pos_yx is not None else 0)
    need = vggt_frame_attn_workspace(S, T, H, flags, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_frame_attn_qknorm",
           lib().vggt_frame_attn_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, H,
                                        _pos(pos_yx, T), rope_base, scale, ctypes.byref(norm), _ptr(ws), nbytes,
                                        _stream(stream)))
    return out


@_on_stream
def vggt_global_attn_qknorm(q, k, v, q_norm, k_norm, eps=1e-5, out=None, pos_yx=None, rope_base=100.0, scale=0.0,
                            kv_splits=0, workspace=None, stream=None):
    """Global attention with per-head LayerNorm of q and k (gamma, beta pairs) before RoPE."""
    S, T, H, out = _check_qkv(q, k, v, out)
    norm = _qk_norm(q_norm, k_norm, eps, H)
    flags = PRE_QKNORM | (PRE_ROPE if pos_yx is not None else 0)
    need = vggt_global_attn_workspace(S, T, H, kv_splits, flags, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_global_attn_qknorm",
           lib().vggt_global_attn_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, H,
                                         _pos(pos_yx, T), rope_base, scale, kv_splits, ctypes.byref(norm), _ptr(ws),
                                         nbytes, _stream(stream)))
    return out


def _norm_arg(q_norm, k_norm, eps, H):
    if q_norm is None and k_norm is None:
        return None, 0
    if q_norm is None or k_norm is None:
        raise ValueError("give both q_norm and k_norm, or neither")
    return ctypes.byref(_qk_norm(q_norm, k_norm, eps, H)), PRE_QKNORM


@_on_stream
def vggt_frame_attn_ex(q, k, v, T_active, out=None, pos_yx=None, rope_base=100.0, scale=0.0, q_norm=None,
                       k_norm=None, eps=1e-5, workspace=None, stream=None):
    """Frame attention over the first T_active tokens of each frame of [S, T, H, 64];
    rows past T_active of `out` are left as they are (allocated empty when out is None)."""
    S, T, H, out = _check_qkv(q, k, v, out)
    norm, flags = _norm_arg(q_norm, k_norm, eps, H)
    flags |= PRE_ROPE if pos_yx is not None else 0
    need = int(lib().vggt_frame_attn_ex_workspace(S, T, T_active, H, flags, _dtype_code(q)))
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_frame_attn_ex",
           lib().vggt_frame_attn_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, T_active, H,
                                    _pos(pos_yx, T), rope_base, scale, norm, _ptr(ws), nbytes, _stream(stream)))
    return out


@_on_stream
def vggt_global_attn_ex(q, k, v, T_active, xq=None, xk=None, xv=None, out=None, xout=None, pos_yx=None,
                        rope_base=100.0, scale=0.0, kv_splits=0, q_norm=None, k_norm=None, eps=1e-5,
                        workspace=None, stream=None):
    """Global attention over the first T_active tokens of every frame plus the extra
    tokens xq/xk/xv [E, H, 64]; returns (out, xout)."""
    S, T, H, out = _check_qkv(q, k, v, out)
    E = 0 if xq is None else int(xq.shape[0])
    if E:
        for n, t in (("xq", xq), ("xk", xk), ("xv", xv)):
            if t is None or tuple(t.shape) != (E, H, HEAD_DIM) or t.dtype != q.dtype or not t.is_contiguous():
                raise ValueError(f"{n} must be a contiguous [{E}, {H}, 64] tensor of q's dtype")
        xout = torch.empty_like(xq) if xout is None else xout
    norm, flags = _norm_arg(q_norm, k_norm, eps, H)
    flags |= PRE_ROPE if pos_yx is not None else 0
    need = int(lib().vggt_global_attn_ex_workspace(S, T, T_active, E, H, kv_splits, flags, _dtype_code(q)))
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_global_attn_ex",
           lib().vggt_global_attn_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), S, T, T_active, H,
                                     _ptr(xq if E else None), _ptr(xk if E else None), _ptr(xv if E else None),
                                     _ptr(xout if E else None), E, _pos(pos_yx, T), rope_base, scale, kv_splits,
                                     norm, _ptr(ws), nbytes, _stream(stream)))
    return out, (xout if E else None)


@_on_stream
def vggt_frame_attn_train(q, k, v, out=None, lse=None, pos_yx=None, rope_base=100.0, scale=0.0, workspace=None,
                          stream=None):
    """Frame attention that also returns the log-normaliser lse [S*T, H] (float32); returns (out, lse)."""
    S, T, H, out = _check_qkv(q, k, v, out)
    lse = torch.empty((S * T, H), dtype=torch.float32, device=q.device) if lse is None else lse
    need = vggt_frame_attn_workspace(S, T, H, pos_yx is not None, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_frame_attn_train",
           lib().vggt_frame_attn_train(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), S, T, H,
                                       _pos(pos_yx, T), rope_base, scale, _ptr(ws), nbytes, _stream(stream)))
    return out, lse


@_on_stream
def vggt_global_attn_train(q, k, v, out=None, lse=None, pos_yx=None, rope_base=100.0, scale=0.0, kv_splits=0,
                           workspace=None, stream=None):
    """Global attention that also returns the log-normaliser lse [S*T, H] (float32); returns (out, lse)."""
    S, T, H, out = _check_qkv(q, k, v, out)
    lse = torch.empty((S * T, H), dtype=torch.float32, device=q.device) if lse is None else lse
    need = vggt_global_attn_workspace(S, T, H, kv_splits, pos_yx is not None, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_global_attn_train",
           lib().vggt_global_attn_train(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), S, T, H,
                                        _pos(pos_yx, T), rope_base, scale, kv_splits, _ptr(ws), nbytes,
                                        _stream(stream)))
    return out, lse


def _backward(name, global_, q, k, v, out, dout, lse, pos_yx, rope_base, scale, workspace, stream, grads):
    S, T, H, _ = _check_qkv(q, k, v, out)
    if tuple(dout.shape) != tuple(q.shape) or dout.dtype != q.dtype or not dout.is_contiguous():
        raise ValueError("dout must match q")
    if lse.dtype != torch.float32 or lse.numel() != S * T * H or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous float32 of {S * T * H} elements")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3)) if grads is None else grads
    need = int(lib().vggt_attn_backward_workspace(S, T, H, int(global_), int(pos_yx is not None), _dtype_code(q)))
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(name, getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                      _ptr(dv), _dtype_code(q), S, T, H, _pos(pos_yx, T), rope_base, scale, _ptr(ws),
                                      nbytes, _stream(stream)))
    return dq, dk, dv


@_on_stream
def vggt_frame_attn_backward(q, k, v, out, dout, lse, pos_yx=None, rope_base=100.0, scale=0.0, workspace=None,
                             stream=None, grads=None):
    """Gradients (dq, dk, dv) of frame attention from the training forward's out and lse."""
    return _backward("vggt_frame_attn_backward", False, q, k, v, out, dout, lse, pos_yx, rope_base, scale, workspace,
                     stream, grads)


@_on_stream
def vggt_global_attn_backward(q, k, v, out, dout, lse, pos_yx=None, rope_base=100.0, scale=0.0, workspace=None,
                              stream=None, grads=None):
    """Gradients (dq, dk, dv) of global attention from the training forward's out and lse."""
    return _backward("vggt_global_attn_backward", True, q, k, v, out, dout, lse, pos_yx, rope_base, scale, workspace,
                     stream, grads)


def vggt_descriptor_count(T, gh, gw, ph, pw) -> int:
    return int(lib().vggt_descriptor_count(T, gh, gw, ph, pw))


@_on_stream
def vggt_descriptor_pool(k, v, gh, gw, patch_begin, ph=2, pw=2, kd=None, vd=None, stream=None):
    """Pool K and V [S, T, H, 64] into descriptors [S, Dn, H, 64]; returns (kd, vd)."""
    S, T, H = _tok(k, "k")
    if _tok(v, "v") != (S, T, H) or v.dtype != k.dtype:
        raise ValueError("v must match k")
    Dn = vggt_descriptor_count(T, gh, gw, ph, pw)
    if Dn < 1:
        raise ValueError("bad pooling grid")
    kd = torch.empty((S, Dn, H, HEAD_DIM), dtype=k.dtype, device=k.device) if kd is None else kd
    vd = torch.empty((S, Dn, H, HEAD_DIM), dtype=k.dtype, device=k.device) if vd is None else vd
    for n, t in (("kd", kd), ("vd", vd)):
        if _tok(t, n) != (S, Dn, H) or t.dtype != k.dtype:
            raise ValueError(f"{n} must be [{S}, {Dn}, {H}, 64]")
    _check("vggt_descriptor_pool",
           lib().vggt_descriptor_pool(_ptr(k), _ptr(v), _ptr(kd), _ptr(vd), _dtype_code(k), S, T, H, gh, gw,
                                      patch_begin, ph, pw, _stream(stream)))
    return kd, vd


def vggt_descriptor_xattn_workspace(S, T, Dn, H, kv_splits, dtype=torch.bfloat16) -> int:
    return int(lib().vggt_descriptor_xattn_workspace(S, T, Dn, H, kv_splits, BF16 if dtype == torch.bfloat16 else F32))


@_on_stream
def vggt_descriptor_xattn(q, kd, vd, out=None, scale=0.0, kv_splits=0, workspace=None, stream=None):
    """All S*T queries attend to all S*Dn descriptors; returns out."""
    S, T, H = _tok(q, "q")
    S2, Dn, H2 = _tok(kd, "kd")
    if (S2, H2) != (S, H) or _tok(vd, "vd") != (S, Dn, H) or kd.dtype != q.dtype or vd.dtype != q.dtype:
        raise ValueError("kd/vd must be [S, Dn, H, 64] of q's dtype")
    out = torch.empty_like(q) if out is None else out
    if _tok(out, "out") != (S, T, H) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = vggt_descriptor_xattn_workspace(S, T, Dn, H, kv_splits, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_descriptor_xattn",
           lib().vggt_descriptor_xattn(_ptr(q), _ptr(kd), _ptr(vd), _ptr(out), _dtype_code(q), S, T, Dn, H, scale,
                                       kv_splits, _ptr(ws), nbytes, _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# FlashVGGT chunk-recursive attention over a descriptor cache
# ---------------------------------------------------------------------------

def _code(dtype) -> int:
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dtype}; use bfloat16 or float32")


def vggt_descriptor_cache_bytes(capacity: int, H: int, dtype=torch.bfloat16) -> int:
    return int(lib().vggt_descriptor_cache_bytes(capacity, H, _code(dtype)))


@_on_stream
def vggt_descriptor_cache_append(cache: torch.Tensor, capacity: int, H: int, used: int, kd: torch.Tensor,
                                 vd: torch.Tensor, dtype=None, stream=None) -> int:
    """Append descriptors kd/vd [..., H, 64] (flattened to [n, H, 64]) at position `used` of the
    cache buffer (uint8 device tensor); returns the new count."""
    dtype = kd.dtype if dtype is None else dtype
    for n, t in (("kd", kd), ("vd", vd)):
        if t.dtype != dtype or t.shape[-2:] != (H, HEAD_DIM) or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{n} must be a contiguous GPU tensor [..., {H}, 64] of {dtype}")
    n = kd.numel() // (H * HEAD_DIM)
    if vd.numel() != kd.numel():
        raise ValueError("kd and vd must hold the same number of descriptors")
    _check("vggt_descriptor_cache_append",
           lib().vggt_descriptor_cache_append(_ptr(cache), _code(dtype), capacity, H, used, _ptr(kd), _ptr(vd), n,
                                              _stream(stream)))
    return used + n


def vggt_descriptor_cache_attn_workspace(nq: int, used: int, H: int, kv_splits: int, dtype=torch.bfloat16) -> int:
    return int(lib().vggt_descriptor_cache_attn_workspace(nq, used, H, kv_splits, _code(dtype)))


@_on_stream
def vggt_descriptor_cache_attn(q: torch.Tensor, cache: torch.Tensor, capacity: int, used: int, out=None, scale=0.0,
                               kv_splits=0, workspace=None, stream=None) -> torch.Tensor:
    """Query tokens q [..., H, 64] attend to the first `used` cached descriptors; returns out (q's shape)."""
    H = int(q.shape[-2])
    if q.shape[-1] != HEAD_DIM or not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous GPU tensor [..., H, 64]")
    nq = q.numel() // (H * HEAD_DIM)
    out = torch.empty_like(q) if out is None else out
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    need = vggt_descriptor_cache_attn_workspace(nq, used, H, kv_splits, q.dtype)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check("vggt_descriptor_cache_attn",
           lib().vggt_descriptor_cache_attn(_ptr(q), _ptr(cache), _ptr(out), _dtype_code(q), capacity, H, used, nq,
                                            scale, kv_splits, _ptr(ws), nbytes, _stream(stream)))
    return out


@_on_stream
def vggt_descriptor_chunked_xattn(q: torch.Tensor, cache: torch.Tensor, capacity: int, Dn: int, chunk_frames: int,
                                  out=None, scale=0.0, stream=None) -> torch.Tensor:
    """All chunks in one launch: q [S, T, H, 64]; the cache holds the S*Dn descriptors of all frames."""
    S, T, H = _tok(q, "q")
    out = torch.empty_like(q) if out is None else out
    if _tok(out, "out") != (S, T, H) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    _check("vggt_descriptor_chunked_xattn",
           lib().vggt_descriptor_chunked_xattn(_ptr(q), _ptr(cache), _ptr(out), _dtype_code(q), capacity, H, S, T, Dn,
                                               chunk_frames, scale, _stream(stream)))
    return out


class DescriptorCache:
    """Caller-side bookkeeping for one descriptor cache: the device buffer, its
    capacity and the number of descriptors appended so far."""

    def __init__(self, capacity: int, H: int = 16, dtype=torch.bfloat16, device="cuda"):
        nbytes = vggt_descriptor_cache_bytes(capacity, H, dtype)
        if nbytes == 0:
            raise ValueError("bad cache shape")
        self.capacity, self.H, self.dtype = capacity, H, dtype
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.used = 0

    def append(self, kd: torch.Tensor, vd: torch.Tensor, stream=None) -> int:
        self.used = vggt_descriptor_cache_append(self.buffer, self.capacity, self.H, self.used, kd, vd, self.dtype,
                                                 stream)
        return self.used

    def attend(self, q: torch.Tensor, out=None, scale=0.0, kv_splits=0, workspace=None, stream=None) -> torch.Tensor:
        return vggt_descriptor_cache_attn(q, self.buffer, self.capacity, self.used, out, scale, kv_splits, workspace,
                                          stream)

    def attend_chunked(self, q: torch.Tensor, Dn: int, chunk_frames: int, out=None, scale=0.0,
                       stream=None) -> torch.Tensor:
        return vggt_descriptor_chunked_xattn(q, self.buffer, self.capacity, Dn, chunk_frames, out, scale, stream)


# ---------------------------------------------------------------------------
# diagnostics: attention kernel timer
# ---------------------------------------------------------------------------

_timer_capacity = 0


def vggt_timer_start(capacity: int) -> None:
    """Arm device-side timing of the next `capacity` attention kernel launches."""
    global _timer_capacity
    _check("vggt_timer_start", lib().vggt_timer_start(capacity))
    _timer_capacity = capacity


def vggt_timer_stop() -> list[tuple[str, float]]:
    """Wait for the recorded launches and return [(call kind, kernel ms), ...] in launch order."""
    n_max = max(_timer_capacity, 1)
    ms = (ctypes.c_float * n_max)()
    kinds = (ctypes.c_int * n_max)()
    n = ctypes.c_int(0)
    _check("vggt_timer_stop", lib().vggt_timer_stop(ms, kinds, n_max, ctypes.byref(n)))
    return [(TIMER_KINDS.get(kinds[i], str(kinds[i])), float(ms[i])) for i in range(min(n.value, n_max))]
