"""Python front of the float64 reference oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports this
package and this package never imports the GPU library; the two share nothing
but the seeded inputs of the `workload` module.

Each function converts its inputs exactly to float64 (bf16 bit patterns or
float32 both widen without rounding) and calls the C definition.  Citations
for every definition are in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BUILD_CMD = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", _LIB, _SRC, "-lm", "-lpthread"]

_lib = None


def build() -> str:
    subprocess.run(BUILD_CMD, check=True)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lp = ctypes.POINTER(ctypes.c_int64)
        L.oracle_rope_freq.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int]
        L.oracle_rope_freq.restype = ctypes.c_double
        L.oracle_rope.argtypes = [dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ip, ctypes.c_double]
        L.oracle_rope.restype = None
        L.oracle_attention.argtypes = [dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_double, lp, ctypes.c_int64,
                                       ctypes.c_int]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_layer_norm.argtypes = [dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, dp, dp, ctypes.c_double]
        L.oracle_layer_norm.restype = None
        L.oracle_attention_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_double, lp, ctypes.c_int64, lp, ctypes.c_int64, ctypes.c_int]
        L.oracle_attention_backward.restype = ctypes.c_int
        L.oracle_descriptor_count.argtypes = [ctypes.c_int] * 5
        L.oracle_descriptor_count.restype = ctypes.c_int
        L.oracle_descriptor_pool.argtypes = [dp, dp] + [ctypes.c_int] * 9
        L.oracle_descriptor_pool.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def _dp(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening: uint16 arrays are bf16 bit patterns; float32/float64 as is."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(x, dtype=np.float64)


def rope_freq(base: float, d_axis: int, k: int) -> float:
    return lib().oracle_rope_freq(base, d_axis, k)


def rope(x: np.ndarray, pos_tok: np.ndarray, base: float) -> np.ndarray:
    """Rotated copy of x [n_tok, H, D] (float64) for per-token positions
    pos_tok [n_tok, 2] (row, col)."""
    y = np.array(to_f64(x), dtype=np.float64, order="C", copy=True)
    n_tok, H, D = y.shape
    p = np.ascontiguousarray(pos_tok, dtype=np.int32).reshape(n_tok, 2)
    lib().oracle_rope(_dp(y), n_tok, H, D, p.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), float(base))
    return y


def layer_norm(x: np.ndarray, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """Per-head LayerNorm copy of x [n_tok, H, D] (float64) with gamma/beta [D]."""
    y = np.array(to_f64(x), dtype=np.float64, order="C", copy=True)
    n_tok, H, D = y.shape
    g = np.ascontiguousarray(to_f64(gamma), dtype=np.float64).reshape(D)
    b = np.ascontiguousarray(to_f64(beta), dtype=np.float64).reshape(D)
    lib().oracle_layer_norm(_dp(y), n_tok, H, D, _dp(g), _dp(b), float(eps))
    return y


def _prologue(x, pos, base, norm, S):
    """Q/K prologue: optional per-head LayerNorm (gamma, beta, eps), then RoPE."""
    if norm is not None:
        x = layer_norm(x, norm[0], norm[1], norm[2])
    if pos is not None:
        x = rope(x, _frame_positions(pos, S), base)
    return x


def attention(q, k, v, *, group_q: int = 0, group_k: int = 0, scale: float | None = None, rows=None,
              nthreads: int | None = None) -> np.ndarray:
    """Multi-head softmax attention.  q [nq, H, D], k/v [nk, H, D] (any of
    bf16-bits/float32/float64).  Returns float64 [len(rows) or nq, H, D]."""
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    nq, H, D = q64.shape
    nk = k64.shape[0]
    assert k64.shape == (nk, H, D) and v64.shape == (nk, H, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        r = None
        nrows = nq
        rp = None
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = r.size
        rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    o = np.zeros((nrows, H, D), dtype=np.float64)
    rc = lib().oracle_attention(_dp(q64), _dp(k64), _dp(v64), _dp(o), nq, nk, H, D, group_q, group_k, float(scale),
                                rp, nrows, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attention: bad arguments")
    return o


def _frame_positions(pos: np.ndarray, S: int) -> np.ndarray:
    return np.tile(np.asarray(pos, dtype=np.int32).reshape(-1, 2), (S, 1))


def frame_attn(q, k, v, S: int, T: int, pos=None, base: float = 100.0, scale=None, rows=None, nthreads=None,
               q_norm=None, k_norm=None):
    """Frame-wise attention: S independent sequences of T tokens.
    q/k/v [S, T, H, D]; pos [T, 2] shared by all frames (None: no RoPE);
    q_norm/k_norm (gamma, beta, eps) or None: per-head LayerNorm before RoPE.
    rows index tokens of the flattened [S*T] axis."""
    H, D = q.shape[-2:]
    qf, kf, vf = (to_f64(x).reshape(S * T, H, D) for x in (q, k, v))
    qf, kf = _prologue(qf, pos, base, q_norm, S), _prologue(kf, pos, base, k_norm, S)
    return attention(qf, kf, vf, group_q=T, group_k=T, scale=scale, rows=rows, nthreads=nthreads)


def global_attn(q, k, v, S: int, T: int, pos=None, base: float = 100.0, scale=None, rows=None, nthreads=None,
                q_norm=None, k_norm=None):
    """Global attention: one sequence of S*T tokens; each token keeps its own
    within-frame (row, col) position for RoPE.  q_norm/k_norm as for frame_attn."""
    H, D = q.shape[-2:]
    qf, kf, vf = (to_f64(x).reshape(S * T, H, D) for x in (q, k, v))
    qf, kf = _prologue(qf, pos, base, q_norm, S), _prologue(kf, pos, base, k_norm, S)
    return attention(qf, kf, vf, scale=scale, rows=rows, nthreads=nthreads)


def descriptor_count(T: int, gh: int, gw: int, ph: int, pw: int) -> int:
    return lib().oracle_descriptor_count(T, gh, gw, ph, pw)


def descriptor_pool(x, S: int, T: int, gh: int, gw: int, patch_begin: int, ph: int, pw: int) -> np.ndarray:
    """x [S, T, H, D] -> float64 [S, Dn, H, D]."""
    H, D = x.shape[-2:]
    x64 = to_f64(x).reshape(S, T, H, D)
    Dn = descriptor_count(T, gh, gw, ph, pw)
    out = np.zeros((S, Dn, H, D), dtype=np.float64)
    rc = lib().oracle_descriptor_pool(_dp(x64), _dp(out), S, T, H, D, gh, gw, patch_begin, ph, pw)
    if rc != 0:
        raise ValueError("oracle_descriptor_pool: bad arguments")
    return out


def descriptor_xattn(q, kd, vd, scale=None, rows=None, nthreads=None) -> np.ndarray:
    """Every query token [S, T, H, D] attends to every descriptor [S, Dn, H, D]."""
    H, D = q.shape[-2:]
    qf = to_f64(q).reshape(-1, H, D)
    kf = to_f64(kd).reshape(-1, H, D)
    vf = to_f64(vd).reshape(-1, H, D)
    return attention(qf, kf, vf, scale=scale, rows=rows, nthreads=nthreads)


def descriptor_stream_xattn(q, kd, vd, chunk_frames: int, scale=None, rows=None, nthreads=None) -> np.ndarray:
    """Chunk-recursive descriptor attention (FlashVGGT project page, Overview:
    online inference over long sequences that reuses the cached descriptors of
    earlier chunks; Key Arguments: --chunksize, default 10 frames).

    Frames are taken in consecutive chunks of `chunk_frames` (the last may be
    shorter).  A query token of chunk c attends to the descriptors of every
    frame of chunks 0..c, its own chunk included (the cache after chunk c has
    been appended), in frame order.  q [S, T, H, D], kd/vd [S, Dn, H, D];
    rows index the flattened [S*T] query axis.  float64 [len(rows) or S*T, H, D]."""
    S, T, H, D = q.shape
    Dn = kd.shape[1]
    if chunk_frames < 1:
        raise ValueError("chunk_frames must be >= 1")
    qf = to_f64(q).reshape(S * T, H, D)
    kf = to_f64(kd).reshape(S * Dn, H, D)
    vf = to_f64(vd).reshape(S * Dn, H, D)
    want = np.arange(S * T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.zeros((want.size, H, D), dtype=np.float64)
    for c in range((S + chunk_frames - 1) // chunk_frames):
        f_end = min(S, (c + 1) * chunk_frames)  # frames whose descriptors are cached after chunk c
        sel = (want >= c * chunk_frames * T) & (want < f_end * T)
        if sel.any():
            out[sel] = attention(qf, kf[:f_end * Dn], vf[:f_end * Dn], scale=scale, rows=want[sel],
                                 nthreads=nthreads)
    return out


def frame_attn_ex(q, k, v, S: int, T: int, T_active: int, pos=None, base: float = 100.0, scale=None,
                  nthreads=None, q_norm=None, k_norm=None) -> np.ndarray:
    """Frame attention over the first T_active tokens of each frame only
    (VGGT-Omega-1B-512-bf16 config article, special-token notes: the 16
    register tokens that follow each frame's patches join attention only in
    some blocks).  q/k/v [S, T, H, D]; returns float64 [S, T_active, H, D]."""
    H, D = q.shape[-2:]
    sub = [to_f64(x).reshape(S, T, H, D)[:, :T_active] for x in (q, k, v)]
    p = None if pos is None else np.asarray(pos).reshape(T, 2)[:T_active]
    o = frame_attn(*sub, S, T_active, pos=p, base=base, scale=scale, nthreads=nthreads, q_norm=q_norm,
                   k_norm=k_norm)
    return o.reshape(S, T_active, H, D)


def global_attn_ex(q, k, v, S: int, T: int, T_active: int, xq, xk, xv, pos=None, base: float = 100.0, scale=None,
                   nthreads=None, q_norm=None, k_norm=None, rows=None):
    """Global attention over the first T_active tokens of every frame plus
    n_extra sequence-level tokens (VGGT-Omega config article, special-token
    notes: 4 storage tokens shared by all frames as global memory and one
    camera token that gathers every frame's camera information).  The token
    set is the active frame tokens in frame order followed by the extra
    tokens; every token of the set is a query and a key.  Extra tokens carry
    no position (identity rotation); the LayerNorm, if any, applies to all.
    Returns (float64 [S, T_active, H, D], float64 [n_extra, H, D]); with rows
    (indices into the set: frame tokens first, then the extras) it returns
    float64 [len(rows), H, D] instead."""
    H, D = q.shape[-2:]
    E = 0 if xq is None else int(np.asarray(xq).shape[0])

    def tokens(x, xx):
        a = to_f64(x).reshape(S, T, H, D)[:, :T_active].reshape(S * T_active, H, D)
        return a if E == 0 else np.concatenate([a, to_f64(xx).reshape(E, H, D)])

    qf, kf, vf = tokens(q, xq), tokens(k, xk), tokens(v, xv)
    if q_norm is not None:
        qf = layer_norm(qf, *q_norm)
    if k_norm is not None:
        kf = layer_norm(kf, *k_norm)
    if pos is not None:
        pt = np.concatenate([_frame_positions(np.asarray(pos).reshape(T, 2)[:T_active], S),
                             np.zeros((E, 2), dtype=np.int32)])
        qf, kf = rope(qf, pt, base), rope(kf, pt, base)
    if rows is not None:
        return attention(qf, kf, vf, scale=scale, rows=rows, nthreads=nthreads)
    o = attention(qf, kf, vf, scale=scale, nthreads=nthreads)
    return o[:S * T_active].reshape(S, T_active, H, D), o[S * T_active:]


def _idx(a):
    if a is None:
        return None, 0, None
    r = np.ascontiguousarray(a, dtype=np.int64).reshape(-1)
    return r, r.size, r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def attention_backward(q, k, v, dout, *, group_q: int = 0, group_k: int = 0, scale=None, rows=None, cols=None,
                       nthreads=None):
    """Gradients of multi-head attention (oracle.c, oracle_attention_backward).
    q/dout [nq, H, D], k/v [nk, H, D].  Returns (dq [len(rows) or nq, H, D],
    dk, dv [len(cols) or nk, H, D], lse [nq, H]) in float64; lse is the natural
    log-normaliser of each query row that the requested gradients read (zero
    for the other rows)."""
    q64, k64, v64, d64 = (np.ascontiguousarray(to_f64(x), dtype=np.float64) for x in (q, k, v, dout))
    nq, H, D = q64.shape
    nk = k64.shape[0]
    assert k64.shape == v64.shape == (nk, H, D) and d64.shape == (nq, H, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    r, nr, rp = _idx(rows)
    c, nc, cp = _idx(cols)
    dq = np.zeros((nr if r is not None else nq, H, D))
    dk = np.zeros((nc if c is not None else nk, H, D))
    dv = np.zeros_like(dk)
    lse = np.zeros((nq, H))
    rc = lib().oracle_attention_backward(_dp(q64), _dp(k64), _dp(v64), _dp(d64), _dp(dq), _dp(dk), _dp(dv),
                                         _dp(lse), nq, nk, H, D, group_q, group_k, float(scale), rp, nr, cp, nc,
                                         nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attention_backward: bad arguments")
    return dq, dk, dv, lse


def _attn_backward(q, k, v, dout, S, T, pos, base, scale, rows, cols, nthreads, frame):
    """RoPE-aware gradients: the attention runs on q' = R q and k' = R k (R a
    rotation per position), so dq = R^T dq' and dk = R^T dk', and R^T is the
    rotation by the negated position."""
    H, D = q.shape[-2:]
    qf, kf, vf, df = (to_f64(x).reshape(S * T, H, D) for x in (q, k, v, dout))
    if pos is not None:
        pt = _frame_positions(pos, S)
        qf, kf = rope(qf, pt, base), rope(kf, pt, base)
    g = T if frame else 0
    dq, dk, dv, lse = attention_backward(qf, kf, vf, df, group_q=g, group_k=g, scale=scale, rows=rows, cols=cols,
                                         nthreads=nthreads)
    if pos is not None:
        pt = _frame_positions(pos, S)
        back = -pt
        dq = rope(dq, back if rows is None else back[np.asarray(rows)], base)
        dk = rope(dk, back if cols is None else back[np.asarray(cols)], base)
    return dq, dk, dv, lse


def frame_attn_backward(q, k, v, dout, S: int, T: int, pos=None, base: float = 100.0, scale=None, rows=None,
                        cols=None, nthreads=None):
    """Gradients of frame_attn: (dq, dk, dv, lse); rows/cols index the [S*T] token axis."""
    return _attn_backward(q, k, v, dout, S, T, pos, base, scale, rows, cols, nthreads, True)


def global_attn_backward(q, k, v, dout, S: int, T: int, pos=None, base: float = 100.0, scale=None, rows=None,
                         cols=None, nthreads=None):
    """Gradients of global_attn: (dq, dk, dv, lse); rows/cols index the [S*T] token axis."""
    return _attn_backward(q, k, v, dout, S, T, pos, base, scale, rows, cols, nthreads, False)
