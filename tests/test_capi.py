"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, and rejects bad arguments with the
documented status before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import feed_forward_view_amd as ffv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vggt_attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS = 0, 1, 2, 3, 4, 5, 6


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vggt_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ffv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ffv.lib()


def test_exports_match_header(L):
    declared = header_functions()
    assert len(declared) == 31
    out = subprocess.run(["nm", "-D", "--defined-only", ffv.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted(set(m for m in re.findall(r"\bT (vggt_\w+)", out)))
    assert exported == declared
    assert sorted(ffv.SIGNATURES) == declared


def test_version_and_status_strings(L):
    assert L.vggt_abi_version() == 6
    for code, name in ffv.STATUS.items():
        assert L.vggt_status_str(code).decode() == name
    assert L.vggt_status_str(99).decode() == "VGGT_ERR_UNKNOWN"


def test_descriptor_count(L):
    assert L.vggt_descriptor_count(1374, 37, 37, 2, 2) == 366
    assert L.vggt_descriptor_count(1040, 32, 32, 2, 2) == 16 + 256
    assert L.vggt_descriptor_count(261, 16, 16, 1, 1) == 261
    assert L.vggt_descriptor_count(10, 4, 4, 2, 2) == -1  # grid larger than T


def test_workspace_queries(L):
    BF16, F32 = 0, 1
    S, T, H = 4, 261, 16
    tensor = S * T * H * 64
    # bf16: K in 64-key tiles (keys padded to 64 per sequence), and V^T tiles too when 32 or
    # more 256-query tiles share a key set (else V is read in place); with RoPE also the
    # cos/sin table
    tiles = S * H * 5 * 64 * 64 * 2
    assert L.vggt_frame_attn_workspace(S, T, H, 0, BF16) == tiles
    assert L.vggt_frame_attn_workspace(S, T, H, 1, BF16) >= tiles + T * 32 * 8
    # fp32 debug: nothing without RoPE, rotated Q and K copies with it
    assert L.vggt_frame_attn_workspace(S, T, H, 0, F32) == 0
    assert L.vggt_frame_attn_workspace(S, T, H, 1, F32) >= 2 * tensor * 4
    # explicit splits add the fp32 partials (64 values + max + sum per row and head)
    n = S * T
    base = L.vggt_global_attn_workspace(S, T, H, 1, 0, BF16)
    assert base == H * 17 * 64 * 64 * 2  # 5 query tiles: V in place
    big = (32 * 256 + 63) // 64  # 32 query tiles of one sequence: K and V^T tiles
    assert L.vggt_global_attn_workspace(1, 32 * 256, H, 1, 0, BF16) == 2 * H * big * 64 * 64 * 2
    assert L.vggt_global_attn_workspace(1, 31 * 256, H, 1, 0, BF16) == H * (31 * 4) * 64 * 64 * 2
    assert L.vggt_global_attn_workspace(S, T, H, 3, 0, BF16) >= base + 3 * n * H * (64 + 2) * 4
    assert L.vggt_global_attn_workspace(S, T, H, 1, 0, F32) == 0
    assert L.vggt_descriptor_xattn_workspace(100, 1374, 366, 16, 1, F32) == 0
    # invalid arguments give 0
    assert L.vggt_global_attn_workspace(S, T, H, 65, 0, BF16) == 0
    assert L.vggt_frame_attn_workspace(S, 0, H, 1, BF16) == 0


def _p(addr):
    return ctypes.c_void_p(addr)


A = 0x100000  # fake, aligned, never dereferenced: every call below fails validation first
B = 0x200000
C = 0x300000
O = 0x400000


def test_rejects_bad_arguments_without_device(L):
    f = L.vggt_frame_attn
    # null pointer
    assert f(None, _p(B), _p(C), _p(O), 0, 2, 8, 1, None, 100.0, 0.0, None, 0, None) == NULL
    # bad shapes / dtype
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 0, 1, None, 100.0, 0.0, None, 0, None) == SHAPE
    assert f(_p(A), _p(B), _p(C), _p(O), 0, -1, 8, 1, None, 100.0, 0.0, None, 0, None) == SHAPE
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 0, None, 100.0, 0.0, None, 0, None) == SHAPE
    assert f(_p(A), _p(B), _p(C), _p(O), 7, 2, 8, 1, None, 100.0, 0.0, None, 0, None) == UNSUP
    # misaligned
    assert f(_p(A + 2), _p(B), _p(C), _p(O), 0, 2, 8, 1, None, 100.0, 0.0, None, 0, None) == ALIGN
    # output aliases an input
    assert f(_p(A), _p(B), _p(C), _p(A + 64), 0, 2, 8, 1, None, 100.0, 0.0, None, 0, None) == ALIAS
    # RoPE needs a workspace; too small one
    pos = _p(0x500000)
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 1, pos, 100.0, 0.0, None, 0, None) == WS
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 1, pos, 100.0, 0.0, _p(0x600000), 16, None) == WS
    # bad rope base
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 1, pos, -1.0, 0.0, _p(0x600000), 1 << 20, None) == SHAPE
    # S == 0 is a no-op
    assert f(None, None, None, None, 0, 0, 8, 1, None, 100.0, 0.0, None, 0, None) == OK

    g = L.vggt_global_attn
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 1, None, 100.0, 0.0, 65, None, 0, None) == SHAPE
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 1, None, 100.0, 0.0, -1, None, 0, None) == SHAPE
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 64, 64, 1, None, 100.0, 0.0, 4, None, 0, None) == WS

    r = L.vggt_attn_rope
    assert r(_p(A), 0, 2, 8, 1, None, 100.0, None) == NULL
    assert r(_p(A), 0, 2, 8, 1, _p(0x500000), 0.0, None) == SHAPE
    assert r(_p(A + 8), 0, 2, 8, 1, _p(0x500000), 100.0, None) == ALIGN

    pl = L.vggt_descriptor_pool
    assert pl(_p(A), _p(B), None, _p(O), 0, 2, 14, 1, 3, 4, 2, 2, 2, None) == NULL
    assert pl(_p(A), _p(B), _p(C), _p(O), 0, 2, 14, 1, 3, 4, 3, 2, 2, None) == SHAPE  # grid past T
    assert pl(_p(A), _p(B), _p(A), _p(O), 0, 2, 14, 1, 3, 4, 2, 2, 2, None) == ALIAS

    x = L.vggt_descriptor_xattn
    assert x(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 0, 1, 0.0, 0, None, 0, None) == SHAPE
    assert x(_p(A), _p(B), _p(C), _p(B), 0, 2, 8, 3, 1, 0.0, 1, None, 0, None) == ALIAS
    assert L.vggt_last_error().decode() != ""


def test_descriptor_cache_sizes(L):
    BF16, F32 = 0, 1
    # bf16: K tiles and transposed-V tiles of 64 descriptors per head; fp32: plain K then V
    assert L.vggt_descriptor_cache_bytes(36600, 16, BF16) == 2 * 16 * 572 * 64 * 64 * 2
    assert L.vggt_descriptor_cache_bytes(65, 2, BF16) == 2 * 2 * 2 * 64 * 64 * 2
    assert L.vggt_descriptor_cache_bytes(65, 2, F32) == 2 * 65 * 2 * 64 * 4
    assert L.vggt_descriptor_cache_bytes(0, 16, BF16) == 0
    assert L.vggt_descriptor_cache_bytes(10, 0, BF16) == 0
    # attention on the cache needs only split partials
    assert L.vggt_descriptor_cache_attn_workspace(13740, 3660, 16, 1, BF16) == 0
    assert L.vggt_descriptor_cache_attn_workspace(1000, 3660, 16, 3, BF16) >= 3 * 1000 * 16 * 66 * 4
    assert L.vggt_descriptor_cache_attn_workspace(1000, 0, 16, 3, BF16) == 0


def test_descriptor_cache_rejects_bad_arguments(L):
    ap = L.vggt_descriptor_cache_append
    # (cache, dt, capacity, H, used, kd, vd, n, stream)
    assert ap(_p(A), 0, 100, 2, 90, _p(B), _p(C), 11, None) == SHAPE   # past capacity
    assert ap(_p(A), 0, 100, 2, -1, _p(B), _p(C), 1, None) == SHAPE
    assert ap(_p(A), 0, 100, 2, 0, _p(B), _p(C), 0, None) == OK        # nothing to append
    assert ap(_p(A), 0, 100, 2, 0, None, _p(C), 5, None) == NULL
    assert ap(_p(A), 0, 100, 2, 0, _p(B + 4), _p(C), 5, None) == ALIGN
    assert ap(_p(A), 0, 100, 2, 0, _p(A + 256), _p(C), 5, None) == ALIAS  # kd inside the cache
    assert ap(_p(A), 5, 100, 2, 0, _p(B), _p(C), 5, None) == UNSUP
    at = L.vggt_descriptor_cache_attn
    # (q, cache, o, dt, capacity, H, used, nq, scale, kv_splits, ws, ws_bytes, stream)
    assert at(_p(B), _p(A), _p(O), 0, 100, 2, 0, 10, 0.0, 0, None, 0, None) == SHAPE    # nothing cached
    assert at(_p(B), _p(A), _p(O), 0, 100, 2, 101, 10, 0.0, 0, None, 0, None) == SHAPE  # used > capacity
    assert at(_p(B), _p(A), _p(A), 0, 100, 2, 50, 10, 0.0, 0, None, 0, None) == ALIAS   # o is the cache
    assert at(_p(B), _p(A), _p(O), 0, 100, 2, 50, 10, 0.0, 65, None, 0, None) == SHAPE
    assert at(_p(B), _p(A), _p(O), 0, 4000, 2, 3000, 1000, 0.0, 3, None, 0, None) == WS
    assert at(None, None, None, 0, 100, 2, 50, 0, 0.0, 0, None, 0, None) == OK          # no queries
    ch = L.vggt_descriptor_chunked_xattn
    # (q, cache, o, dt, capacity, H, S, T, Dn, chunk_frames, scale, stream)
    assert ch(_p(B), _p(A), _p(O), 0, 100, 2, 3, 8, 34, 1, 0.0, None) == SHAPE  # 3*34 > capacity
    assert ch(_p(B), _p(A), _p(O), 0, 100, 2, 3, 8, 30, 0, 0.0, None) == SHAPE  # chunk of zero frames
    assert ch(None, _p(A), _p(O), 0, 100, 2, 3, 8, 30, 1, 0.0, None) == NULL
    assert ch(_p(B), _p(A), _p(B), 0, 100, 2, 3, 8, 30, 1, 0.0, None) == ALIAS


def test_timer_arguments(L):
    # no device work: a stop without a start and bad capacities fail before any HIP call
    n = ctypes.c_int(-1)
    assert L.vggt_timer_stop(None, None, 0, ctypes.byref(n)) == SHAPE
    assert n.value == -1
    assert L.vggt_timer_start(0) == SHAPE
    assert L.vggt_timer_start((1 << 20) + 1) == SHAPE


def test_qk_norm_arguments(L):
    BF16, F32 = 0, 1
    S, T, H = 2, 40, 2
    # the LayerNorm adds nothing to the bf16 workspace; fp32 keeps normalised copies of q and k
    assert L.vggt_frame_attn_workspace(S, T, H, 2, BF16) == L.vggt_frame_attn_workspace(S, T, H, 0, BF16)
    assert L.vggt_frame_attn_workspace(S, T, H, 2, F32) >= 2 * S * T * H * 64 * 4
    assert L.vggt_global_attn_workspace(S, T, H, 1, 3, F32) == L.vggt_global_attn_workspace(S, T, H, 1, 1, F32)
    G, Bt, KG, KB = 0x700000, 0x700100, 0x700200, 0x700300
    norm = ffv.QkNorm(G, Bt, KG, KB, 1e-5)
    f = L.vggt_frame_attn_qknorm
    args = (_p(A), _p(B), _p(C), _p(O), 0, S, T, H, None, 100.0, 0.0)
    bad = ffv.QkNorm(G, None, KG, KB, 1e-5)
    assert f(*args, ctypes.byref(bad), None, 0, None) == NULL
    bad = ffv.QkNorm(G, Bt, KG, KB, 0.0)
    assert f(*args, ctypes.byref(bad), None, 0, None) == SHAPE
    bad = ffv.QkNorm(G + 2, Bt, KG, KB, 1e-5)
    assert f(*args, ctypes.byref(bad), None, 0, None) == ALIGN
    bad = ffv.QkNorm(O + 64, Bt, KG, KB, 1e-5)  # gamma inside the output
    assert f(*args, ctypes.byref(bad), _p(0x10000000), 1 << 24, None) == ALIAS
    g = L.vggt_global_attn_qknorm
    assert g(_p(A), _p(B), _p(C), _p(O), 0, S, T, H, None, 100.0, 0.0, 65, ctypes.byref(norm), None, 0,
             None) == SHAPE


def test_omega_variant_arguments(L):
    BF16, F32 = 0, 1
    S, T, Ta, E, H = 4, 1040, 1024, 5, 16
    # bf16: K tiles of the compacted key set (frame: per frame, V read in place; global: active
    # tokens plus extras, with V^T tiles)
    assert L.vggt_frame_attn_ex_workspace(S, T, Ta, H, 0, BF16) == S * H * 16 * 64 * 64 * 2
    ws = L.vggt_global_attn_ex_workspace(S, T, Ta, E, H, 1, 0, BF16)
    assert ws >= 2 * H * ((S * Ta + E + 63) // 64) * 64 * 64 * 2
    assert L.vggt_global_attn_ex_workspace(S, T, T + 1, E, H, 1, 0, BF16) == 0
    assert L.vggt_global_attn_ex_workspace(S, T, Ta, 4097, H, 1, 0, BF16) == 0
    # fp32 global always gathers the key set
    assert L.vggt_global_attn_ex_workspace(S, T, Ta, E, H, 1, 0, F32) >= 2 * (S * Ta + E) * H * 64 * 4
    g = L.vggt_global_attn_ex
    X, XK, XV, XO = 0x800000, 0x810000, 0x820000, 0x830000
    # (q, k, v, o, dt, S, T, T_active, H, xq, xk, xv, xo, n_extra, pos, base, scale, kv_splits, norm, ws, ws_bytes, st)
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 9, 1, None, None, None, None, 0, None, 100.0, 0.0, 0, None,
             None, 0, None) == SHAPE  # T_active > T
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 6, 1, _p(X), None, _p(XV), _p(XO), 2, None, 100.0, 0.0, 0, None,
             _p(0x10000000), 1 << 24, None) == NULL
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 6, 1, _p(X), _p(XK), _p(XV), _p(A), 2, None, 100.0, 0.0, 0,
             None, _p(0x10000000), 1 << 24, None) == ALIAS  # xo is q
    assert g(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 6, 1, _p(X + 8), _p(XK), _p(XV), _p(XO), 2, None, 100.0, 0.0, 0,
             None, _p(0x10000000), 1 << 24, None) == ALIGN
    f = L.vggt_frame_attn_ex
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 0, 1, None, 100.0, 0.0, None, None, 0, None) == SHAPE
    assert f(_p(A), _p(B), _p(C), _p(O), 0, 2, 8, 6, 1, None, 100.0, 0.0, None, None, 0, None) == WS


def test_backward_arguments(L):
    BF16, F32 = 0, 1
    S, T, H = 4, 100, 2
    n, tiles = S * T, (S * T + 63) // 64
    # bf16 global: four row-tile sets (K, V, Q, dO) plus two statistics rows per head; RoPE adds the
    # table and a rotated copy of K
    base = L.vggt_attn_backward_workspace(S, T, H, 1, 0, BF16)
    assert base >= 4 * H * tiles * 64 * 64 * 2 + 2 * H * tiles * 64 * 4
    assert L.vggt_attn_backward_workspace(S, T, H, 1, 1, BF16) >= base + n * H * 64 * 2 + T * 32 * 8
    assert L.vggt_attn_backward_workspace(S, T, H, 0, 0, BF16) >= 4 * S * H * 2 * 64 * 64 * 2
    assert L.vggt_attn_backward_workspace(S, T, H, 1, 1, F32) >= 4 * n * H * 64 * 4
    assert L.vggt_attn_backward_workspace(S, 0, H, 1, 0, BF16) == 0
    b = L.vggt_global_attn_backward
    Q, K, V, Ot, DO, LS, DQ, DK, DV, WSP = (0x1000000 * (i + 1) for i in range(10))
    big = 1 << 24
    args = lambda **kw: [_p(kw.get(n, d)) if d is not None else None for n, d in
                         (("q", Q), ("k", K), ("v", V), ("o", Ot), ("do", DO), ("lse", LS), ("dq", DQ), ("dk", DK),
                          ("dv", DV))]
    tail = [0, 2, 8, 1, None, 100.0, 0.0, _p(WSP), big, None]
    assert b(*args(lse=None), *tail) == NULL
    assert b(*args(dq=Q), *tail) == ALIAS             # dq is q
    assert b(*args(dk=DQ), *tail) == ALIAS            # dk is dq
    assert b(*args(dv=LS), *tail) == ALIAS            # dv is lse
    assert b(*args(lse=LS + 2), *tail) == ALIGN
    assert b(*args(), 0, 2, 8, 1, None, 100.0, 0.0, _p(WSP), 16, None) == WS
    assert b(*args(), 0, 2, 0, 1, None, 100.0, 0.0, _p(WSP), big, None) == SHAPE
    t = L.vggt_global_attn_train
    assert t(_p(A), _p(B), _p(C), _p(O), None, 0, 2, 8, 1, None, 100.0, 0.0, 0, _p(0x10000000), big, None) == NULL
    assert t(_p(A), _p(B), _p(C), _p(O), _p(A + 64), 0, 2, 8, 1, None, 100.0, 0.0, 0, _p(0x10000000), big,
             None) == ALIAS


def test_empty_calls_are_noops(L):
    """S = 0 (n = 0 / nq = 0 for the cache calls) returns OK without reading a
    pointer or touching the device; workspace queries return 0.  Global
    attention with extra tokens but no frames is rejected."""
    BF16, F32 = 0, 1
    norm = ffv.QkNorm(0x900000, 0x900100, 0x900200, 0x900300, 1e-5)
    pn = ctypes.byref(norm)
    for dt in (BF16, F32):
        assert L.vggt_attn_rope(None, dt, 0, 8, 1, None, 100.0, None) == OK
        assert L.vggt_frame_attn(None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, None, 0, None) == OK
        assert L.vggt_global_attn(None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, 0, None, 0, None) == OK
        assert L.vggt_frame_attn_qknorm(None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, pn, None, 0, None) == OK
        assert L.vggt_global_attn_qknorm(None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, 0, pn, None, 0,
                                         None) == OK
        assert L.vggt_frame_attn_ex(None, None, None, None, dt, 0, 8, 6, 1, None, 100.0, 0.0, None, None, 0,
                                    None) == OK
        assert L.vggt_global_attn_ex(None, None, None, None, dt, 0, 8, 6, 1, None, None, None, None, 0, None, 100.0,
                                     0.0, 0, None, None, 0, None) == OK
        assert L.vggt_frame_attn_train(None, None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, None, 0,
                                       None) == OK
        assert L.vggt_global_attn_train(None, None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, 0, None, 0,
                                        None) == OK
        for back in (L.vggt_frame_attn_backward, L.vggt_global_attn_backward):
            assert back(None, None, None, None, None, None, None, None, None, dt, 0, 8, 1, None, 100.0, 0.0, None,
                        0, None) == OK
        assert L.vggt_descriptor_pool(None, None, None, None, dt, 0, 14, 1, 3, 4, 2, 2, 2, None) == OK
        assert L.vggt_descriptor_xattn(None, None, None, None, dt, 0, 8, 3, 1, 0.0, 0, None, 0, None) == OK
        assert L.vggt_descriptor_cache_append(None, dt, 64, 1, 0, None, None, 0, None) == OK
        assert L.vggt_descriptor_cache_attn(None, None, None, dt, 64, 1, 1, 0, 0.0, 0, None, 0, None) == OK
        assert L.vggt_descriptor_chunked_xattn(None, None, None, dt, 64, 1, 0, 8, 3, 1, 0.0, None) == OK
        # workspace queries
        assert L.vggt_frame_attn_workspace(0, 8, 1, 1, dt) == 0
        assert L.vggt_global_attn_workspace(0, 8, 1, 0, 1, dt) == 0
        assert L.vggt_frame_attn_ex_workspace(0, 8, 6, 1, 1, dt) == 0
        assert L.vggt_global_attn_ex_workspace(0, 8, 6, 0, 1, 0, 1, dt) == 0
        assert L.vggt_descriptor_xattn_workspace(0, 8, 3, 1, 0, dt) == 0
        assert L.vggt_descriptor_cache_attn_workspace(0, 1, 1, 0, dt) == 0
        assert L.vggt_attn_backward_workspace(0, 8, 1, 1, 1, dt) == 0
        # the size checks still run first
        assert L.vggt_frame_attn(None, None, None, None, dt, 0, 0, 1, None, 100.0, 0.0, None, 0, None) == SHAPE
        assert L.vggt_global_attn(None, None, None, None, dt, 0, 8, 0, None, 100.0, 0.0, 0, None, 0, None) == SHAPE
        # extra tokens without frames
        X = _p(0x800000)
        assert L.vggt_global_attn_ex(None, None, None, None, dt, 0, 8, 6, 1, X, X, X, X, 2, None, 100.0, 0.0, 0,
                                     None, None, 0, None) == SHAPE
        assert L.vggt_global_attn_ex_workspace(0, 8, 6, 2, 1, 0, 1, dt) == 0


def test_noalloc_frame_attn_arguments(L):
    """The allocation-free frame attention rejects, before touching the device,
    shapes whose workspace exceeds its scratch array and the usual bad arguments."""
    f = L.vggt_frame_attn_noalloc
    p = ctypes.c_void_p(1 << 20)
    pos = ctypes.c_void_p(1 << 21)
    limit = 64 << 20
    assert L.vggt_frame_attn_workspace(8, 1374, 16, 1, 0) <= limit
    assert L.vggt_frame_attn_workspace(32, 1374, 16, 1, 0) > limit
    assert f(p, p, p, p, 0, 32, 1374, 16, pos, 100.0, 0.0, None) == WS
    assert f(p, p, p, p, 1, 8, 1374, 16, pos, 100.0, 0.0, None) == WS  # fp32 rotated copies: 90 MB
    assert f(p, p, p, p, 2, 8, 1374, 16, None, 100.0, 0.0, None) == UNSUP
    assert f(p, p, p, p, 0, 8, 0, 16, None, 100.0, 0.0, None) == SHAPE
    assert f(None, p, p, p, 0, 8, 1374, 16, None, 100.0, 0.0, None) == NULL
    assert f(ctypes.c_void_p((1 << 20) + 8), p, p, ctypes.c_void_p(1 << 30), 0, 8, 1374, 16, None, 100.0, 0.0,
             None) == ALIGN
    assert f(None, None, None, None, 0, 0, 1374, 16, None, 100.0, 0.0, None) == OK  # empty call
