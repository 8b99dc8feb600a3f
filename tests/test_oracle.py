"""Pins of the float64 oracle against facts fixed outside the oracle itself:
values printed on the pages (tests/golden), closed forms, invariants,
library routines and brute force on tiny inputs.  CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return np.array(rows)


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Printed worked examples
# --------------------------------------------------------------------------

def test_softmax_matches_printed_slide_example():
    """Slide deck Section V 4/10: scores (2, 1, 0.5, -1) -> (0.61, 0.22, 0.14, 0.03).
    With V = one-hot rows the attention output of one query is the softmax
    vector itself; D = 4 gives scale 1/2, so q = 4 e0 and k_j0 = s_j / 2."""
    g = _load("softmax_slide.txt")
    scores, printed = g[:, 0], g[:, 1]
    D = 4
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 4.0
    k = np.zeros((4, 1, D)); k[:, 0, 0] = scores / 2.0
    v = np.eye(4).reshape(4, 1, D)
    o = oracle.attention(q, k, v)[0, 0]
    assert np.all(np.abs(o - printed) <= 0.005 + 1e-12)
    assert abs(o.sum() - 1.0) < 1e-15
    # and the exact values against the closed form e^s / sum e^s
    np.testing.assert_allclose(o, np.exp(scores) / np.exp(scores).sum(), rtol=1e-15)


def test_rope_frequency_table_matches_printed_sinusoid_slide():
    """Slide deck Section IV 6/6 prints the first values of the base-10000
    sinusoidal encoding at pos 1..3.  The oracle's RoPE rotates pair (0,1) of
    an axis by pos*freq(k=0) and pair (2,3) by pos*freq(k=1); with d_axis = 4
    and base 10000, rotating the unit vectors e0 and e2 must reproduce
    (sin, cos, sin, cos) of the printed table.  Checked on both axes."""
    g = _load("sinusoid_slide.txt")
    D = 8  # two axes of width 4
    for axis in (0, 1):
        for row in g:
            p = int(row[0])
            pos = np.zeros((2, 2), dtype=np.int32)
            pos[:, axis] = p
            x = np.zeros((2, 1, D))
            x[0, 0, 4 * axis + 0] = 1.0   # e0 of this axis
            x[1, 0, 4 * axis + 2] = 1.0   # e2 of this axis
            y = oracle.rope(x, pos, 10000.0)
            c0, s0 = y[0, 0, 4 * axis + 0], y[0, 0, 4 * axis + 1]
            c1, s1 = y[1, 0, 4 * axis + 2], y[1, 0, 4 * axis + 3]
            got = np.array([s0, c0, s1, c1])
            assert np.all(np.abs(got - row[1:]) <= 0.005 + 1e-12), (axis, p, got, row)
            # the other axis is untouched
            other = [i for i in range(D) if i // 4 != axis]
            assert np.all(y[:, 0, other] == 0.0)
    assert oracle.rope_freq(10000.0, 4, 1) == pytest.approx(0.01, rel=1e-15)
    assert oracle.rope_freq(100.0, 32, 0) == 1.0


# --------------------------------------------------------------------------
# RoPE closed forms
# --------------------------------------------------------------------------

def test_rope_identity_at_origin_is_bitwise():
    x = workload.normal_f32(11, (7, 3, 64)).astype(np.float64)
    y = oracle.rope(x, np.zeros((7, 2), np.int32), 100.0)
    assert np.array_equal(x, y)


def test_rope_preserves_norm_and_rotates_pairs():
    r = _rng(1)
    x = r.standard_normal((50, 2, 64))
    pos = r.integers(0, 40, size=(50, 2)).astype(np.int32)
    y = oracle.rope(x, pos, 100.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # each pair keeps its own norm (a rotation of that pair only)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]),
                               rtol=1e-12, atol=1e-14)
    # explicit angle of one pair: dims (32+2k, 33+2k) rotate by col * 100^(-2k/32)
    t, h, k = 3, 1, 5
    theta = pos[t, 1] * 100.0 ** (-2 * k / 32)
    a, b = x[t, h, 32 + 2 * k], x[t, h, 33 + 2 * k]
    assert y[t, h, 32 + 2 * k] == pytest.approx(a * math.cos(theta) - b * math.sin(theta), abs=1e-13)
    assert y[t, h, 33 + 2 * k] == pytest.approx(a * math.sin(theta) + b * math.cos(theta), abs=1e-13)


def test_rope_relative_position_property():
    """<rope(q, p), rope(k, p')> = <rope(q, p - p'), k> for every head vector."""
    r = _rng(2)
    q = r.standard_normal((20, 1, 64))
    k = r.standard_normal((20, 1, 64))
    p = r.integers(-30, 30, size=(20, 2)).astype(np.int32)
    pp = r.integers(-30, 30, size=(20, 2)).astype(np.int32)
    lhs = np.sum(oracle.rope(q, p, 100.0) * oracle.rope(k, pp, 100.0), axis=-1)
    rhs = np.sum(oracle.rope(q, (p - pp).astype(np.int32), 100.0) * k, axis=-1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_attention_invariant_under_common_position_shift():
    """Shifting every token's (row, col) by one constant leaves attention
    unchanged (scores depend on position differences only)."""
    wl = workload.Workload("t", 9, S=2, gh=3, gw=4, n_special=2, patch_begin=2, H=2, D=64)
    q, k, v = wl.qkv_f32()
    pos = wl.positions()
    a = oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos)
    b = oracle.global_attn(q, k, v, wl.S, wl.T, pos=(pos + np.array([7, -3], np.int32)).astype(np.int32))
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Attention closed forms
# --------------------------------------------------------------------------

def test_identical_keys_average_values():
    r = _rng(3)
    q = r.standard_normal((5, 2, 64))
    k = np.repeat(r.standard_normal((1, 2, 64)), 9, axis=0)
    v = r.standard_normal((9, 2, 64))
    o = oracle.attention(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_value():
    r = _rng(4)
    D = 64
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    k = r.standard_normal((12, 1, D)) * 0.01
    k[7, 0, 0] = 8.0 * 60.0      # score margin >= 50 after the 1/8 scale
    v = r.standard_normal((12, 1, D))
    o = oracle.attention(q, k, v)
    np.testing.assert_allclose(o[0, 0], v[7, 0], rtol=0, atol=12 * math.exp(-50) * 10)


def test_single_key_and_constant_values():
    r = _rng(5)
    q = r.standard_normal((4, 3, 64))
    k1 = r.standard_normal((1, 3, 64))
    v1 = r.standard_normal((1, 3, 64))
    np.testing.assert_allclose(oracle.attention(q, k1, v1), np.broadcast_to(v1, (4, 3, 64)), rtol=1e-15)
    k = r.standard_normal((10, 3, 64))
    v = np.full((10, 3, 64), 0.3125)
    np.testing.assert_allclose(oracle.attention(q, k, v), 0.3125, rtol=1e-14)


def test_softmax_against_library_routine():
    """With V = identity rows (nk = D) the output row is softmax(scale q K^T),
    computed here by scipy.special.softmax."""
    r = _rng(6)
    D = 16
    q = r.standard_normal((6, 2, D)) * 3
    k = r.standard_normal((D, 2, D))
    v = np.repeat(np.eye(D)[:, None, :], 2, axis=1)
    o = oracle.attention(q, k, v, scale=0.37)
    for h in range(2):
        ref = scipy.special.softmax(0.37 * q[:, h, :] @ k[:, h, :].T, axis=-1)
        np.testing.assert_allclose(o[:, h, :], ref, rtol=1e-13, atol=1e-16)


def test_key_shift_invariance():
    """K -> K + 1 c^T changes every score of a row by the same q.c."""
    r = _rng(7)
    q = r.standard_normal((8, 2, 64))
    k = r.standard_normal((30, 2, 64))
    v = r.standard_normal((30, 2, 64))
    c = r.standard_normal((1, 2, 64))
    np.testing.assert_allclose(oracle.attention(q, k, v), oracle.attention(q, k + c, v), rtol=1e-11, atol=1e-13)


def test_linearity_in_values():
    r = _rng(8)
    q = r.standard_normal((8, 1, 64))
    k = r.standard_normal((30, 1, 64))
    v = r.standard_normal((30, 1, 64))
    A = r.standard_normal((64, 64))
    b = r.standard_normal(64)
    lhs = oracle.attention(q, k, (v[:, 0] @ A + b)[:, None, :])
    rhs = oracle.attention(q, k, v)[:, 0] @ A + b
    np.testing.assert_allclose(lhs[:, 0], rhs, rtol=1e-10, atol=1e-11)


def test_heads_are_independent():
    r = _rng(9)
    q = r.standard_normal((6, 3, 64))
    k = r.standard_normal((11, 3, 64))
    v = r.standard_normal((11, 3, 64))
    o = oracle.attention(q, k, v)
    for h in range(3):
        oh = oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1])
        np.testing.assert_array_equal(o[:, h:h + 1], oh)


def test_token_and_kv_permutation():
    """Global attention without RoPE: permuting queries permutes outputs;
    permuting keys and values together changes nothing."""
    r = _rng(10)
    q = r.standard_normal((13, 2, 64))
    k = r.standard_normal((17, 2, 64))
    v = r.standard_normal((17, 2, 64))
    o = oracle.attention(q, k, v)
    pq = r.permutation(13)
    pk = r.permutation(17)
    np.testing.assert_allclose(oracle.attention(q[pq], k, v), o[pq], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.attention(q, k[pk], v[pk]), o, rtol=1e-12, atol=1e-14)


def test_frame_permutation_equivariance_with_rope():
    """Positions are within-frame only, so permuting whole frames permutes
    the outputs of both frame and global attention, RoPE on."""
    wl = workload.Workload("t", 8, S=3, gh=3, gw=4, n_special=2, patch_begin=2, H=2, D=64)
    q, k, v = wl.qkv_f32()
    pos = wl.positions()
    perm = np.array([2, 0, 1])
    for fn in (oracle.frame_attn, oracle.global_attn):
        o = fn(q, k, v, wl.S, wl.T, pos=pos).reshape(wl.S, wl.T, 2, 64)
        op = fn(q[perm], k[perm], v[perm], wl.S, wl.T, pos=pos).reshape(wl.S, wl.T, 2, 64)
        np.testing.assert_allclose(op, o[perm], rtol=1e-12, atol=1e-14)


def _einsum_attention(q, k, v, scale):
    # brute force on tiny inputs: full score tensor, library exp/sum
    s = np.einsum("qhd,khd->hqk", q, k) * scale
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hqk,khd->qhd", p, v)


def _einsum_rope(x, pos, base):
    # rotation written as a complex multiply per (2k, 2k+1) pair
    n, H, D = x.shape
    half = D // 2
    out = np.empty_like(x)
    for a in range(2):
        z = x[..., a * half:(a + 1) * half:2] + 1j * x[..., a * half + 1:(a + 1) * half:2]
        freqs = base ** (-2.0 * np.arange(half // 2) / half)
        rot = np.exp(1j * pos[:, a, None].astype(np.float64) * freqs[None, :])
        z = z * rot[:, None, :]
        out[..., a * half:(a + 1) * half:2] = z.real
        out[..., a * half + 1:(a + 1) * half:2] = z.imag
    return out


@pytest.mark.parametrize("S,H", [(1, 1), (2, 2), (3, 2)])
def test_brute_force_tiny(S, H):
    wl = workload.Workload("t", 7, S=S, gh=3, gw=4, n_special=2, patch_begin=2, H=H, D=64)
    q, k, v = (x.astype(np.float64) for x in wl.qkv_f32())
    pos = wl.positions()
    T = wl.T
    pt = np.tile(pos, (S, 1))
    qr = _einsum_rope(q.reshape(S * T, H, 64), pt, 100.0)
    kr = _einsum_rope(k.reshape(S * T, H, 64), pt, 100.0)
    vv = v.reshape(S * T, H, 64)
    g_ref = _einsum_attention(qr, kr, vv, 0.125)
    np.testing.assert_allclose(oracle.global_attn(q, k, v, S, T, pos=pos), g_ref, rtol=1e-11, atol=1e-13)
    f_ref = np.concatenate([_einsum_attention(qr[s * T:(s + 1) * T], kr[s * T:(s + 1) * T], vv[s * T:(s + 1) * T],
                                              0.125) for s in range(S)])
    np.testing.assert_allclose(oracle.frame_attn(q, k, v, S, T, pos=pos), f_ref, rtol=1e-11, atol=1e-13)


def test_frame_vs_global_consistency_and_row_sampling():
    wl = workload.Workload("t", 6, S=3, gh=4, gw=4, n_special=5, patch_begin=5, H=2, D=64)
    q, k, v = wl.qkv_bf16()
    pos = wl.positions()
    T = wl.T
    f = oracle.frame_attn(q, k, v, wl.S, T, pos=pos)
    for s in range(wl.S):
        g1 = oracle.global_attn(q[s:s + 1], k[s:s + 1], v[s:s + 1], 1, T, pos=pos)
        np.testing.assert_array_equal(f[s * T:(s + 1) * T], g1)
    rows = np.array([0, 4, T, 2 * T + 3, 3 * T - 1])
    np.testing.assert_array_equal(oracle.frame_attn(q, k, v, wl.S, T, pos=pos, rows=rows), f[rows])
    g = oracle.global_attn(q, k, v, wl.S, T, pos=pos)
    np.testing.assert_array_equal(oracle.global_attn(q, k, v, wl.S, T, pos=pos, rows=rows), g[rows])


# --------------------------------------------------------------------------
# Per-head Q/K LayerNorm
# --------------------------------------------------------------------------

def _torch_layer_norm(x, g, b, eps):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return torch.nn.functional.layer_norm(t, (x.shape[-1],), torch.from_numpy(np.asarray(g, np.float64)),
                                          torch.from_numpy(np.asarray(b, np.float64)), eps).numpy()


def test_layer_norm_against_library_routine():
    r = _rng(40)
    x = r.standard_normal((7, 3, 64)) * 3.0 + 1.5
    g, b = r.standard_normal(64), r.standard_normal(64)
    for eps in (1e-5, 0.5):
        np.testing.assert_allclose(oracle.layer_norm(x, g, b, eps), _torch_layer_norm(x, g, b, eps),
                                   rtol=1e-12, atol=1e-13)


def test_layer_norm_closed_forms():
    r = _rng(41)
    g, b = r.standard_normal(64), r.standard_normal(64)
    # a constant head vector has no deviation: the output is beta
    np.testing.assert_array_equal(oracle.layer_norm(np.full((2, 2, 64), 3.25), g, b, 1e-5)[0, 1], b)
    x = r.standard_normal((5, 2, 64))
    ones, zeros = np.ones(64), np.zeros(64)
    y = oracle.layer_norm(x, ones, zeros, 0.0)
    np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(axis=-1), 1.0, rtol=1e-13)
    # invariant under positive scaling and shifting of the input (eps = 0)
    np.testing.assert_allclose(oracle.layer_norm(2.5 * x - 7.0, g, b, 0.0), oracle.layer_norm(x, g, b, 0.0),
                               rtol=1e-12, atol=1e-12)
    # eps shrinks the normalised deviation by sqrt(var / (var + eps))
    var = x.var(axis=-1, keepdims=True)
    y_eps = oracle.layer_norm(x, ones, zeros, 0.3)
    np.testing.assert_allclose(y_eps, y * np.sqrt(var / (var + 0.3)), rtol=1e-12, atol=1e-14)


def test_attention_with_qk_norm_brute_force():
    wl = workload.Workload("t", 11, S=2, gh=3, gw=4, n_special=2, patch_begin=2, H=2, D=64)
    q, k, v = (x.astype(np.float64) for x in wl.qkv_f32())
    r = _rng(42)
    qn = (r.standard_normal(64), r.standard_normal(64), 1e-5)
    kn = (r.standard_normal(64), r.standard_normal(64), 1e-5)
    pos = wl.positions()
    S, T = wl.S, wl.T
    pt = np.tile(pos, (S, 1))
    qr = _einsum_rope(_torch_layer_norm(q.reshape(S * T, 2, 64), *qn), pt, 100.0)
    kr = _einsum_rope(_torch_layer_norm(k.reshape(S * T, 2, 64), *kn), pt, 100.0)
    vv = v.reshape(S * T, 2, 64)
    got = oracle.global_attn(q, k, v, S, T, pos=pos, q_norm=qn, k_norm=kn)
    np.testing.assert_allclose(got, _einsum_attention(qr, kr, vv, 0.125), rtol=1e-11, atol=1e-13)
    f = oracle.frame_attn(q, k, v, S, T, pos=pos, q_norm=qn, k_norm=kn)
    ref = np.concatenate([_einsum_attention(qr[s * T:(s + 1) * T], kr[s * T:(s + 1) * T], vv[s * T:(s + 1) * T],
                                            0.125) for s in range(S)])
    np.testing.assert_allclose(f, ref, rtol=1e-11, atol=1e-13)


def test_qk_norm_with_zero_gain_makes_keys_identical():
    # gamma = 0 maps every key to beta: no RoPE, so the output averages the values
    wl = workload.Workload("t", 12, S=2, gh=3, gw=3, n_special=1, patch_begin=0, H=1, D=64)
    q, k, v = wl.qkv_bf16()
    beta = _rng(43).standard_normal(64)
    got = oracle.global_attn(q, k, v, wl.S, wl.T, k_norm=(np.zeros(64), beta, 1e-5))
    vm = oracle.to_f64(v).reshape(-1, 1, 64).mean(axis=0)
    np.testing.assert_allclose(got, np.broadcast_to(vm, got.shape), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# VGGT-Omega variants: register-free blocks and global-only extra tokens
# --------------------------------------------------------------------------

def _omega_tiny(seed, S=2, gh=3, gw=3, n_reg=2, E=3, H=2):
    wl = workload.Workload("t", seed, S=S, gh=gh, gw=gw, n_special=n_reg, patch_begin=0, H=H, D=64)
    q, k, v = (x.astype(np.float64) for x in wl.qkv_f32())
    x = [workload.normal_f32(0xE0 + seed * 8 + i, (E, H, 64)).astype(np.float64) for i in range(3)]
    return wl, q, k, v, x


def test_global_ex_brute_force_with_registers_out_and_extras():
    wl, q, k, v, (xq, xk, xv) = _omega_tiny(13)
    S, T, Ta, H = wl.S, wl.T, wl.gh * wl.gw, wl.H
    pos = wl.positions()
    pt = np.concatenate([np.tile(pos[:Ta], (S, 1)), np.zeros((3, 2), dtype=np.int32)])
    qs = np.concatenate([q[:, :Ta].reshape(-1, H, 64), xq])
    ks = np.concatenate([k[:, :Ta].reshape(-1, H, 64), xk])
    vs = np.concatenate([v[:, :Ta].reshape(-1, H, 64), xv])
    ref = _einsum_attention(_einsum_rope(qs, pt, 100.0), _einsum_rope(ks, pt, 100.0), vs, 0.125)
    of, ox = oracle.global_attn_ex(q, k, v, S, T, Ta, xq, xk, xv, pos=pos)
    np.testing.assert_allclose(of.reshape(-1, H, 64), ref[:S * Ta], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(ox, ref[S * Ta:], rtol=1e-11, atol=1e-13)
    rows = np.array([0, Ta, S * Ta - 1, S * Ta, S * Ta + 2])
    np.testing.assert_array_equal(oracle.global_attn_ex(q, k, v, S, T, Ta, xq, xk, xv, pos=pos, rows=rows),
                                  np.concatenate([of.reshape(-1, H, 64), ox])[rows])
    # register rows take no part: changing them changes nothing
    k2, v2 = k.copy(), v.copy()
    k2[:, Ta:] += 5.0
    v2[:, Ta:] -= 2.0
    of2, ox2 = oracle.global_attn_ex(q, k2, v2, S, T, Ta, xq, xk, xv, pos=pos)
    np.testing.assert_array_equal(of2, of)
    np.testing.assert_array_equal(ox2, ox)
    # frame variant: the active tokens of each frame only
    fe = oracle.frame_attn_ex(q, k, v, S, T, Ta, pos=pos)
    pf = np.tile(pos[:Ta], (S, 1))
    qr, kr = _einsum_rope(q[:, :Ta].reshape(-1, H, 64), pf, 100.0), _einsum_rope(k[:, :Ta].reshape(-1, H, 64), pf, 100.0)
    vr = v[:, :Ta].reshape(-1, H, 64)
    fref = np.concatenate([_einsum_attention(qr[s * Ta:(s + 1) * Ta], kr[s * Ta:(s + 1) * Ta], vr[s * Ta:(s + 1) * Ta],
                                             0.125) for s in range(S)])
    np.testing.assert_allclose(fe.reshape(-1, H, 64), fref, rtol=1e-11, atol=1e-13)


def test_global_ex_reduces_to_global_attention():
    wl, q, k, v, _ = _omega_tiny(14)
    pos = wl.positions()
    of, ox = oracle.global_attn_ex(q, k, v, wl.S, wl.T, wl.T, None, None, None, pos=pos)
    assert ox.shape[0] == 0
    np.testing.assert_array_equal(of.reshape(wl.N, wl.H, 64), oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos))


def test_global_ex_extra_tokens_are_keys_and_queries_of_everything():
    wl, q, k, v, (xq, xk, xv) = _omega_tiny(15, H=1)
    S, T, Ta = wl.S, wl.T, wl.gh * wl.gw
    # a dominant extra key: every query selects that extra token's value
    xk2 = xk.copy()
    xk2[1] = 0.0
    qpos = np.abs(q).max() + 1.0
    q2 = np.zeros_like(q) + qpos
    xq2 = np.zeros_like(xq) + qpos
    xk2[1, :, :] = 40.0
    of, ox = oracle.global_attn_ex(q2, k, v, S, T, Ta, xq2, xk2, xv)
    np.testing.assert_allclose(of, np.broadcast_to(xv[1], of.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ox, np.broadcast_to(xv[1], ox.shape), rtol=0, atol=1e-12)
    # identical keys: each output is the mean of the values of all active and extra tokens
    zk, zx = np.zeros_like(k), np.zeros_like(xk)
    of, ox = oracle.global_attn_ex(q, zk, v, S, T, Ta, xq, zx, xv)
    mean = np.concatenate([v[:, :Ta].reshape(-1, 1, 64), xv]).mean(axis=0)
    np.testing.assert_allclose(of, np.broadcast_to(mean, of.shape), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ox, np.broadcast_to(mean, ox.shape), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Attention gradients
# --------------------------------------------------------------------------

def _fd_grads(f, xs, dout, eps=1e-5):
    """Central differences of L = sum(dout * f(*xs)) with respect to every input element."""
    grads = []
    for n in range(len(xs)):
        g = np.zeros_like(xs[n])
        it = np.nditer(xs[n], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in xs]
            minus = [x.copy() for x in xs]
            plus[n][idx] += eps
            minus[n][idx] -= eps
            g[idx] = (np.sum(dout * f(*plus)) - np.sum(dout * f(*minus))) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("frame", [False, True])
def test_backward_matches_finite_differences_with_rope(frame):
    r = _rng(60 + frame)
    S, T, H, D = 2, 3, 1, 8
    q, k, v = (r.standard_normal((S, T, H, D)) for _ in range(3))
    dout = r.standard_normal((S * T, H, D))
    pos = np.array([[0, 0], [1, 2], [3, 1]], dtype=np.int32)
    fwd = oracle.frame_attn if frame else oracle.global_attn
    bwd = oracle.frame_attn_backward if frame else oracle.global_attn_backward
    fd = _fd_grads(lambda a, b, c: fwd(a, b, c, S, T, pos=pos, base=100.0), [q, k, v], dout.reshape(S * T, H, D))
    dq, dk, dv, _ = bwd(q, k, v, dout, S, T, pos=pos, base=100.0)
    for got, ref, name in ((dq, fd[0], "dq"), (dk, fd[1], "dk"), (dv, fd[2], "dv")):
        np.testing.assert_allclose(got, ref.reshape(got.shape), rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_against_torch_autograd():
    import torch
    r = _rng(62)
    nq, nk, H, D = 7, 9, 2, 64
    q, dout = r.standard_normal((nq, H, D)), r.standard_normal((nq, H, D))
    k, v = r.standard_normal((nk, H, D)), r.standard_normal((nk, H, D))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = torch.einsum("qhd,khd->hqk", tq, tk) * 0.125
    o = torch.einsum("hqk,khd->qhd", torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(dout))
    dq, dk, dv, lse = oracle.attention_backward(q, k, v, dout)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).T.detach().numpy(), rtol=1e-13)


def test_backward_closed_forms():
    r = _rng(63)
    nq, nk, H, D = 6, 5, 2, 16
    q, dout = r.standard_normal((nq, H, D)), r.standard_normal((nq, H, D))
    k, v = r.standard_normal((nk, H, D)), r.standard_normal((nk, H, D))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, dout)
    # every softmax row's gradient sums to zero, so the key gradients cancel
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-13)
    # every probability row sums to one, so the value gradients add up to dout
    np.testing.assert_allclose(dv.sum(axis=0), dout.sum(axis=0), rtol=1e-12, atol=1e-13)
    # one key: the output is that value whatever q and k are
    dq1, dk1, dv1, _ = oracle.attention_backward(q, k[:1], v[:1], dout)
    np.testing.assert_allclose(dq1, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk1, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv1[0], dout.sum(axis=0), rtol=1e-13)
    # sampled query rows and key rows are the corresponding rows of the full result
    rows, cols = np.array([5, 0, 3]), np.array([4, 1])
    sq, sk, sv, _ = oracle.attention_backward(q, k, v, dout, rows=rows, cols=cols)
    np.testing.assert_array_equal(sq, dq[rows])
    np.testing.assert_array_equal(sk, dk[cols])
    np.testing.assert_array_equal(sv, dv[cols])


# --------------------------------------------------------------------------
# Descriptor pooling and cross-attention
# --------------------------------------------------------------------------

def _brute_pool(x, gh, gw, pb, ph, pw):
    S, T, H, D = x.shape
    spec = [t for t in range(T) if not (pb <= t < pb + gh * gw)]
    out = []
    for s in range(S):
        toks = [x[s, t] for t in spec]
        grid = x[s, pb:pb + gh * gw].reshape(gh, gw, H, D)
        for a in range(0, gh, ph):
            for b in range(0, gw, pw):
                toks.append(grid[a:a + ph, b:b + pw].reshape(-1, H, D).mean(axis=0))
        out.append(np.stack(toks))
    return np.stack(out)


def test_descriptor_count():
    assert oracle.descriptor_count(1374, 37, 37, 2, 2) == 366
    assert oracle.descriptor_count(1040, 32, 32, 2, 2) == 16 + 256
    assert oracle.descriptor_count(261, 16, 16, 1, 1) == 261


@pytest.mark.parametrize("gh,gw,pb,ns,ph,pw", [(5, 7, 3, 3, 2, 2), (4, 4, 0, 2, 2, 2), (3, 5, 1, 1, 3, 2),
                                               (6, 6, 2, 2, 1, 1)])
def test_pool_brute_force(gh, gw, pb, ns, ph, pw):
    r = _rng(gh * 100 + gw)
    T = gh * gw + ns
    x = r.standard_normal((2, T, 2, 8))
    got = oracle.descriptor_pool(x, 2, T, gh, gw, pb, ph, pw)
    np.testing.assert_allclose(got, _brute_pool(x, gh, gw, pb, ph, pw), rtol=1e-14, atol=1e-15)
    if ph == pw == 1:
        # identity up to moving the specials in front
        spec = [t for t in range(T) if not (pb <= t < pb + gh * gw)]
        order = spec + list(range(pb, pb + gh * gw))
        np.testing.assert_array_equal(got, x[:, order])


def test_pool_constant_and_ceil_edges():
    S, gh, gw, pb = 1, 37, 37, 5
    T = gh * gw + 5
    x = np.full((S, T, 1, 4), 2.5)
    np.testing.assert_array_equal(oracle.descriptor_pool(x, S, T, gh, gw, pb, 2, 2), 2.5)
    r = _rng(12)
    x = r.standard_normal((S, T, 1, 4))
    out = oracle.descriptor_pool(x, S, T, gh, gw, pb, 2, 2)
    grid = x[0, pb:pb + gh * gw].reshape(gh, gw, 1, 4)
    # corner cell (18, 18) covers only grid cell (36, 36)
    np.testing.assert_array_equal(out[0, 5 + 18 * 19 + 18], grid[36, 36])
    # last-column cell (0, 18) averages the two cells (0,36), (1,36)
    np.testing.assert_allclose(out[0, 5 + 18], (grid[0, 36] + grid[1, 36]) / 2, rtol=1e-15)
    # an interior cell averages four
    np.testing.assert_allclose(out[0, 5 + 19 + 1], grid[2:4, 2:4].mean(axis=(0, 1)), rtol=1e-15)
    # specials come first, unchanged
    np.testing.assert_array_equal(out[0, :5], x[0, :5])


def test_xattn_with_unit_window_equals_global_attention():
    wl = workload.Workload("t", 5, S=2, gh=3, gw=3, n_special=2, patch_begin=2, H=2, D=64)
    q, k, v = wl.qkv_bf16()
    T = wl.T
    kd = oracle.descriptor_pool(k, wl.S, T, 3, 3, 2, 1, 1)
    vd = oracle.descriptor_pool(v, wl.S, T, 3, 3, 2, 1, 1)
    # same key set up to a permutation inside each frame
    np.testing.assert_allclose(oracle.descriptor_xattn(q, kd, vd), oracle.global_attn(q, k, v, wl.S, T),
                               rtol=1e-12, atol=1e-14)


def _masked_einsum_attention(q, k, v, allowed, scale):
    # brute force with an explicit [query, key] visibility matrix
    s = np.einsum("qhd,khd->hqk", q, k) * scale
    s = np.where(allowed[None], s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hqk,khd->qhd", p, v)


@pytest.mark.parametrize("S,F", [(5, 2), (4, 1), (3, 3), (3, 7)])
def test_stream_xattn_brute_force(S, F):
    wl = workload.Workload("t", 8, S=S, gh=3, gw=3, n_special=2, patch_begin=1, H=2, D=64)
    q, k, v = wl.qkv_bf16()
    T = wl.T
    kd = oracle.descriptor_pool(k, S, T, 3, 3, 1, 2, 2)
    vd = oracle.descriptor_pool(v, S, T, 3, 3, 1, 2, 2)
    Dn = kd.shape[1]
    q_frame = np.repeat(np.arange(S), T)
    k_frame = np.repeat(np.arange(S), Dn)
    # a query of frame f sees the descriptors of frames before the end of f's chunk
    allowed = k_frame[None, :] < ((q_frame // F + 1) * F)[:, None]
    ref = _masked_einsum_attention(oracle.to_f64(q).reshape(S * T, 2, 64), kd.reshape(-1, 2, 64),
                                   vd.reshape(-1, 2, 64), allowed, 0.125)
    got = oracle.descriptor_stream_xattn(q, kd, vd, F)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)
    rows = np.array([0, T - 1, T, S * T - 1])
    np.testing.assert_array_equal(oracle.descriptor_stream_xattn(q, kd, vd, F, rows=rows), got[rows])
    if F >= S:
        # one chunk holds every frame: the single-forward descriptor attention
        np.testing.assert_array_equal(got, oracle.descriptor_xattn(q, kd, vd))


def test_stream_xattn_is_causal_over_chunks_and_averages_prefix():
    S, F = 5, 2
    wl = workload.Workload("t", 9, S=S, gh=4, gw=4, n_special=1, patch_begin=0, H=1, D=64)
    q, k, v = wl.qkv_bf16()
    T = wl.T
    kd = oracle.descriptor_pool(k, S, T, 4, 4, 0, 2, 2)
    vd = oracle.descriptor_pool(v, S, T, 4, 4, 0, 2, 2)
    Dn = kd.shape[1]
    base = oracle.descriptor_stream_xattn(q, kd, vd, F)
    # changing the frames of the last chunk leaves every earlier chunk unchanged
    kd2, vd2 = kd.copy(), vd.copy()
    kd2[4] += 3.0
    vd2[4] -= 1.0
    alt = oracle.descriptor_stream_xattn(q, kd2, vd2, F)
    np.testing.assert_array_equal(alt[:4 * T], base[:4 * T])
    assert np.abs(alt[4 * T:] - base[4 * T:]).max() > 1e-3
    # identical (zero) keys: each chunk's output is the mean of the cached value rows
    zero = np.zeros_like(kd)
    got = oracle.descriptor_stream_xattn(q, zero, vd, F)
    for c, f_end in enumerate((2, 4, 5)):
        mean = vd[:f_end].reshape(f_end * Dn, 1, 64).mean(axis=0)
        rows = slice(c * F * T, min(S, (c + 1) * F) * T)
        np.testing.assert_allclose(got[rows], np.broadcast_to(mean, got[rows].shape), rtol=1e-13, atol=1e-15)


def test_stream_xattn_first_chunk_of_one_frame_is_frame_attention():
    # unit pooling window and one frame per chunk: chunk 0 attends to frame 0's own tokens
    wl = workload.Workload("t", 10, S=3, gh=3, gw=4, n_special=2, patch_begin=2, H=2, D=64)
    q, k, v = wl.qkv_bf16()
    T = wl.T
    kd = oracle.descriptor_pool(k, wl.S, T, 3, 4, 2, 1, 1)
    vd = oracle.descriptor_pool(v, wl.S, T, 3, 4, 2, 1, 1)
    got = oracle.descriptor_stream_xattn(q, kd, vd, 1)
    np.testing.assert_allclose(got[:T], oracle.frame_attn(q, k, v, wl.S, T)[:T], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Input generator
# --------------------------------------------------------------------------

def test_splitmix64_reference_outputs_and_normals():
    # first outputs of SplitMix64 seeded with 0 (published reference stream)
    assert [int(x) for x in workload.splitmix64(0, 0, 2)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4]
    z = workload.normal_f64(123, 400001)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert np.array_equal(z[:1001], workload.normal_f64(123, 1001))
    b = workload.f32_to_bf16_bits(np.array([1.0, 1.00390625, 1.01171875, -2.0, 3.0e-3], np.float32))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> up to 1+2^-6
    np.testing.assert_array_equal(workload.bf16_bits_to_f32(b)[:4], [1.0, 1.0, 1.015625, -2.0])


# --------------------------------------------------------------------------
# Sensitivity of the GPU parity bars (tests/checks.py)
# --------------------------------------------------------------------------

def test_bf16_bars_see_a_lost_key_tile_at_full_size():
    """Global attention at 32 frames of 518x518 (N = 43968, RoPE base 100), on
    every 400th query row.  A result that lost the last 64-key tile, rounded to
    bf16 like a kernel output, passes the absolute bars (max 2e-2, mean 2e-3)
    but fails the scale-aware ones; the complete result rounded to bf16 passes
    all of them."""
    import checks

    wl = workload.WORKLOADS["vggt-518-s32"]
    q, k, v = wl.qkv_bf16()
    H = wl.H
    pos = np.tile(wl.positions(), (wl.S, 1))
    qr = oracle.rope(q.reshape(wl.N, H, 64), pos, 100.0)
    kr = oracle.rope(k.reshape(wl.N, H, 64), pos, 100.0)
    vf = oracle.to_f64(v).reshape(wl.N, H, 64)
    rows = np.arange(0, wl.N, 400)
    ref = oracle.attention(qr, kr, vf, rows=rows)
    lost = oracle.attention(qr, kr[:-64], vf[:-64], rows=rows)

    def as_bf16(x):
        return oracle.to_f64(workload.f32_to_bf16_bits(x.astype(np.float32))).reshape(x.shape)

    e_lost = checks.bf16_errors(as_bf16(lost), ref)
    e_full = checks.bf16_errors(as_bf16(ref), ref)
    assert checks.bf16_absolute_ok(e_lost), e_lost  # the absolute bars alone accept it ...
    assert not checks.bf16_ok(e_lost), e_lost  # ... the scale-aware bars reject it
    assert e_lost["nrmse"] > 2 * checks.BF16_NRMSE, e_lost
    assert checks.bf16_ok(e_full) and e_full["nrmse"] < 0.2 * checks.BF16_NRMSE, e_full


def test_bf16_bars_sit_between_input_noise_and_plausible_bugs():
    """Noise-floor calibration on global attention at 4 frames of 224x224 (N = 1044, RoPE
    base 100), every row: the exact result rounded to bf16 and the result of inputs with one
    element moved by one bf16 ulp pass the bars with room to spare; a kernel that forgot
    the log2(e) factor of its exp2 scores, one that scaled by 1/d instead of 1/sqrt(d), and
    ones that left a single rotation pair unrotated (highest row frequency, highest column
    frequency, lowest row frequency) all fail them."""
    import checks

    wl = workload.WORKLOADS["vggt-224-s4"]
    q, k, v = wl.qkv_bf16()
    S, T, H, N = wl.S, wl.T, wl.H, wl.N
    pos_grid = wl.positions()
    pos = np.tile(pos_grid, (S, 1))
    ref = oracle.global_attn(q, k, v, S, T, pos=pos_grid)

    def as_bf16(x):
        return oracle.to_f64(workload.f32_to_bf16_bits(x.astype(np.float32))).reshape(x.shape)

    e_floor = checks.bf16_errors(as_bf16(ref), ref)
    assert checks.bf16_ok(e_floor) and e_floor["nrmse"] < 0.2 * checks.BF16_NRMSE, e_floor
    q1 = q.copy()
    q1[0, 7, 0, 5] += 1  # one bf16 ulp on one element
    e_ulp = checks.bf16_errors(as_bf16(oracle.global_attn(q1, k, v, S, T, pos=pos_grid)), ref)
    assert checks.bf16_ok(e_ulp) and e_ulp["nrmse"] < 0.2 * checks.BF16_NRMSE, e_ulp

    for scale in (0.125 / np.log2(np.e), 1.0 / 64):
        e = checks.bf16_errors(as_bf16(oracle.global_attn(q, k, v, S, T, pos=pos_grid, scale=scale)), ref)
        assert not checks.bf16_ok(e), (scale, e)

    qf, kf = oracle.to_f64(q).reshape(N, H, 64), oracle.to_f64(k).reshape(N, H, 64)
    qr, kr = oracle.rope(q.reshape(N, H, 64), pos, 100.0), oracle.rope(k.reshape(N, H, 64), pos, 100.0)
    vf = oracle.to_f64(v).reshape(N, H, 64)
    for d in (2, 34, 30):
        q2, k2 = qr.copy(), kr.copy()
        q2[..., d:d + 2] = qf[..., d:d + 2]
        k2[..., d:d + 2] = kf[..., d:d + 2]
        e = checks.bf16_errors(as_bf16(oracle.attention(q2, k2, vf)), ref.reshape(N, H, 64))
        assert not checks.bf16_ok(e), (d, e)
