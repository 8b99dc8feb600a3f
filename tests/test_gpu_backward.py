"""GPU parity of the training forward (log-normaliser) and of the attention
gradients (dQ, dK, dV; frame and global, RoPE on and off) against the float64
oracle.

Bars.  fp32 debug mode: NRMSE <= 1e-5 for every tensor.  bf16: the
gradients pass through more roundings than the forward output (rotated and
scaled Q/K operands, the probabilities and the score gradients are each
rounded to bf16, relative 2^-9, before their products; the output is rounded
once more), so they are compared relative to their own scale: NRMSE <= 1e-2
and max |gpu - oracle| <= 5e-2 * max |oracle| per tensor.  The log-normaliser
is fp32 from fp32 sums of bf16-rounded probabilities: max |delta| <= 1e-2."""
import numpy as np
import pytest
import torch

import feed_forward_view_amd as ffv
import oracle
import workload
from test_gpu_parity import dev, sample_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ffv.lib()
    yield
    torch.cuda.synchronize()


def _nrmse(got, ref):
    return float(np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))


def check_grad(got, ref, label, bf16):
    got = got.reshape(ref.shape)
    e = _nrmse(got, ref)
    mx = float(np.abs(got - ref).max())
    print(f"{label}: nrmse {e:.3e} max_abs {mx:.3e} (ref max {np.abs(ref).max():.3e})")
    assert np.isfinite(got).all(), label
    if bf16:
        assert e <= 1e-2 and mx <= 5e-2 * float(np.abs(ref).max()), label
    else:
        assert e <= 1e-5, label


def _dout(seed, shape, dtype):
    return (workload.normal_bf16 if dtype == torch.bfloat16 else workload.normal_f32)(seed, shape)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rope", [True, False])
@pytest.mark.parametrize("glob", [True, False])
def test_backward_small_full(dtype, rope, glob):
    wl = workload.Workload("t", 61, S=3, gh=9, gw=9, n_special=5, patch_begin=5, H=2)
    S, T, H = wl.S, wl.T, wl.H
    q, k, v = wl.qkv_bf16() if dtype == torch.bfloat16 else wl.qkv_f32()
    g = _dout(0xD0D0, (S, T, H, 64), dtype)
    pos = wl.positions() if rope else None
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    pd = torch.from_numpy(pos).to(dev()) if rope else None
    bf16 = dtype == torch.bfloat16
    tag = f"{'global' if glob else 'frame'} {'bf16' if bf16 else 'f32'} rope={rope}"
    if glob:
        o, lse = ffv.vggt_global_attn_train(qd, kd, vd, pos_yx=pd)
        dq, dk, dv = ffv.vggt_global_attn_backward(qd, kd, vd, o, gd, lse, pos_yx=pd)
        rq, rk, rv, rl = oracle.global_attn_backward(q, k, v, g, S, T, pos=pos)
    else:
        o, lse = ffv.vggt_frame_attn_train(qd, kd, vd, pos_yx=pd)
        dq, dk, dv = ffv.vggt_frame_attn_backward(qd, kd, vd, o, gd, lse, pos_yx=pd)
        rq, rk, rv, rl = oracle.frame_attn_backward(q, k, v, g, S, T, pos=pos)
    torch.cuda.synchronize()
    lmax = float(np.abs(lse.cpu().numpy().astype(np.float64) - rl).max())
    print(f"{tag} lse: max_abs {lmax:.3e}")
    assert lmax <= (1e-2 if bf16 else 1e-5)
    check_grad(to_f64(dq), rq, f"{tag} dq", bf16)
    check_grad(to_f64(dk), rk, f"{tag} dk", bf16)
    check_grad(to_f64(dv), rv, f"{tag} dv", bf16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("glob", [True, False])
@pytest.mark.parametrize("shape", ["one_tile", "whole_tiles", "four_tiles"])
def test_backward_tile_edges(dtype, glob, shape):
    """Key and query ranges at tile edges: one frame of 7 x 7 patches + 5 special tokens
    (54 rows: a single ragged tile, the first tile also the last), frames of 8 x 8
    patches with no special tokens (64 rows: whole tiles, nothing masked), and frames of
    15 x 15 patches + 5 special tokens (230 rows: four key tiles per frame, eight for the
    pair, the last ragged, so the tile ring wraps and its last copies repeat the last tile)."""
    if shape == "one_tile":
        wl = workload.Workload("t", 81, S=1, gh=7, gw=7, n_special=5, patch_begin=5, H=2)
    elif shape == "whole_tiles":
        wl = workload.Workload("t", 82, S=2, gh=8, gw=8, n_special=0, patch_begin=0, H=2)
    else:
        wl = workload.Workload("t", 83, S=2, gh=15, gw=15, n_special=5, patch_begin=5, H=2)
    S, T, H = wl.S, wl.T, wl.H
    q, k, v = wl.qkv_bf16() if dtype == torch.bfloat16 else wl.qkv_f32()
    g = _dout(0xD0D1, (S, T, H, 64), dtype)
    pos = wl.positions()
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    pd = torch.from_numpy(pos).to(dev())
    bf16 = dtype == torch.bfloat16
    tag = f"{shape} {'global' if glob else 'frame'} {'bf16' if bf16 else 'f32'}"
    if glob:
        o, lse = ffv.vggt_global_attn_train(qd, kd, vd, pos_yx=pd)
        dq, dk, dv = ffv.vggt_global_attn_backward(qd, kd, vd, o, gd, lse, pos_yx=pd)
        rq, rk, rv, rl = oracle.global_attn_backward(q, k, v, g, S, T, pos=pos)
    else:
        o, lse = ffv.vggt_frame_attn_train(qd, kd, vd, pos_yx=pd)
        dq, dk, dv = ffv.vggt_frame_attn_backward(qd, kd, vd, o, gd, lse, pos_yx=pd)
        rq, rk, rv, rl = oracle.frame_attn_backward(q, k, v, g, S, T, pos=pos)
    torch.cuda.synchronize()
    lmax = float(np.abs(lse.cpu().numpy().astype(np.float64) - rl).max())
    print(f"{tag} lse: max_abs {lmax:.3e}")
    assert lmax <= (1e-2 if bf16 else 1e-5)
    check_grad(to_f64(dq), rq, f"{tag} dq", bf16)
    check_grad(to_f64(dk), rk, f"{tag} dk", bf16)
    check_grad(to_f64(dv), rv, f"{tag} dv", bf16)


def test_backward_is_deterministic_and_matches_plain_forward():
    wl = workload.Workload("t", 62, S=2, gh=12, gw=12, n_special=5, patch_begin=5, H=3)
    q, k, v = wl.qkv_bf16()
    g = _dout(0xD0D1, (wl.S, wl.T, wl.H, 64), torch.bfloat16)
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    pd = torch.from_numpy(wl.positions()).to(dev())
    o, lse = ffv.vggt_global_attn_train(qd, kd, vd, pos_yx=pd, kv_splits=1)
    assert torch.equal(o, ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=1))
    o3, lse3 = ffv.vggt_global_attn_train(qd, kd, vd, pos_yx=pd, kv_splits=3)
    assert (lse3 - lse).abs().max().item() <= 1e-4  # the split merge reproduces the normaliser
    a = ffv.vggt_global_attn_backward(qd, kd, vd, o, gd, lse, pos_yx=pd)
    b = ffv.vggt_global_attn_backward(qd, kd, vd, o, gd, lse, pos_yx=pd)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _full(name, S=None, glob=True, rows=None, cols=None):
    wl = workload.WORKLOADS[name]
    S = wl.S if S is None else S
    q, k, v = wl.qkv_bf16(S)
    g = _dout(0xD0D2 + wl.index, (S, wl.T, wl.H, 64), torch.bfloat16)
    pos = wl.positions()
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    pd = torch.from_numpy(pos).to(dev())
    train = ffv.vggt_global_attn_train if glob else ffv.vggt_frame_attn_train
    back = ffv.vggt_global_attn_backward if glob else ffv.vggt_frame_attn_backward
    ref_fn = oracle.global_attn_backward if glob else oracle.frame_attn_backward
    o, lse = train(qd, kd, vd, pos_yx=pd)
    dq, dk, dv = back(qd, kd, vd, o, gd, lse, pos_yx=pd)
    rq, rk, rv, _ = ref_fn(q, k, v, g, S, wl.T, pos=pos, rows=rows, cols=cols)
    n, H = S * wl.T, wl.H
    tag = f"{name} S={S} {'global' if glob else 'frame'}"
    check_grad(to_f64(dq).reshape(n, H, 64)[rows], rq, f"{tag} dq ({rows.size} rows)", True)
    if cols.size:
        check_grad(to_f64(dk).reshape(n, H, 64)[cols], rk, f"{tag} dk ({cols.size} rows)", True)
        check_grad(to_f64(dv).reshape(n, H, 64)[cols], rv, f"{tag} dv ({cols.size} rows)", True)


def test_backward_global_full_size_dq():
    # the S = 32 launch (N = 43968): query gradients need only their own rows' normalisers
    wl = workload.WORKLOADS["vggt-518-s32"]
    rows = sample_rows(wl.N, wl.T, wl.S, seed=31, n_random=24)
    _full("vggt-518-s32", rows=rows, cols=np.zeros(0, dtype=np.int64))


def test_backward_global_sampled_all_gradients():
    # key and value gradients sum over every query: 4 frames (N = 5496) keep the oracle to seconds
    wl = workload.WORKLOADS["vggt-518-s8"]
    n = 4 * wl.T
    _full("vggt-518-s8", S=4, rows=sample_rows(n, wl.T, 4, seed=41, n_random=24),
          cols=sample_rows(n, wl.T, 4, seed=42, n_random=24))


def test_backward_frame_full_size_sampled():
    # frame attention at S = 32: rows and keys of three frames
    wl = workload.WORKLOADS["vggt-518-s32"]
    T = wl.T
    pick = np.concatenate([f * T + np.array([0, 4, 5, 700, T - 64, T - 1]) for f in (0, 17, 31)])
    _full("vggt-518-s32", glob=False, rows=pick, cols=pick[::-1].copy())
