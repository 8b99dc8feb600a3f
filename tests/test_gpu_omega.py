"""GPU parity of the VGGT-Omega block variants -- attention over the first
T_active tokens of each frame (register tokens left out) and global attention
with sequence-level extra tokens -- against the float64 oracle; bars as in the
other parity tests.  Output rows of left-out tokens must keep what the
caller stored there."""
import numpy as np
import pytest
import torch

import feed_forward_view_amd as ffv
import oracle
import workload
from checks import check_bf16, check_f32
from test_gpu_parity import dev, sample_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ffv.lib()
    yield
    torch.cuda.synchronize()


def _extras(seed, E, H, dtype):
    gen = workload.normal_bf16 if dtype == torch.bfloat16 else workload.normal_f32
    return [gen(seed + i, (E, H, 64)) for i in range(3)]


def _norms(seed):
    host = []
    for i in range(2):
        g = (1.0 + 0.3 * workload.normal_f32(seed + 2 * i, (64,))).astype(np.float32)
        b = (0.3 * workload.normal_f32(seed + 2 * i + 1, (64,))).astype(np.float32)
        host.append((g, b, 1e-5))
    devp = [(torch.from_numpy(g).to(dev()), torch.from_numpy(b).to(dev())) for g, b, _ in host]
    return host, devp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rope,norm", [(True, False), (False, False), (True, True)])
def test_omega_variants_small(dtype, rope, norm):
    # 6 x 6 patches first, then 4 register tokens; 3 extra tokens
    wl = workload.Workload("t", 51, S=3, gh=6, gw=6, n_special=4, patch_begin=0, H=2)
    S, T, H, Ta, E = wl.S, wl.T, wl.H, 36, 3
    q, k, v = wl.qkv_bf16() if dtype == torch.bfloat16 else wl.qkv_f32()
    xq, xk, xv = _extras(0xE77A, E, H, dtype)
    pos = wl.positions() if rope else None
    pd = torch.from_numpy(pos).to(dev()) if rope else None
    (qn, kn), (qp, kp) = _norms(0x0E6A) if norm else ((None, None), (None, None))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    xqd, xkd, xvd = to_dev(xq), to_dev(xk), to_dev(xv)
    check = check_bf16 if dtype == torch.bfloat16 else check_f32
    tag = f"{'bf16' if dtype == torch.bfloat16 else 'f32'} rope={rope} norm={norm}"

    fo = torch.full_like(qd, SENTINEL)
    ffv.vggt_frame_attn_ex(qd, kd, vd, Ta, out=fo, pos_yx=pd, q_norm=qp, k_norm=kp)
    ref = oracle.frame_attn_ex(q, k, v, S, T, Ta, pos=pos, q_norm=qn, k_norm=kn)
    check(to_f64(fo)[:, :Ta], ref, f"frame_ex {tag}")
    assert bool((fo[:, Ta:] == SENTINEL).all()), "register rows of the output were written"

    rf, rx = oracle.global_attn_ex(q, k, v, S, T, Ta, xq, xk, xv, pos=pos, q_norm=qn, k_norm=kn)
    for splits in (1, 3):
        go = torch.full_like(qd, SENTINEL)
        go, xo = ffv.vggt_global_attn_ex(qd, kd, vd, Ta, xqd, xkd, xvd, out=go, pos_yx=pd, kv_splits=splits,
                                         q_norm=qp, k_norm=kp)
        check(to_f64(go)[:, :Ta], rf, f"global_ex frames {tag} splits={splits}")
        check(to_f64(xo), rx, f"global_ex extras {tag} splits={splits}")
        assert bool((go[:, Ta:] == SENTINEL).all()), "register rows of the output were written"


def test_frame_ex_reads_no_register_rows():
    # The register tokens (rows T_active .. T-1 of each frame) are outside every key set:
    # with their K and V all NaN the active rows must still match the oracle.  Frame calls
    # read V rows in place and stop at the last active key of each frame.
    wl = workload.Workload("t", 53, S=3, gh=6, gw=11, n_special=4, patch_begin=0, H=2)
    S, T, H, Ta = wl.S, wl.T, wl.H, 66  # 66 active keys: a full 64-key tile and 2 more
    q, k, v = wl.qkv_bf16()
    pos = wl.positions()
    ref = oracle.frame_attn_ex(q, k, v, S, T, Ta, pos=pos)
    k[:, Ta:] = 0x7FC0
    v[:, Ta:] = 0x7FC0
    fo = ffv.vggt_frame_attn_ex(to_dev(q), to_dev(k), to_dev(v), Ta, pos_yx=torch.from_numpy(pos).to(dev()))
    check_bf16(to_f64(fo[:, :Ta].contiguous()), ref, "frame_ex with NaN register rows")


def test_global_ex_reads_no_register_rows():
    # the same for the compacted global key set (active rows of every frame, then extras)
    wl = workload.Workload("t", 54, S=3, gh=6, gw=11, n_special=4, patch_begin=0, H=2)
    S, T, H, Ta, E = wl.S, wl.T, wl.H, 66, 2
    q, k, v = wl.qkv_bf16()
    xq, xk, xv = _extras(0xE78A, E, H, torch.bfloat16)
    pos = wl.positions()
    rf, rx = oracle.global_attn_ex(q, k, v, S, T, Ta, xq, xk, xv, pos=pos)
    k[:, Ta:] = 0x7FC0
    v[:, Ta:] = 0x7FC0
    go, xo = ffv.vggt_global_attn_ex(to_dev(q), to_dev(k), to_dev(v), Ta, to_dev(xq), to_dev(xk), to_dev(xv),
                                     pos_yx=torch.from_numpy(pos).to(dev()))
    check_bf16(to_f64(go[:, :Ta].contiguous()), rf, "global_ex frames with NaN register rows")
    check_bf16(to_f64(xo), rx, "global_ex extras with NaN register rows")


@pytest.mark.parametrize("splits", [1, 3])
def test_global_ex_without_extras_matches_global(splits):
    # N = 3 * 149 = 447 keys: 7 key tiles, the last holding 63 keys
    wl = workload.Workload("t", 52, S=3, gh=12, gw=12, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_bf16()
    pd = torch.from_numpy(wl.positions()).to(dev())
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    a, x = ffv.vggt_global_attn_ex(qd, kd, vd, wl.T, pos_yx=pd, kv_splits=splits)
    assert x is None
    b = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=splits)
    # same keys, key tiles and arithmetic per query; the query-tile grouping differs, and the
    # V operand comes from V^T tiles (compacted key set) in one call and from V rows read in
    # place (two query tiles) in the other
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), \
        f"max diff {(a.float() - b.float()).abs().max().item():.3e}"


def test_omega_full_size():
    wl = workload.WORKLOADS["omega-512-s64"]
    q, k, v = wl.qkv_bf16()
    S, T, H = wl.S, wl.T, wl.H
    Ta, E = wl.gh * wl.gw, 5  # 1024 patches; 4 storage tokens + 1 camera token
    assert (T, Ta) == (1040, 1024)
    pos = wl.positions()
    xq, xk, xv = _extras(0x0E6A5, E, H, torch.bfloat16)
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    go, xo = ffv.vggt_global_attn_ex(qd, kd, vd, Ta, to_dev(xq), to_dev(xk), to_dev(xv), pos_yx=pd)
    n = S * Ta
    rows = sample_rows(n, Ta, S, seed=wl.index + 11, n_random=48)
    ref = oracle.global_attn_ex(q, k, v, S, T, Ta, xq, xk, xv, pos=pos, rows=np.concatenate([rows, n + np.arange(E)]))
    got = to_f64(go[:, :Ta].contiguous()).reshape(n, H, 64)[rows]
    check_bf16(got, ref[:rows.size], f"s64 global_ex frames ({rows.size} rows)")
    check_bf16(to_f64(xo), ref[rows.size:], "s64 global_ex extras")
    del go
    fo = ffv.vggt_frame_attn_ex(qd, kd, vd, Ta, pos_yx=pd)
    fr = oracle.frame_attn(q[:, :Ta], k[:, :Ta], v[:, :Ta], S, Ta, pos=pos[:Ta], rows=rows)
    check_bf16(to_f64(fo[:, :Ta].contiguous()).reshape(n, H, 64)[rows], fr, f"s64 frame_ex ({rows.size} rows)")


def test_omega_softmax_range():
    """The Omega forms (registers left out, extra sequence-level tokens) on logits in the
    hundreds (scale 8 ln 2), so their workgroups rerun their key ranges exactly.  No RoPE
    or LayerNorm: at this scale the bf16 rounding of rotated or normalised operands, which
    the float64 oracle does not share, would move the weights by far more than the bar.
    With scale * log2(e) = 8 the kernels' operands are exact."""
    wl = workload.Workload("t", 53, S=3, gh=6, gw=6, n_special=4, patch_begin=0, H=2)
    S, T, H, Ta, E = wl.S, wl.T, wl.H, 36, 3
    q, k, v = wl.qkv_bf16()
    xq, xk, xv = _extras(0xE77B, E, H, torch.bfloat16)
    scale = float(np.float32(8.0 * np.log(2.0)))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    xqd, xkd, xvd = to_dev(xq), to_dev(xk), to_dev(xv)
    fo = ffv.vggt_frame_attn_ex(qd, kd, vd, Ta, scale=scale)
    ref = oracle.frame_attn_ex(q, k, v, S, T, Ta, scale=scale)
    check_bf16(to_f64(fo)[:, :Ta], ref, "sharp frame_ex")
    rf, rx = oracle.global_attn_ex(q, k, v, S, T, Ta, xq, xk, xv, scale=scale)
    for splits in (1, 3):
        go, xo = ffv.vggt_global_attn_ex(qd, kd, vd, Ta, xqd, xkd, xvd, scale=scale, kv_splits=splits)
        check_bf16(to_f64(go)[:, :Ta], rf, f"sharp global_ex frames splits={splits}")
        check_bf16(to_f64(xo), rx, f"sharp global_ex extras splits={splits}")
