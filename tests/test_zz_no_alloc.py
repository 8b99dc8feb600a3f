"""The allocation-free frame attention (vggt_frame_attn_noalloc) through the C
ABI against the workspace-taking vggt_frame_attn on the same inputs: two calls
in a row, the second smaller than the first (its scratch array still holds the
first call's tiles), in bf16 with and without RoPE and in fp32; results must be
bit-identical, and the smaller call also meets the parity bars against the
float64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import feed_forward_view_amd as ffv
import oracle
import workload
from checks import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _f64(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return oracle.to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def _noalloc(q, k, v, out, pos, scale=0.0):
    S, T, H, _ = q.shape
    dt = ffv.BF16 if q.dtype == torch.bfloat16 else ffv.F32
    st = ffv.lib().vggt_frame_attn_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), dt, S, T, H, None if pos is None else ctypes.c_void_p(pos.data_ptr()),
        100.0, scale, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, ffv.lib().vggt_last_error()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ffv.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rope", [True, False])
def test_noalloc_matches_workspace_call(dtype, rope):
    # first call: 8 frames of 1374 tokens x 16 heads (bf16) / 2 frames (fp32, whose rotated
    # copies are 4x larger); second call: 3 frames of 86 tokens x 2 heads
    big = workload.Workload("t", 81, S=8 if dtype == "bf16" else 2, gh=37, gw=37, n_special=5, patch_begin=5)
    small = workload.Workload("t", 82, S=3, gh=9, gw=9, n_special=5, patch_begin=5, H=2)
    for n, wl in enumerate((big, small)):
        q, k, v = wl.qkv_bf16() if dtype == "bf16" else wl.qkv_f32()
        pos = wl.positions()
        qd, kd, vd = _dev(q), _dev(k), _dev(v)
        pd = torch.from_numpy(pos).cuda() if rope else None
        ref = ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd)
        out = torch.full_like(qd, float("nan"))
        _noalloc(qd, kd, vd, out, pd)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16) if dtype == "bf16" else out.view(torch.int32),
                           ref.view(torch.int16) if dtype == "bf16" else ref.view(torch.int32))
        assert same, f"call {n}: differs from vggt_frame_attn by {(out.float() - ref.float()).abs().max().item()}"
        if n == 1:
            r = oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos if rope else None)
            (check_bf16 if dtype == "bf16" else check_f32)(_f64(out), r, f"noalloc {dtype} rope={rope}")


def test_noalloc_rejects_oversized_shapes():
    q = torch.empty(32, 1374, 16, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    S, T, H, _ = q.shape
    st = ffv.lib().vggt_frame_attn_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                           ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(o.data_ptr()), ffv.BF16,
                                           S, T, H, None, 100.0, 0.0, None)
    assert st == 6  # VGGT_ERR_WORKSPACE
