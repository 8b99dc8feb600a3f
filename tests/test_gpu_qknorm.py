"""GPU parity of the fused per-head Q/K LayerNorm + RoPE prologue (frame and
global attention) against the float64 oracle; bars as in the other parity
tests.  gamma/beta are seeded float32 vectors around (1, 0)."""
import numpy as np
import pytest
import torch

import feed_forward_view_amd as ffv
import oracle
import workload
from checks import check_bf16, check_f32
from test_gpu_parity import dev, sample_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ffv.lib()
    yield
    torch.cuda.synchronize()


def _params(seed):
    g = (1.0 + 0.3 * workload.normal_f32(seed, (64,))).astype(np.float32)
    b = (0.3 * workload.normal_f32(seed + 1, (64,))).astype(np.float32)
    return g, b


def _norms(seed, eps=1e-5):
    qg, qb = _params(seed)
    kg, kb = _params(seed + 2)
    host = ((qg, qb, eps), (kg, kb, eps))
    devp = tuple((torch.from_numpy(g).to(dev()), torch.from_numpy(b).to(dev())) for g, b, _ in host)
    return host, devp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rope", [True, False])
def test_qknorm_small_full(dtype, rope):
    wl = workload.Workload("t", 41, S=3, gh=9, gw=9, n_special=5, patch_begin=5, H=4)
    q, k, v = wl.qkv_bf16() if dtype == torch.bfloat16 else wl.qkv_f32()
    pos = wl.positions() if rope else None
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pd = torch.from_numpy(pos).to(dev()) if rope else None
    (qn, kn), ((qg, qb), (kg, kb)) = _norms(0xA11CE)
    check = check_bf16 if dtype == torch.bfloat16 else check_f32
    tag = f"{'bf16' if dtype == torch.bfloat16 else 'f32'} rope={rope}"
    fo = ffv.vggt_frame_attn_qknorm(qd, kd, vd, (qg, qb), (kg, kb), eps=1e-5, pos_yx=pd)
    check(to_f64(fo), oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos, q_norm=qn, k_norm=kn), f"frame qknorm {tag}")
    ref = oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos, q_norm=qn, k_norm=kn)
    for splits in (1, 3):
        go = ffv.vggt_global_attn_qknorm(qd, kd, vd, (qg, qb), (kg, kb), eps=1e-5, pos_yx=pd, kv_splits=splits)
        check(to_f64(go), ref, f"global qknorm {tag} splits={splits}")


def test_qknorm_zero_key_gain_gives_mean_of_values():
    # gamma_k = 0 maps every key to beta_k; without RoPE all scores of a query are equal
    wl = workload.Workload("t", 42, S=2, gh=8, gw=8, n_special=2, patch_begin=2, H=2)
    q, k, v = wl.qkv_bf16()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    one = torch.ones(64, device=dev())
    zero = torch.zeros(64, device=dev())
    beta = torch.from_numpy(workload.normal_f32(77, (64,))).to(dev())
    go = ffv.vggt_global_attn_qknorm(qd, kd, vd, (one, zero), (zero, beta), kv_splits=1)
    vm = oracle.to_f64(v).reshape(-1, 2, 64).mean(axis=0)
    check_bf16(to_f64(go), np.broadcast_to(vm, (wl.N, 2, 64)).reshape(wl.S, wl.T, 2, 64), "zero key gain")


def test_qknorm_full_size():
    wl = workload.WORKLOADS["vggt-518-s32"]
    q, k, v = wl.qkv_bf16()
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    (qn, kn), (qp, kp) = _norms(0xB0B)
    rows = sample_rows(wl.N, wl.T, wl.S, seed=wl.index + 7, n_random=48)
    fo = ffv.vggt_frame_attn_qknorm(qd, kd, vd, qp, kp, pos_yx=pd)
    check_bf16(to_f64(fo).reshape(wl.N, wl.H, 64)[rows],
               oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos, rows=rows, q_norm=qn, k_norm=kn),
               f"s32 frame qknorm ({rows.size} rows)")
    del fo
    go = ffv.vggt_global_attn_qknorm(qd, kd, vd, qp, kp, pos_yx=pd)
    check_bf16(to_f64(go).reshape(wl.N, wl.H, 64)[rows],
               oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos, rows=rows, q_norm=qn, k_norm=kn),
               f"s32 global qknorm ({rows.size} rows)")
