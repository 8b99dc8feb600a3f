"""GPU parity of FlashVGGT chunk-recursive attention over the descriptor cache
(append + attend per chunk, and all chunks in one launch) against the float64
oracle.  Same bars as the other parity tests: bf16 max-abs <= 2e-2 and
mean-abs <= 2e-3, fp32 NRMSE <= 1e-5.  Cache buffers start filled with 0xFF
bytes (NaN in both dtypes), so a tile slot that the append leaves unzeroed or
that the attention reads past the cached descriptors shows up as NaN."""
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


def _nan_cache(capacity, H, dtype):
    c = ffv.DescriptorCache(capacity, H, dtype, device=dev())
    c.buffer.fill_(255)
    return c


def _check(got, ref, label, dtype):
    (check_bf16 if dtype == torch.bfloat16 else check_f32)(got, ref, label)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_stream_small_chunks(dtype):
    S, F, H = 5, 2, 4
    wl = workload.Workload("t", 31, S=S, gh=12, gw=12, n_special=5, patch_begin=5, H=H)
    q, k, v = wl.qkv_bf16() if dtype == torch.bfloat16 else wl.qkv_f32()
    T = wl.T
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kp, vp = ffv.vggt_descriptor_pool(kd, vd, 12, 12, 5, 2, 2)
    Dn = kp.shape[1]
    assert Dn == 41  # chunks of 82 descriptors: appends start inside a tile and inside a 16-byte slot
    kpr = oracle.descriptor_pool(k, S, T, 12, 12, 5, 2, 2)
    vpr = oracle.descriptor_pool(v, S, T, 12, 12, 5, 2, 2)
    ref = oracle.descriptor_stream_xattn(q, kpr, vpr, F).reshape(S, T, H, 64)
    cache = _nan_cache(S * Dn + 7, H, dtype)
    outs = []
    for c in range((S + F - 1) // F):
        f0, f1 = c * F, min(S, (c + 1) * F)
        cache.append(kp[f0:f1], vp[f0:f1])
        assert cache.used == f1 * Dn
        splits = (1, 3, 0)[c % 3]
        o = cache.attend(qd[f0:f1], kv_splits=splits)
        _check(to_f64(o), ref[f0:f1], f"stream chunk {c} splits={splits}", dtype)
        outs.append(cache.attend(qd[f0:f1], kv_splits=1))
    oc = cache.attend_chunked(qd, Dn, F)
    _check(to_f64(oc), ref, "chunked one launch", dtype)
    # one launch and chunk-by-chunk run the same arithmetic per query
    assert torch.equal(oc, torch.cat(outs))


def test_stream_one_chunk_equals_descriptor_xattn():
    wl = workload.Workload("t", 32, S=3, gh=9, gw=9, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_bf16()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kp, vp = ffv.vggt_descriptor_pool(kd, vd, 9, 9, 5, 2, 2)
    Dn = kp.shape[1]
    cache = _nan_cache(wl.S * Dn, 2, torch.bfloat16)
    cache.append(kp, vp)
    for splits in (1, 2):
        x = ffv.vggt_descriptor_xattn(qd, kp, vp, kv_splits=splits)
        assert torch.equal(cache.attend(qd, kv_splits=splits), x)
    assert torch.equal(cache.attend_chunked(qd, Dn, wl.S), ffv.vggt_descriptor_xattn(qd, kp, vp, kv_splits=1))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cache_ragged_appends(dtype):
    # appends of 1..66 descriptors land on every kind of tile and slot boundary
    H, nq = 3, 77
    sizes = [1, 7, 8, 3, 64, 1, 66, 13]
    cap = sum(sizes)
    gen = workload.normal_bf16 if dtype == torch.bfloat16 else workload.normal_f32
    kd = gen(0xCAC4E, (cap, H, 64))
    vd = gen(0xCAC4F, (cap, H, 64))
    q = gen(0xCAC50, (nq, H, 64))
    qd, kdd, vdd = to_dev(q), to_dev(kd), to_dev(vd)
    cache = _nan_cache(cap, H, dtype)
    for n in sizes:
        u = cache.used
        cache.append(kdd[u:u + n], vdd[u:u + n])
        got = to_f64(cache.attend(qd))
        ref = oracle.attention(q, kd[:cache.used], vd[:cache.used])
        _check(got, ref, f"cache of {cache.used}", dtype)


def test_full_size_streaming():
    wl = workload.WORKLOADS["flashvggt-518-s100"]
    q, k, v = wl.qkv_bf16()
    S, T, H = wl.S, wl.T, wl.H
    F = 10
    ph, pw = wl.pool
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kp, vp = ffv.vggt_descriptor_pool(kd, vd, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    Dn = kp.shape[1]
    del kd, vd
    kpr = oracle.descriptor_pool(k, S, T, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    vpr = oracle.descriptor_pool(v, S, T, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    cache = _nan_cache(S * Dn, H, torch.bfloat16)
    out = torch.empty_like(qd)
    for c in range(S // F):
        cache.append(kp[c * F:(c + 1) * F], vp[c * F:(c + 1) * F])
        cache.attend(qd[c * F:(c + 1) * F], out=out[c * F:(c + 1) * F])
    rows = sample_rows(wl.N, T, S, seed=wl.index + 100, n_random=60, tile=F * T)
    ref = oracle.descriptor_stream_xattn(q, kpr, vpr, F, rows=rows)
    check_bf16(to_f64(out).reshape(wl.N, H, 64)[rows], ref, f"s100 streaming ({rows.size} rows)")
    oc = cache.attend_chunked(qd, Dn, F)
    check_bf16(to_f64(oc).reshape(wl.N, H, 64)[rows], ref, f"s100 chunked ({rows.size} rows)")


def test_kernel_timer_brackets_attention_kernels():
    wl = workload.Workload("t", 33, S=4, gh=16, gw=16, n_special=5, patch_begin=5, H=4)
    q, k, v = wl.qkv_bf16()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pos = torch.from_numpy(wl.positions()).to(dev())
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ffv.vggt_timer_start(8)
    a.record(stream)
    ffv.vggt_global_attn(qd, kd, vd, pos_yx=pos, kv_splits=2)
    b.record(stream)
    ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pos)
    rec = ffv.vggt_timer_stop()
    assert [kind for kind, _ in rec] == ["global", "frame"]
    assert all(ms > 0 for _, ms in rec)
    # the kernel alone takes no longer than the whole call (prep + kernel + merge)
    assert rec[0][1] <= a.elapsed_time(b) + 1e-3
    # launches past the capacity are not recorded; the timer can be re-armed
    ffv.vggt_timer_start(1)
    ffv.vggt_frame_attn(qd, kd, vd)
    ffv.vggt_frame_attn(qd, kd, vd)
    assert [kind for kind, _ in ffv.vggt_timer_stop()] == ["frame"]


@pytest.mark.parametrize("kind", ["sharp", "negative"])
def test_stream_softmax_range(kind):
    """Cache attention (per chunk, split and unsplit), the one-launch chunked form and the
    full cross-attention on rows whose softmax leaves the optimistic pass's range: logits
    in the hundreds (scale 8 ln 2) or all far below zero (q >= 0 >= k), so workgroups rerun
    their key ranges exactly, with per-sequence key prefixes and a shared key set.  The
    descriptors are seeded bf16 values given directly (41 per frame, ragged against the
    64-key tiles), so both sides start from identical inputs."""
    S, F, H, T, Dn = 5, 2, 2, 86, 41
    q = workload.normal_bf16(0x5A0, (S, T, H, 64))
    kp = workload.normal_bf16(0x5A1, (S, Dn, H, 64))
    vp = workload.normal_bf16(0x5A2, (S, Dn, H, 64))
    if kind == "negative":
        q = q & np.uint16(0x7FFF)
        kp = kp | np.uint16(0x8000)
    scale = float(np.float32(8.0 * np.log(2.0)))
    qd, kpd, vpd = to_dev(q), to_dev(kp), to_dev(vp)
    ref = oracle.descriptor_stream_xattn(q, kp, vp, F, scale=scale).reshape(S, T, H, 64)
    cache = _nan_cache(S * Dn, H, torch.bfloat16)
    for c in range((S + F - 1) // F):
        f0, f1 = c * F, min(S, (c + 1) * F)
        cache.append(kpd[f0:f1], vpd[f0:f1])
        for splits in (1, 3, 0):
            o = cache.attend(qd[f0:f1], scale=scale, kv_splits=splits)
            check_bf16(to_f64(o), ref[f0:f1], f"{kind} stream chunk {c} splits={splits}")
    check_bf16(to_f64(cache.attend_chunked(qd, Dn, F, scale=scale)), ref, f"{kind} chunked one launch")
    xref = oracle.attention(q.reshape(S * T, H, 64), kp.reshape(S * Dn, H, 64), vp.reshape(S * Dn, H, 64),
                            scale=scale)
    for splits in (1, 2):
        x = ffv.vggt_descriptor_xattn(qd, kpd, vpd, scale=scale, kv_splits=splits)
        check_bf16(to_f64(x), xref.reshape(S, T, H, 64), f"{kind} descriptor xattn splits={splits}")
