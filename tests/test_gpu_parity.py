"""GPU parity: the HIP library (through the C ABI) against the float64 oracle.

Bars (tests/checks.py): bf16 max |gpu - oracle| <= 2e-2, mean <= 2e-3, NRMSE
<= 1e-2 and max <= 0.25 rms(oracle) per output tensor, for unit-normal Q/K/V;
fp32 debug NRMSE <= 1e-5 (sqrt(mean(err^2)) / sqrt(mean(ref^2))).  Small
shapes and the S = 8 VGGT-1B workload (N = 10992) are compared on every row;
the larger workloads on sampled query rows (every special token of the first
and last frame, the first and last rows, the rows around query-tile
boundaries, the last partial tile and seeded random rows) in the launch
configuration the benchmark times.
"""
import functools

import numpy as np
import pytest
import torch

import feed_forward_view_amd as ffv
import oracle
import workload
from checks import check_bf16, check_f32, check_same_up_to_sum_order  # noqa: F401

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ffv.lib()
    yield
    torch.cuda.synchronize()


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def to_f64(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return oracle.to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def sample_rows(n: int, T: int, S: int, seed: int, n_random: int = 96, tile: int = 256) -> np.ndarray:
    rows = set(range(min(5, n)))
    rows |= {(S - 1) * T + t for t in range(min(5, T))}
    rows |= {0, n - 1}
    for b in range(tile, n, tile * max(1, (n // tile) // 8)):
        rows |= {b - 1, b, b + 1}
    last = (n - 1) // tile * tile
    rows |= set(range(last, n, max(1, (n - last) // 8)))
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, n, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


@functools.lru_cache(maxsize=2)
def inputs(name: str):
    wl = workload.WORKLOADS[name]
    q, k, v = wl.qkv_bf16()
    return wl, q, k, v


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_against_oracle(dtype):
    wl = workload.WORKLOADS["vggt-518-s8"]
    S = 2
    x = workload.normal_bf16(wl.seed("q"), (S, wl.T, 16, 64))
    if dtype == "f32":
        x = workload.bf16_bits_to_f32(x).reshape(x.shape)
    pos = wl.positions()
    xd = to_dev(x)
    ffv.vggt_attn_rope(xd, torch.from_numpy(pos).to(dev()), 100.0)
    got = to_f64(xd).reshape(S * wl.T, 16, 64)
    ref = oracle.rope(oracle.to_f64(x).reshape(S * wl.T, 16, 64), np.tile(pos, (S, 1)), 100.0)
    xin = oracle.to_f64(x).reshape(S * wl.T, 16, 64)
    # fp32 rotation error, relative to the magnitude of the rotated pair
    pair = np.abs(xin) + np.abs(xin.reshape(-1, 2)[:, ::-1].reshape(xin.shape))
    eps32 = 2.0 ** -21 * pair
    if dtype == "bf16":
        # one fp32 rotation then one rounding to bf16: within half a bf16 ulp
        # (plus the fp32 error) of the exact value, and equal to its
        # round-to-nearest-even almost everywhere
        mag = np.maximum(np.maximum(np.abs(ref), np.abs(got)), 1e-30)
        ulp = np.exp2(np.floor(np.log2(mag)) - 7)
        excess = np.abs(got - ref) - (0.5 * ulp + eps32)
        assert excess.max() <= 0, f"rope bf16: worst excess {excess.max():.3e}"
        rne = oracle.to_f64(workload.f32_to_bf16_bits(ref.astype(np.float32))).reshape(ref.shape)
        frac = float(np.mean(got == rne))
        print(f"rope bf16: exact-RNE fraction {frac:.6f}")
        assert frac >= 0.999
    else:
        excess = np.abs(got - ref) - (2.0 ** -23 * np.abs(ref) + eps32)
        assert excess.max() <= 0, f"rope f32: worst excess {excess.max():.3e}"
    # special tokens (position (0,0)) are untouched, bit for bit
    specials = np.concatenate([np.arange(5) + s * wl.T for s in range(S)])
    np.testing.assert_array_equal(got[specials], xin[specials])


# ---------------------------------------------------------------------------
# Frame / global attention, small shapes compared in full
# ---------------------------------------------------------------------------

def test_frame_and_global_small_full():
    wl, q, k, v = inputs("vggt-224-s4")
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    fo = to_f64(ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd, rope_base=100.0))
    check_bf16(fo, oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos), "frame 4x261")
    ref_g = oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos)
    for splits in (0, 1, 2, 3, 7):
        go = to_f64(ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, rope_base=100.0, kv_splits=splits))
        check_bf16(go, ref_g, f"global N=1044 splits={splits}")


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 129, 257])
@pytest.mark.parametrize("H", [1, 3])
def test_ragged_shapes(T, H):
    S = 3
    seed = 1000 + 10 * T + H
    q = workload.normal_bf16(seed, (S, T, H, 64))
    k = workload.normal_bf16(seed + 1, (S, T, H, 64))
    v = workload.normal_bf16(seed + 2, (S, T, H, 64))
    gh = max(1, int(np.sqrt(max(T - 2, 1))))
    gw = max(1, (T - 2) // gh) if T > 2 else 1
    pb = T - gh * gw
    pos = workload.positions(T, gh, gw, pb)
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    for use_pos in (True, False):
        p_host = pos if use_pos else None
        p_dev = pd if use_pos else None
        fo = to_f64(ffv.vggt_frame_attn(qd, kd, vd, pos_yx=p_dev))
        check_bf16(fo, oracle.frame_attn(q, k, v, S, T, pos=p_host), f"frame T={T} H={H} rope={use_pos}")
        ref = oracle.global_attn(q, k, v, S, T, pos=p_host)
        for splits in (1, 2):
            go = to_f64(ffv.vggt_global_attn(qd, kd, vd, pos_yx=p_dev, kv_splits=splits))
            check_bf16(go, ref, f"global T={T} H={H} rope={use_pos} splits={splits}")


@pytest.mark.parametrize("T", [69, 128])
def test_frame_v_rows_stay_inside_the_frame(T):
    # Frame attention reads V rows in place; the last key tile of frame 0 covers rows of
    # frame 1 (T = 69: 59 of its 64 rows).  With frame 1's V all NaN, frames 0 and 2 must
    # still match the oracle: rows past a frame's keys are never read into the P V product.
    S, H = 3, 2
    q = workload.normal_bf16(0xF0, (S, T, H, 64))
    k = workload.normal_bf16(0xF1, (S, T, H, 64))
    v = workload.normal_bf16(0xF2, (S, T, H, 64))
    v[1] = 0x7FC0  # bf16 quiet NaN
    with np.errstate(invalid="ignore"):  # frame 1's NaN outputs
        out = to_f64(ffv.vggt_frame_attn(to_dev(q), to_dev(k), to_dev(v)))
    for s in (0, 2):
        ref = oracle.frame_attn(q[s:s + 1], k[s:s + 1], v[s:s + 1], 1, T)
        check_bf16(out[s:s + 1], ref, f"frame {s} beside a NaN frame, T={T}")
    assert np.isnan(out[1]).all()


def test_long_frames_take_vt_tiles():
    # Frames of 8229 tokens have 33 query tiles per key set, so frame attention builds V^T
    # tiles per frame instead of reading V in place (7900 tokens: 31 tiles, V in place);
    # sampled rows against the oracle, RoPE on a 90 x 91 grid plus 39 special tokens
    H = 2
    for S, T in ((2, 8229), (2, 7900)):
        gh, gw = 90, (T - 39) // 90
        pos = workload.positions(T, gh, gw, T - gh * gw)
        q = workload.normal_bf16(0xB0 + T, (S, T, H, 64))
        k = workload.normal_bf16(0xB1 + T, (S, T, H, 64))
        v = workload.normal_bf16(0xB2 + T, (S, T, H, 64))
        out = ffv.vggt_frame_attn(to_dev(q), to_dev(k), to_dev(v), pos_yx=torch.from_numpy(pos).to(dev()))
        rows = sample_rows(S * T, T, S, seed=T, n_random=64)
        ref = oracle.frame_attn(q, k, v, S, T, pos=pos, rows=rows)
        got = to_f64(out).reshape(S * T, H, 64)[rows]
        check_bf16(got, ref, f"frame S={S} T={T} ({rows.size} rows)")


def test_many_heads():
    # 128 heads (the most the library takes): a token row is 16 KiB, the stride the frame
    # kernel uses when it reads V rows in place; global attention at N = 3 x 69 does too
    S, T, H = 3, 69, 128
    q = workload.normal_bf16(0xA0, (S, T, H, 64))
    k = workload.normal_bf16(0xA1, (S, T, H, 64))
    v = workload.normal_bf16(0xA2, (S, T, H, 64))
    pos = workload.positions(T, 8, 8, 5)
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    check_bf16(to_f64(ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd)), oracle.frame_attn(q, k, v, S, T, pos=pos),
               "frame H=128")
    check_bf16(to_f64(ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=2)),
               oracle.global_attn(q, k, v, S, T, pos=pos), "global H=128 splits=2")


def test_single_token_frames_return_values():
    q = workload.normal_bf16(5, (4, 1, 2, 64))
    v = workload.normal_bf16(6, (4, 1, 2, 64))
    out = ffv.vggt_frame_attn(to_dev(q), to_dev(q), to_dev(v))
    np.testing.assert_array_equal(to_f64(out), oracle.to_f64(v))


def test_scale_argument():
    wl = workload.Workload("t", 21, S=2, gh=6, gw=6, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_bf16()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ref = oracle.global_attn(q, k, v, wl.S, wl.T, scale=0.3)
    check_bf16(to_f64(ffv.vggt_global_attn(qd, kd, vd, scale=0.3)), ref, "global scale=0.3")


def test_deterministic_repeat():
    wl, q, k, v = inputs("vggt-224-s4")
    pos = torch.from_numpy(wl.positions()).to(dev())
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    a = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pos, kv_splits=3)
    b = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pos, kv_splits=3)
    c = ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pos)
    d = ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pos)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))


def test_side_stream_launch():
    """Calls on a stream other than torch's current one: the workspace and the
    outputs come from that stream's pool, so the current stream's allocations
    made while the kernels run cannot take their memory."""
    wl, q, k, v = inputs("vggt-224-s4")
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    fo = ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd, stream=side)
    go = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=2, stream=side)
    xo = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=3, stream=side)
    churn = [torch.full((1 << 20,), float(i), device=dev()) for i in range(16)]
    side.synchronize()
    del churn
    check_bf16(to_f64(fo), oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos), "side stream frame")
    ref = oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos)
    check_bf16(to_f64(go), ref, "side stream global splits=2")
    check_bf16(to_f64(xo), ref, "side stream global splits=3")


def test_frame_permutation_equivariance_gpu():
    wl, q, k, v = inputs("vggt-224-s4")
    pos = torch.from_numpy(wl.positions()).to(dev())
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    perm = torch.tensor([2, 0, 3, 1], device=dev())
    g = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pos, kv_splits=1)
    gp = ffv.vggt_global_attn(qd[perm].contiguous(), kd[perm].contiguous(), vd[perm].contiguous(), pos_yx=pos,
                              kv_splits=1)
    # equal up to the summation order of the keys
    check_same_up_to_sum_order(to_f64(gp), to_f64(g[perm].contiguous()), "frame permutation")


# ---------------------------------------------------------------------------
# fp32 debug mode
# ---------------------------------------------------------------------------

def test_f32_debug_mode():
    wl = workload.Workload("t", 22, S=3, gh=9, gw=11, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_f32()
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    check_f32(to_f64(ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd)), oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos),
              "f32 frame")
    ref = oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos)
    for splits in (1, 3):
        check_f32(to_f64(ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=splits)), ref,
                  f"f32 global splits={splits}")
    kp, vp = ffv.vggt_descriptor_pool(kd, vd, 9, 11, 5, 2, 2)
    kpr = oracle.descriptor_pool(k, wl.S, wl.T, 9, 11, 5, 2, 2)
    vpr = oracle.descriptor_pool(v, wl.S, wl.T, 9, 11, 5, 2, 2)
    check_f32(to_f64(kp), kpr, "f32 pool k")
    check_f32(to_f64(ffv.vggt_descriptor_xattn(qd, kp, vp, kv_splits=2)), oracle.descriptor_xattn(q, kpr, vpr),
              "f32 xattn")


# ---------------------------------------------------------------------------
# Descriptor pooling and cross-attention
# ---------------------------------------------------------------------------

def _pool_check(got_bits_f64, ref, label):
    # fp32 sum then one rounding: within one bf16 ulp of the exact mean, and
    # equal to its round-to-nearest-even almost everywhere
    ref32 = ref.astype(np.float32)
    rne = oracle.to_f64(workload.f32_to_bf16_bits(ref32)).reshape(ref.shape)
    got = got_bits_f64.reshape(ref.shape)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    bad = int(np.sum(np.abs(got - ref) > ulp))
    assert bad == 0, f"{label}: {bad} elements beyond one bf16 ulp"
    frac = float(np.mean(got == rne))
    print(f"{label}: exact-RNE fraction {frac:.6f}")
    assert frac >= 0.9999, label


def test_pool_small_grids():
    for (gh, gw, pb, ns, ph, pw) in [(37, 37, 5, 5, 2, 2), (5, 7, 3, 3, 2, 2), (4, 4, 0, 16, 2, 2), (6, 5, 1, 2, 3, 2),
                                     (3, 3, 0, 0, 1, 1)]:
        S, H = 2, 16
        T = gh * gw + ns
        k = workload.normal_bf16(77 + gh, (S, T, H, 64))
        v = workload.normal_bf16(78 + gh, (S, T, H, 64))
        kp, vp = ffv.vggt_descriptor_pool(to_dev(k), to_dev(v), gh, gw, pb, ph, pw)
        _pool_check(to_f64(kp), oracle.descriptor_pool(k, S, T, gh, gw, pb, ph, pw), f"pool k {gh}x{gw}/{ph}x{pw}")
        _pool_check(to_f64(vp), oracle.descriptor_pool(v, S, T, gh, gw, pb, ph, pw), f"pool v {gh}x{gw}/{ph}x{pw}")


def test_xattn_small_full_and_unit_window():
    wl = workload.Workload("t", 23, S=3, gh=12, gw=12, n_special=5, patch_begin=5, H=4)
    q, k, v = wl.qkv_bf16()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kp, vp = ffv.vggt_descriptor_pool(kd, vd, 12, 12, 5, 2, 2)
    kpr = oracle.descriptor_pool(k, wl.S, wl.T, 12, 12, 5, 2, 2)
    vpr = oracle.descriptor_pool(v, wl.S, wl.T, 12, 12, 5, 2, 2)
    # descriptors as the pool stores them: the oracle's means rounded to bf16 (RNE) on the host
    ref = oracle.descriptor_xattn(q, workload.f32_to_bf16_bits(kpr.astype(np.float32)),
                                  workload.f32_to_bf16_bits(vpr.astype(np.float32)))
    for splits in (0, 1, 3):
        check_bf16(to_f64(ffv.vggt_descriptor_xattn(qd, kp, vp, kv_splits=splits)), ref, f"xattn splits={splits}")
    # and end to end against the oracle's own pooled descriptors
    check_bf16(to_f64(ffv.vggt_descriptor_xattn(qd, kp, vp)), oracle.descriptor_xattn(q, kpr, vpr), "xattn e2e")
    # unit window: descriptor attention equals global attention without RoPE
    k1, v1 = ffv.vggt_descriptor_pool(kd, vd, 12, 12, 5, 1, 1)
    a = to_f64(ffv.vggt_descriptor_xattn(qd, k1, v1, kv_splits=1))
    check_bf16(a, oracle.global_attn(q, k, v, wl.S, wl.T), "xattn unit window vs global")


# ---------------------------------------------------------------------------
# Full-size workloads on sampled rows
# ---------------------------------------------------------------------------

def test_s8_frame_all_rows():
    """VGGT-1B at 8 frames: frame attention compared on every row."""
    wl, q, k, v = inputs("vggt-518-s8")
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    fo = ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd, rope_base=100.0)
    check_bf16(to_f64(fo), oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos), "vggt-518-s8 frame (all rows)")


def test_s8_global_all_rows():
    """VGGT-1B at 8 frames: global attention (N = 10992) compared on every row."""
    wl, q, k, v = inputs("vggt-518-s8")
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    go = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, rope_base=100.0)
    check_bf16(to_f64(go), oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos), "vggt-518-s8 global (all rows)")


@pytest.mark.parametrize("name", ["vggt-518-s32", "omega-512-s64"])
def test_full_size_frame_and_global(name):
    wl, q, k, v = inputs(name)
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    rows = sample_rows(wl.N, wl.T, wl.S, seed=wl.index, n_random=64)
    fo = ffv.vggt_frame_attn(qd, kd, vd, pos_yx=pd, rope_base=100.0)
    got = to_f64(fo).reshape(wl.N, wl.H, 64)[rows]
    check_bf16(got, oracle.frame_attn(q, k, v, wl.S, wl.T, pos=pos, rows=rows), f"{name} frame ({rows.size} rows)")
    del fo
    go = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, rope_base=100.0)
    got = to_f64(go).reshape(wl.N, wl.H, 64)[rows]
    check_bf16(got, oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos, rows=rows), f"{name} global ({rows.size} rows)")


def test_full_size_descriptor_path():
    wl, q, k, v = inputs("flashvggt-518-s100")
    ph, pw = wl.pool
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kp, vp = ffv.vggt_descriptor_pool(kd, vd, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    Dn = kp.shape[1]
    assert Dn == 366
    kpr = oracle.descriptor_pool(k, wl.S, wl.T, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    _pool_check(to_f64(kp), kpr, "s100 pool k")
    vpr = oracle.descriptor_pool(v, wl.S, wl.T, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    _pool_check(to_f64(vp), vpr, "s100 pool v")
    xo = ffv.vggt_descriptor_xattn(qd, kp, vp)
    rows = sample_rows(wl.N, wl.T, wl.S, seed=wl.index, n_random=48)
    got = to_f64(xo).reshape(wl.N, wl.H, 64)[rows]
    qs = q.reshape(wl.N, wl.H, 64)[rows]
    ref = oracle.attention(qs, kpr.reshape(-1, wl.H, 64), vpr.reshape(-1, wl.H, 64))
    check_bf16(got, ref, f"s100 xattn ({rows.size} rows)")


def test_split_count_independence_full_size():
    wl, q, k, v = inputs("vggt-518-s8")
    pos = wl.positions()
    qd, kd, vd, pd = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(pos).to(dev())
    rows = sample_rows(wl.N, wl.T, wl.S, seed=3, n_random=32)
    ref = oracle.global_attn(q, k, v, wl.S, wl.T, pos=pos, rows=rows)
    outs = []
    for splits in (1, 2, 3, 7):
        go = ffv.vggt_global_attn(qd, kd, vd, pos_yx=pd, kv_splits=splits)
        outs.append(to_f64(go))
        check_bf16(outs[-1].reshape(wl.N, wl.H, 64)[rows], ref, f"s8 global splits={splits}")
    for splits, o in zip((2, 3, 7), outs[1:]):
        # different split counts only reorder fp32 sums: results agree to bf16 rounding
        check_same_up_to_sum_order(o, outs[0], f"s8 global splits={splits} vs 1")


def test_empty_batch_through_the_binding():
    # zero frames: empty CUDA tensors (null data pointers) in, empty results out
    e = [torch.empty(0, 8, 2, 64, dtype=torch.bfloat16, device=dev()) for _ in range(4)]
    q, k, v, g = e
    assert ffv.vggt_frame_attn(q, k, v).shape == (0, 8, 2, 64)
    assert ffv.vggt_global_attn(q, k, v).shape == (0, 8, 2, 64)
    o, lse = ffv.vggt_global_attn_train(q, k, v)
    assert o.shape == (0, 8, 2, 64) and lse.numel() == 0
    dq, dk, dv = ffv.vggt_global_attn_backward(q, k, v, o, g, lse)
    assert dq.shape == dk.shape == dv.shape == (0, 8, 2, 64)
    torch.cuda.synchronize()
