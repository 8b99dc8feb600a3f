"""GPU parity when the scores leave the range in which the bf16 kernels'
softmax reference stays at zero.

Unit-normal inputs at the default scale keep every row's scores within a few
units of zero, so they never exercise three exact paths of the online softmax
(the normalised-exponential step that the VGGT pages' attention layers compute):

* sharp rows: logits in the hundreds, so a tile maximum moves the row
  reference during the key loop and the running O and l are rescaled;
* rows whose scores all lie far below zero, so the first tile moves the
  reference down and the log-normaliser is far below zero;
* a row maximum that first appears in a late (or the last, masked) key tile;
* only some rows sharp (one frame's queries scaled up), so some workgroups
  rerun exactly and others keep their optimistic result, and split partials
  with and without a reference are merged;
* frames whose row sums sit just inside and just outside the optimistic
  pass's acceptance bound, so results from both sides of it are compared.

Split launches then merge partials whose references differ by hundreds.

The scale is 8 ln 2 (or ln 2 / 8 for the offset, mixed and edge cases), which makes
scale * log2(e) = 8 (1/8) to within a float32 ulp.  The kernels' scaled bf16
query operand is then exact, and the comparison sees only the softmax
arithmetic.  Bars:

* bf16: as in the other parity tests;
* the gradients: as in the backward tests.  They are checked on the sharp,
  late and offset cases.  In the all-negative case nearly every row is
  one-hot: its score gradient P (dP - D) cancels to the rounding of the
  stored bf16 output inside D, for any bf16 flash backward, so that case is
  a forward-only test;
* the fp32 debug mode: float32 dot products of 64 terms give scores of
  magnitude |s| an error of about 64 * 2^-24 * |s| (natural-log units), which
  is the relative error of the weights; the NRMSE bar is that bound at the
  largest |s| of the case, and the log-normaliser bar is the same absolute
  bound.
"""
import numpy as np
import pytest
import torch

import feed_forward_view_amd as ffv
import oracle
import workload
from checks import check_bf16
from test_gpu_parity import dev, to_dev, to_f64
from test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu

SHARP = float(np.float32(8.0 * np.log(2.0)))
MILD = float(np.float32(np.log(2.0) / 8.0))
KINDS = ["sharp", "negative", "late", "offset", "mixed", "edge"]
MILD_KINDS = ("offset", "mixed", "edge")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ffv.lib()
    yield
    torch.cuda.synchronize()


def _case(kind, dtype):
    """3 frames of 86 tokens (9 x 9 patches + 5 special), 2 heads."""
    wl = workload.Workload("t", 71, S=3, gh=9, gw=9, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_bf16()
    if kind == "negative":
        # q >= 0 >= k in every channel: each score is a sum of 64 non-positive
        # products, about -40 +- 8, i.e. -330 +- 60 in log2 units after the scale
        q = q & np.uint16(0x7FFF)
        k = k | np.uint16(0x8000)
    elif kind == "offset":
        # channel 63 of every query is +256 and of every key -12: each score
        # gets -3072 (-384 in log2 units at scale ln2/8) on top of an ordinary
        # unit-spread score, so whole rows sit far below zero without being
        # sharp.  A component shared by all keys drops out of dQ exactly (a
        # row's score gradients sum to zero) but in bf16 only up to their
        # rounding, times that component; the offset therefore sits mostly on
        # the query side, where it is a genuine part of dK.
        qf, kf = workload.bf16_bits_to_f32(q), workload.bf16_bits_to_f32(k)
        qf[..., 63] = 256.0
        kf[..., 63] = -12.0
        q, k = workload.f32_to_bf16_bits(qf), workload.f32_to_bf16_bits(kf)
    elif kind == "mixed":
        # frame 1's queries x 64: their scores spread over hundreds of log2 units
        qf = workload.bf16_bits_to_f32(q)
        qf[1] *= 64.0
        q = workload.f32_to_bf16_bits(qf)
    elif kind == "edge":
        # channel 63: query 31, 35, 37 in frames 0, 1, 2 and key -16, so frame
        # f's scores sit near -62, -70, -74 log2 units and its frame-attention
        # row sums near 2^-55, 2^-63.2 and 2^-67.3: frame 1 is just inside the
        # optimistic pass's bound (2^-64), frame 2 just outside
        qf, kf = workload.bf16_bits_to_f32(q), workload.bf16_bits_to_f32(k)
        for f, c in enumerate((31.0, 35.0, 37.0)):
            qf[f, :, :, 63] = c
        kf[..., 63] = -16.0
        q, k = workload.f32_to_bf16_bits(qf), workload.f32_to_bf16_bits(kf)
    elif kind == "late":
        # key 70 of frame 2 (global key 242, in the fourth of five key tiles;
        # frame-local key 70 is in the last, masked tile) gets 4x the scores
        kf = workload.bf16_bits_to_f32(k)
        kf[2, 70] *= 4.0
        k = workload.f32_to_bf16_bits(kf)
    if dtype == torch.float32:
        q, k, v = (workload.bf16_bits_to_f32(x) for x in (q, k, v))
    scale = MILD if kind in MILD_KINDS else SHARP
    return wl, q, k, v, scale


def _score_bound(q, k, S, T, glob, scale):
    """Largest |scale <q, k>| over the case's (query, key) pairs, natural-log units."""
    qf, kf = oracle.to_f64(q), oracle.to_f64(k)
    if glob:
        s = np.einsum("ihd,jhd->hij", qf.reshape(S * T, -1, 64), kf.reshape(S * T, -1, 64))
    else:
        s = np.einsum("fihd,fjhd->fhij", qf, kf)
    return scale * float(np.abs(s).max())


def _check_f32(got, ref, label, smax):
    bar = 64 * 2.0 ** -24 * smax
    diff = got.reshape(ref.shape) - ref
    nrmse = float(np.sqrt(np.mean(diff ** 2)) / np.sqrt(np.mean(ref ** 2)))
    print(f"{label}: nrmse {nrmse:.3e} (bar {bar:.3e}, max |s| {smax:.1f})")
    assert np.isfinite(got).all() and nrmse <= bar, label


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", KINDS)
def test_softmax_range_forward(kind, dtype):
    wl, q, k, v, SCALE = _case(kind, dtype)
    S, T = wl.S, wl.T
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    bf16 = dtype == torch.bfloat16
    tag = f"{kind} {'bf16' if bf16 else 'f32'}"

    fo = ffv.vggt_frame_attn(qd, kd, vd, scale=SCALE)
    ref = oracle.frame_attn(q, k, v, S, T, scale=SCALE)
    if bf16:
        check_bf16(to_f64(fo), ref, f"frame {tag}")
    else:
        _check_f32(to_f64(fo), ref, f"frame {tag}", _score_bound(q, k, S, T, False, SCALE))

    ref = oracle.global_attn(q, k, v, S, T, scale=SCALE)
    smax = _score_bound(q, k, S, T, True, SCALE)
    for splits in (1, 3):
        go = ffv.vggt_global_attn(qd, kd, vd, scale=SCALE, kv_splits=splits)
        if bf16:
            check_bf16(to_f64(go), ref, f"global {tag} splits={splits}")
        else:
            _check_f32(to_f64(go), ref, f"global {tag} splits={splits}", smax)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", ["sharp", "late", "offset", "mixed"])
def test_softmax_range_backward(kind, dtype):
    wl, q, k, v, SCALE = _case(kind, dtype)
    S, T, H = wl.S, wl.T, wl.H
    gen = workload.normal_bf16 if dtype == torch.bfloat16 else workload.normal_f32
    g = gen(0xD0D7, (S, T, H, 64))
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    bf16 = dtype == torch.bfloat16
    tag = f"{kind} {'bf16' if bf16 else 'f32'}"
    o, lse = ffv.vggt_global_attn_train(qd, kd, vd, scale=SCALE, kv_splits=3)
    dq, dk, dv = ffv.vggt_global_attn_backward(qd, kd, vd, o, gd, lse, scale=SCALE)
    rq, rk, rv, rl = oracle.global_attn_backward(q, k, v, g, S, T, scale=SCALE)
    smax = _score_bound(q, k, S, T, True, SCALE)
    lerr = float(np.abs(lse.cpu().numpy().astype(np.float64) - rl).max())
    lbar = 1e-2 if bf16 else 64 * 2.0 ** -24 * smax
    print(f"{tag} lse: max_abs {lerr:.3e} (bar {lbar:.3e}; lse range {rl.min():.1f} .. {rl.max():.1f})")
    assert lerr <= lbar
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        if bf16:
            check_grad(to_f64(got), ref, f"{tag} {name}", True)
        else:
            _check_f32(to_f64(got), ref, f"{tag} {name}", smax)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", ["sharp", "negative", "plain"])
def test_single_tile_key_range(kind, dtype):
    """Key ranges of one 64-key tile (frames of 7 x 7 patches + 5 special = 54 tokens;
    global attention over one frame): the first tile is also the last, in the optimistic
    pass and, for the sharp and all-negative rows, in the exact rerun."""
    wl = workload.Workload("t", 73, S=2, gh=7, gw=7, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_bf16()
    if kind == "negative":
        q = q & np.uint16(0x7FFF)
        k = k | np.uint16(0x8000)
    scale = SHARP if kind != "plain" else float(np.float32(0.125))
    bf16 = dtype == torch.bfloat16
    if not bf16:
        q, k, v = (workload.bf16_bits_to_f32(x) for x in (q, k, v))
    S, T = wl.S, wl.T
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    tag = f"{kind} {'bf16' if bf16 else 'f32'}"
    fo = ffv.vggt_frame_attn(qd, kd, vd, scale=scale)
    ref = oracle.frame_attn(q, k, v, S, T, scale=scale)
    if bf16:
        check_bf16(to_f64(fo), ref, f"frame one tile {tag}")
    else:
        _check_f32(to_f64(fo), ref, f"frame one tile {tag}", _score_bound(q, k, S, T, False, scale))
    # one frame as the global sequence: N = 54 keys, one tile
    q1, k1, v1 = q[:1], k[:1], v[:1]
    go = ffv.vggt_global_attn(to_dev(q1), to_dev(k1), to_dev(v1), scale=scale)
    ref = oracle.global_attn(q1, k1, v1, 1, T, scale=scale)
    if bf16:
        check_bf16(to_f64(go), ref, f"global one tile {tag}")
    else:
        _check_f32(to_f64(go), ref, f"global one tile {tag}", _score_bound(q1, k1, 1, T, True, scale))


VSHIFT = 34  # V scaled by 2^34


def _large_value_case(dtype):
    """3 frames of 86 tokens, 2 heads: channel 63 is 256 on every query and
    2.8125 on every key, so at scale ln2/8 each score sits near 90 log2 units
    and every row's sum of weights 2^s lies in [2^96.5, 2^98.7], inside the
    optimistic pass's bound on the row sum.  V is scaled by 2^34, so the
    un-normalised outputs sum_j 2^s_j v_j exceed 2^128 in every row: the
    optimistic pass overflows float32 and must hand the rows to the exact pass
    (weights <= 1), whose accumulators stay below keys * max|V|."""
    wl = workload.Workload("t", 72, S=3, gh=9, gw=9, n_special=5, patch_begin=5, H=2)
    q, k, v = wl.qkv_bf16()
    qf, kf, vf = (workload.bf16_bits_to_f32(x) for x in (q, k, v))
    qf[..., 63] = 256.0
    kf[..., 63] = 2.8125
    vf = vf * np.float32(2.0 ** VSHIFT)
    q, k, v = (workload.f32_to_bf16_bits(x) for x in (qf, kf, vf))  # exact: powers of two and 8-bit values
    if dtype == torch.float32:
        q, k, v = (workload.bf16_bits_to_f32(x) for x in (q, k, v))
    return wl, q, k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_values_leave_the_optimistic_pass(dtype):
    wl, q, k, v = _large_value_case(dtype)
    S, T = wl.S, wl.T
    # the case does what it says: row sums inside the bound, un-normalised outputs beyond float32
    qf, kf, vf = (oracle.to_f64(x).reshape(S * T, 2, 64) for x in (q, k, v))
    p = np.exp2(np.einsum("ihd,jhd->hij", qf, kf) * (MILD / np.log(2.0)))
    assert np.log2(p.sum(-1)).max() < 100
    assert (np.abs(np.einsum("hij,jhd->hid", p, vf)).max(-1) > 2.0 ** 128).all()
    unit = 2.0 ** -VSHIFT
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    bf16 = dtype == torch.bfloat16
    smax = _score_bound(q, k, S, T, True, MILD)
    check = check_bf16 if bf16 else (lambda g, r, lab: _check_f32(g, r, lab, smax))
    fo = to_f64(ffv.vggt_frame_attn(qd, kd, vd, scale=MILD))
    check(fo * unit, oracle.frame_attn(q, k, v, S, T, scale=MILD) * unit, f"large V frame {dtype}")
    ref = oracle.global_attn(q, k, v, S, T, scale=MILD) * unit
    for splits in (1, 3):
        go = to_f64(ffv.vggt_global_attn(qd, kd, vd, scale=MILD, kv_splits=splits))
        check(go * unit, ref, f"large V global {dtype} splits={splits}")
