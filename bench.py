"""Benchmark of the alternating-attention hot path on one MI355X.

One step = one pass over every call of the path on one batch of 32 frames of
518x518 (VGGT-1B shape: 37x37 patches + 1 camera + 4 register tokens = 1374
tokens per frame, N = 43968, 16 heads of 64, bf16, 2D RoPE base 100):

  frame attention (RoPE)      32 x 1374^2           247.4 GFLOP
  global attention (RoPE)     43968^2              7917.8 GFLOP
  descriptor pooling of K, V  2x2 windows -> 32 x 366 descriptors
  descriptor cross-attention  43968 x 11712        2109.2 GFLOP

FLOP = 4 * Nq * Nk * H * 64 (QK^T plus PV, 2 flop per multiply-add).  Inputs
are seeded N(0,1) bf16 tensors already resident in HBM.  `value` is the
metric: global-attention TFLOP/s, the global call's FLOP over its mean
duration within the timed steps (the whole call: RoPE table, K/V tile passes,
attention kernel and any split merge); `step_tflops` is all of the step's
attention FLOP over the step time.  Per-call times come from HIP events
recorded on the launch stream.  The oracle (float64, CPU) is timed on a row
sample of the same step as the CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "global-attention TFLOP/s + ms/layer at S frames; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# HBM traffic of one global-attention kernel launch per workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs scaled by the counters' reading on a plain 1 GiB
# copy (profiles/attn_fwd_bf16_*_counters.md): (read bytes, written bytes).
# Valid only for the kernel source the counters were taken on.
PROFILED_TRAFFIC = {
    "kernel_source_sha256": "55696b166e80aa9e64ed8a746d201adfd896f2adb8ddbb04ac594f94cfcbbb9d",
    "vggt-518-s32": (1165.5e6, 90.0e6),
    "omega-512-s64": (2930.3e6, 920.1e6),
}


def attn_flops(nq: int, nk: int, H: int = 16, d: int = 64) -> float:
    return 4.0 * nq * nk * H * d


def kernel_source_sha256():
    """Hash of the attention kernel's source and of the header that fixes its LDS tile
    layout, without comments and blank lines, or None if they cannot be read."""
    import hashlib

    # the kernel's source and the header that fixes its LDS tile layout, without comments
    # and blank lines (the sources hold no "//" inside string literals)
    h = hashlib.sha256()
    try:
        for name in ("attn_bf16.hip", "common.h"):
            with open(os.path.join(ROOT, "feed_forward_view_amd", "csrc", name)) as f:
                for line in f:
                    code = line.split("//", 1)[0].rstrip()
                    if code:
                        h.update(code.encode() + b"\n")
    except OSError:
        return None
    return h.hexdigest()


def profiled_traffic(workload_name="vggt-518-s32"):
    """HBM bytes per global-attention launch on a workload if the kernel is the one the
    counters were taken on, else None."""
    if workload_name not in PROFILED_TRAFFIC or kernel_source_sha256() != PROFILED_TRAFFIC["kernel_source_sha256"]:
        return None
    return sum(PROFILED_TRAFFIC[workload_name])


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="vggt-518-s32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the FlashVGGT chunk-recursive measurement")
    ap.add_argument("--no-omega", action="store_true", help="skip the VGGT-Omega 64-frame measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the attention-gradient measurement")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step (no Q/K-norm, streaming or Omega sections)")
    ap.add_argument("--no-power", action="store_true", help="skip the socket power / clock sampling")
    ap.add_argument("--cpu-row-stride", type=int, default=48)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (hardware-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path has no multi-GPU execution in this library "
              "(see the sharding notes); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import feed_forward_view_amd as ffv
    import workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    wl = workload.WORKLOADS[args.workload]
    S, T, H, N = wl.S, wl.T, wl.H, wl.N
    ph, pw = 2, 2

    t0 = time.time()
    q, k, v = wl.qkv_bf16()
    gen_s = time.time() - t0
    pos = wl.positions()

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    posd = torch.from_numpy(pos).to(dev)
    Dn = ffv.vggt_descriptor_count(T, wl.gh, wl.gw, ph, pw)
    fo = torch.empty_like(qd)
    go = torch.empty_like(qd)
    xo = torch.empty_like(qd)
    kpool = torch.empty((S, Dn, H, 64), dtype=torch.bfloat16, device=dev)
    vpool = torch.empty_like(kpool)
    ws_f = torch.empty(max(1, ffv.vggt_frame_attn_workspace(S, T, H, True)), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(max(1, ffv.vggt_global_attn_workspace(S, T, H, 0, True)), dtype=torch.uint8, device=dev)
    ws_x = torch.empty(max(1, ffv.vggt_descriptor_xattn_workspace(S, T, Dn, H, 0)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    calls = ["frame", "global", "pool", "xattn"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        ffv.vggt_frame_attn(qd, kd, vd, out=fo, pos_yx=posd, rope_base=100.0, workspace=ws_f)
        mark(1)
        ffv.vggt_global_attn(qd, kd, vd, out=go, pos_yx=posd, rope_base=100.0, kv_splits=0, workspace=ws_g)
        mark(2)
        ffv.vggt_descriptor_pool(kd, vd, wl.gh, wl.gw, wl.patch_begin, ph, pw, kd=kpool, vd=vpool)
        mark(3)
        ffv.vggt_descriptor_xattn(qd, kpool, vpool, out=xo, kv_splits=0, workspace=ws_x)
        mark(4)

    if args.calibrate_copy_mib > 0:
        # plain copy kernels of known size for hardware-counter calibration:
        # an elementwise float32 copy (reads and writes N bytes each)
        n = (args.calibrate_copy_mib << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    # the library brackets each attention kernel launch with HIP events on the
    # call's stream: kernel-only durations inside the timed region
    ffv.vggt_timer_start(3 * args.steps)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kernel_ms = {}
    for kind, ms in ffv.vggt_timer_stop():
        kernel_ms.setdefault(kind, []).append(ms)

    per_call = {c: [] for c in calls}
    for ev in events:
        for j, c in enumerate(calls):
            per_call[c].append(ev[j].elapsed_time(ev[j + 1]))
    med = {c: float(np.median(x)) for c, x in per_call.items()}

    flops = {
        "frame": attn_flops(T, T, H) * S,
        "global": attn_flops(N, N, H),
        "xattn": attn_flops(N, S * Dn, H),
    }
    step_flops = sum(flops.values())
    ms_per_step = elapsed * 1e3 / args.steps
    step_tflops = step_flops / (ms_per_step * 1e-3) / 1e12
    g_call_ms = float(np.mean(per_call["global"]))
    value = flops["global"] / (g_call_ms * 1e-3) / 1e12
    g_tflops = flops["global"] / (med["global"] * 1e-3) / 1e12
    g_kernel_ms = float(np.mean(kernel_ms["global"]))
    g_kernel_tflops = flops["global"] / (g_kernel_ms * 1e-3) / 1e12
    pool_bytes = 2 * (S * T * H * 64 * 2) + 2 * (S * Dn * H * 64 * 2)  # read K, V; write Kd, Vd

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller N(0,1) Q/K/V, bf16)",
        "config": {
            "workload": f"{wl.name}: S={S} frames x T={T} tokens (37x37 patches + 1 camera + 4 register), "
                        f"N={N}, H={H}, d=64, RoPE base 100; step = frame + global attention + "
                        f"2x2 descriptor pool + descriptor cross-attention ({S * Dn} descriptors)",
            "S": S, "T": T, "N": N, "H": H, "head_dim": 64,
        },
        "value_definition": "global attention: 4*N^2*H*64 flop / mean duration of the vggt_global_attn call "
                            "within the timed steps (HIP events on its stream)",
        "step_tflops": round(step_tflops, 2),
        "ms_per_layer": round(med["frame"] + med["global"], 4),
        "calls_ms_median": {c: round(x, 4) for c, x in med.items()},
        "calls_ms_p10_p90": {c: [round(float(np.percentile(x, 10)), 4), round(float(np.percentile(x, 90)), 4)]
                             for c, x in per_call.items()},
        "global_attention_tflops_median_call": round(g_tflops, 2),
        "global_frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "frame_attention_tflops": round(flops["frame"] / (med["frame"] * 1e-3) / 1e12, 2),
        "xattn_tflops": round(flops["xattn"] / (med["xattn"] * 1e-3) / 1e12, 2),
        "pool_gbs": round(pool_bytes / (med["pool"] * 1e-3) / 1e9, 1),
        "attention_kernel_ms_mean": {c: round(float(np.mean(x)), 4) for c, x in kernel_ms.items()},
        "roofline": {
            "kernel": f"attn_fwd_bf16_kernel, global attention launch ({N} x {N} tokens, {H} heads of 64); "
                      f"4*N*N*H*64 flop per launch / mean kernel time from HIP events on its stream",
            "bound": "mfma",
            "achieved": round(g_kernel_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(g_kernel_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": profiled_traffic(),
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), "max_clock_mhz": _max_clock_mhz()},
        "input_gen_s": round(gen_s, 2),
        # SHA-256 of the host bf16 bit patterns of the headline inputs, for reproduction
        "input_sha256": {name: hashlib.sha256(a.tobytes()).hexdigest() for name, a in (("q", q), ("k", k), ("v", v))},
    }

    if not args.no_power:
        result["power"] = bench_power(ffv, qd, kd, vd, posd, ws_g, flops["global"], S, T, H)
    if not args.no_extras:
        result["qknorm"] = bench_qknorm(ffv, qd, kd, vd, posd, ws_g, ws_f, max(3, args.steps // 2), flops)
    if not args.no_extras:
        result["configs"] = bench_configs(ffv, dev, max(3, args.steps // 2), qd)
    if not (args.no_stream or args.no_extras):
        result["stream"] = bench_stream(ffv, dev, max(3, args.steps // 2), 2)
    if not args.no_extras:
        result["shard"] = bench_shard(ffv, qd, kd, vd, posd, max(5, args.steps // 2), flops["global"])
    if not (args.no_backward or args.no_extras):
        result["backward"] = bench_backward(ffv, qd, kd, vd, posd, max(3, args.steps // 4), flops)
    if not (args.no_omega or args.no_extras):
        result["omega"] = bench_omega(ffv, dev, max(3, args.steps // 4))
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(wl, q, k, v, pos, Dn, ph, pw, go, fo, xo,
                                                                       args.cpu_row_stride)
        # throughput ratio of the step on the GPU to the oracle on the host's cores
        result["gpu_over_cpu_oracle"] = round(step_tflops / result["cpu_baseline"]["value"], 1)
    print(json.dumps(result), flush=True)
    return 0


_FLUSH = None


def _max_clock_mhz():
    """Peak shader clock of device 0 from the HIP runtime (hipDeviceAttributeClockRate, kHz), or None."""
    import ctypes

    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) != 0:  # 5 = hipDeviceAttributeClockRate
            return None
        return khz.value // 1000
    except OSError:
        return None


def _flush_cache():
    """Read 1 GiB of device memory so that the 256 MB Infinity Cache holds none of the next
    call's inputs (HBM-bound measurements); a read leaves clean lines, so no write-back of
    the flush lands inside the timed call."""
    import torch

    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    _FLUSH.sum()


def _median_ms(fn, iters, warm=2, flush=False):
    """Median duration of fn() from HIP events on the current stream (optionally with the
    cache flushed before each timed call, outside the timed interval)."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warm):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        if flush:
            _flush_cache()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def bench_configs(ffv, dev, iters, qd):
    """The smaller workloads (4 frames at 224x224: N=1044; 8 frames at 518x518: N=10992):
    frame and global attention with RoPE, kernel times from the library timer (at N=10992
    also global attention on logits in the hundreds, where every workgroup reruns its key
    range exactly); and the
    standalone in-place RoPE pass on the S=32 Q tensor next to a plain device copy of the
    same bytes."""
    import torch

    import workload

    out = {}
    for name in ("vggt-224-s4", "vggt-518-s8"):
        wl = workload.WORKLOADS[name]
        S, T, H, N = wl.S, wl.T, wl.H, wl.N
        q, k, v = (torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16) for a in wl.qkv_bf16())
        pos = torch.from_numpy(wl.positions()).to(dev)
        o = torch.empty_like(q)
        ws_f = torch.empty(max(1, ffv.vggt_frame_attn_workspace(S, T, H, True)), dtype=torch.uint8, device=dev)
        ws_g = torch.empty(max(1, ffv.vggt_global_attn_workspace(S, T, H, 0, True)), dtype=torch.uint8, device=dev)
        res = {"S": S, "T": T, "N": N}
        for kind, fn, fl in (
                ("frame", lambda: ffv.vggt_frame_attn(q, k, v, out=o, pos_yx=pos, workspace=ws_f), attn_flops(T, T, H) * S),
                ("global", lambda: ffv.vggt_global_attn(q, k, v, out=o, pos_yx=pos, workspace=ws_g), attn_flops(N, N, H))):
            fn()
            torch.cuda.synchronize()
            ffv.vggt_timer_start(iters)
            call_ms = _median_ms(fn, iters, warm=0)
            kern = float(np.mean([ms for _, ms in ffv.vggt_timer_stop()]))
            res[f"{kind}_call_ms"] = round(call_ms, 4)
            res[f"{kind}_kernel_ms"] = round(kern, 4)
            res[f"{kind}_kernel_tflops"] = round(fl / (kern * 1e-3) / 1e12, 2)
            res[f"{kind}_kernel_frac_of_bf16_peak"] = round(fl / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        res["ms_per_layer"] = round(res["frame_call_ms"] + res["global_call_ms"], 4)
        if name == "vggt-518-s8":
            # worst case of the optimistic softmax pass: Q x 32 puts every row's largest logit
            # near 180 (log2 units), its weights overflow, and every workgroup reruns its key
            # range with the exact per-row reference
            qs = q * 32.0
            fn = lambda: ffv.vggt_global_attn(qs, k, v, out=o, pos_yx=pos, workspace=ws_g)
            fn()
            torch.cuda.synchronize()
            ffv.vggt_timer_start(iters)
            for _ in range(iters):
                fn()
            torch.cuda.synchronize()
            kern = float(np.mean([ms for _, ms in ffv.vggt_timer_stop()]))
            res["global_all_rerun_kernel_ms"] = round(kern, 4)
            res["global_all_rerun_over_optimistic"] = round(kern / res["global_kernel_ms"], 3)
        out[name] = res
    # standalone RoPE: read + write every Q element once
    wl = workload.WORKLOADS["vggt-518-s32"]
    x = qd.clone()
    pos = torch.from_numpy(wl.positions()).to(dev)
    rope_ms = _median_ms(lambda: ffv.vggt_attn_rope(x, pos), iters, flush=True)
    y = torch.empty_like(x)
    copy_ms = _median_ms(lambda: y.copy_(x), iters, flush=True)
    nbytes = 2 * x.numel() * x.element_size()
    out["rope_standalone"] = {
        "workload": f"vggt_attn_rope in place on Q of {wl.name} ({x.numel() * 2 / 1e6:.1f} MB read and written); "
                    f"1 GiB read before each timed call so the inputs come from HBM",
        "ms": round(rope_ms, 4),
        "gbs": round(nbytes / (rope_ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(nbytes / (rope_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "device_copy_gbs": round(nbytes / (copy_ms * 1e-3) / 1e9, 1),
    }
    return out


def bench_qknorm(ffv, qd, kd, vd, posd, ws_g, ws_f, iters, flops):
    """Frame and global attention of the same workload with the fused per-head
    Q/K LayerNorm + RoPE prologue (seeded gamma/beta around (1, 0)), into
    outputs of their own."""
    import torch

    import workload

    dev = qd.device
    fo, go = torch.empty_like(qd), torch.empty_like(qd)
    prm = [torch.from_numpy(workload.normal_f32(0x1A7E + i, (64,)) * 0.3 + (1.0 if i % 2 == 0 else 0.0)).to(dev)
           for i in range(4)]
    qn, kn = (prm[0], prm[1]), (prm[2], prm[3])
    stream = torch.cuda.current_stream()

    def call(kind):
        if kind == "frame":
            ffv.vggt_frame_attn_qknorm(qd, kd, vd, qn, kn, out=fo, pos_yx=posd, workspace=ws_f)
        else:
            ffv.vggt_global_attn_qknorm(qd, kd, vd, qn, kn, out=go, pos_yx=posd, workspace=ws_g)

    out = {}
    for kind in ("frame", "global"):
        for _ in range(2):
            call(kind)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        torch.cuda.synchronize()
        ffv.vggt_timer_start(iters)
        for a, b in ev:
            a.record(stream)
            call(kind)
            b.record(stream)
        torch.cuda.synchronize()
        kern = [ms for _, ms in ffv.vggt_timer_stop()]
        call_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        out[f"{kind}_call_ms"] = round(call_ms, 4)
        out[f"{kind}_kernel_ms"] = round(float(np.mean(kern)), 4)
        out[f"{kind}_call_tflops"] = round(flops[kind] / (call_ms * 1e-3) / 1e12, 2)
    return out


def bench_backward(ffv, qd, kd, vd, posd, iters, flops):
    """Gradients of global attention on the same workload (RoPE on): the
    training forward (output + log-normaliser) once, then the backward call
    timed, and its dQ and dK/dV kernels by the library's kernel timer.
    Algorithmic FLOP of the backward: the five N x N x 64 products of the
    chain rule per head (S, dP, dV, dQ, dK) = 2.5 x the forward's 4*N*N*H*64;
    the two kernels execute seven (S and dP are formed in both)."""
    import torch

    import workload

    S, T, H = qd.shape[0], qd.shape[1], qd.shape[2]
    dout = torch.from_numpy(workload.normal_bf16(0xBAC4, tuple(qd.shape)).view(np.int16)).to(qd.device).view(
        torch.bfloat16)
    o, lse = ffv.vggt_global_attn_train(qd, kd, vd, pos_yx=posd)
    grads = tuple(torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(max(1, int(ffv.lib().vggt_attn_backward_workspace(S, T, H, 1, 1, 0))), dtype=torch.uint8,
                     device=qd.device)
    stream = torch.cuda.current_stream()

    def call():
        ffv.vggt_global_attn_backward(qd, kd, vd, o, dout, lse, pos_yx=posd, workspace=ws, grads=grads)

    call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    ffv.vggt_timer_start(2 * iters)
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    kern = {}
    for kind, ms in ffv.vggt_timer_stop():
        kern.setdefault(kind, []).append(ms)
    call_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    bwd_flops = 2.5 * flops["global"]
    dq_ms, dkdv_ms = float(np.mean(kern["bwd_dq"])), float(np.mean(kern["bwd_dkdv"]))
    return {
        "workload": f"global attention gradients, S={S} x T={T}, H={H}, d=64, RoPE base 100, bf16",
        "algorithmic_tflop": round(bwd_flops / 1e12, 3),
        "call_ms": round(call_ms, 4),
        "call_tflops": round(bwd_flops / (call_ms * 1e-3) / 1e12, 2),
        "dq_kernel_ms": round(dq_ms, 4),
        "dkdv_kernel_ms": round(dkdv_ms, 4),
        "kernels_tflops": round(bwd_flops / ((dq_ms + dkdv_ms) * 1e-3) / 1e12, 2),
        "kernels_frac_of_bf16_peak": round(bwd_flops / ((dq_ms + dkdv_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }


def bench_shard(ffv, qd, kd, vd, posd, iters, flop_global, gpus=8, link_tbs=7 * 0.153):
    """One GPU's share of global attention on an 8-GPU node, at its real shape (nothing here
    uses a second GPU): (i) head-parallel, 16/8 = 2 heads of the whole 43968-token sequence
    (after an all-to-all from token shards to head shards); (ii) query-parallel, the queries
    of 32/8 = 4 frames against all keys (after an all-gather of K and V), run as the
    cross-attention launch with the 32 frames' rotated keys viewed as 4 groups of 10992.  RoPE
    is applied to that Q shard and to K before timing (the key owners rotate once per
    layer).  The exchange times are a model: bytes per GPU over 7 xGMI links of 153 GB/s,
    not measured."""
    import torch

    S, T, H = qd.shape[0], qd.shape[1], qd.shape[2]
    N = S * T
    out = {"gpus_modelled": gpus, "note": "kernels measured on one GPU at one GPU's share; exchange times modelled"}
    stream = torch.cuda.current_stream()

    def timed(fn, kind):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        ffv.vggt_timer_start(4 * iters)
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        kern = [ms for k, ms in ffv.vggt_timer_stop() if k == kind]
        return float(np.median([a.elapsed_time(b) for a, b in ev])), float(np.mean(kern))

    hs = H // gpus
    if hs >= 1 and H % gpus == 0:
        hq, hk, hv = (t[:, :, :hs].contiguous() for t in (qd, kd, vd))
        ho = torch.empty_like(hq)
        call, kern = timed(lambda: ffv.vggt_global_attn(hq, hk, hv, out=ho, pos_yx=posd, rope_base=100.0), "global")
        fl = flop_global * hs / H
        # sent per GPU: (gpus-1)/gpus of its token shard of Q, K and V, and of O on the way back
        xbytes = 4 * (N // gpus) * H * 64 * 2 * (gpus - 1) / gpus
        out["head_parallel"] = {
            "shape": f"[{S}, {T}, {hs}, 64] per GPU, N={N}", "tflop": round(fl / 1e12, 4),
            "call_ms": round(call, 4), "kernel_ms": round(kern, 4),
            "kernel_frac_of_bf16_peak": round(fl / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "exchange_mb_per_gpu": round(xbytes / 1e6, 1),
            "exchange_ms_model": round(xbytes / (link_tbs * 1e12) * 1e3, 4),
        }
    sq = S // gpus
    if sq >= 1 and S % gpus == 0:
        qs = qd[:sq].clone()
        ffv.vggt_attn_rope(qs, posd, rope_base=100.0)
        kr = kd.clone()
        ffv.vggt_attn_rope(kr, posd, rope_base=100.0)
        Dn = N // sq
        kv, vv = kr.view(sq, Dn, H, 64), vd.view(sq, Dn, H, 64)
        qo = torch.empty_like(qs)
        call, kern = timed(lambda: ffv.vggt_descriptor_xattn(qs, kv, vv, out=qo), "xattn")
        fl = flop_global / gpus
        # received per GPU: the other shards of K and V
        xbytes = 2 * N * H * 64 * 2 * (gpus - 1) / gpus
        out["query_parallel"] = {
            "shape": f"{sq * T} queries x {N} keys, H={H} per GPU", "tflop": round(fl / 1e12, 4),
            "call_ms": round(call, 4), "kernel_ms": round(kern, 4),
            "kernel_frac_of_bf16_peak": round(fl / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "exchange_mb_per_gpu": round(xbytes / 1e6, 1),
            "exchange_ms_model": round(xbytes / (link_tbs * 1e12) * 1e3, 4),
        }
    return out


def _smi_sample():
    """One `amd-smi metric -p -c` reading: (socket power W, mean gfx clock MHz over the XCDs), or None."""
    import subprocess

    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=5)
        if r.returncode != 0:
            return None
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = [v["clk"]["value"] for k, v in g["clock"].items()
               if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        return float(g["power"]["socket_power"]["value"]), float(sum(clk) / len(clk))
    except Exception:  # tool missing or output format differs: no sample
        return None


def _sustained_power(ffv, call, kinds, seconds, settle):
    """Run `call` back to back for `seconds` while a thread reads `amd-smi metric -p -c`
    every 0.1 s (after `settle` seconds, so the readings reflect the steady state).
    Returns (calls, mean socket W, mean gfx MHz, number of readings, mean ms per call,
    mean kernel ms per call summed over the timer kinds in `kinds`), or None without
    readings."""
    import threading

    import torch

    samples, stop = [], threading.Event()

    def sampler():
        t0 = time.perf_counter()
        while not stop.is_set():
            if time.perf_counter() - t0 >= settle:
                s = _smi_sample()
                if s is not None:
                    samples.append(s)
            stop.wait(0.1)

    call()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    ffv.vggt_timer_start(20000)  # kernel records: up to 10000 calls of at most two timed kernels
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds and n < 10000:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
        n += 8
    wall = time.perf_counter() - t0
    stop.set()
    th.join()
    kern = sum(ms for kind, ms in ffv.vggt_timer_stop() if kind in kinds) / n
    if not samples:
        return None
    return (n, float(np.mean([s[0] for s in samples])), float(np.mean([s[1] for s in samples])), len(samples),
            wall * 1e3 / n, kern)


def bench_power(ffv, qd, kd, vd, posd, ws_g, flop, S, T, H, seconds=2.5, settle=0.8):
    """Socket power and shader clock under sustained global attention, frame attention and
    the global-attention backward (each call back to back for `seconds`, amd-smi read
    every 0.1 s after `settle` seconds).  Kernel times of the same window come from the
    library's kernel timer.  From these: clock cycles per launch (mean kernel time x mean
    clock), energy per call (mean socket power x mean call time) and per algorithmic flop."""
    import torch

    if _smi_sample() is None:
        return None
    go = torch.empty_like(qd)
    r = _sustained_power(ffv, lambda: ffv.vggt_global_attn(qd, kd, vd, out=go, pos_yx=posd, rope_base=100.0,
                                                            kv_splits=0, workspace=ws_g),
                         ("global",), seconds, settle)
    if r is None:
        return None
    n, watts, mhz, ns, call_ms, kms = r
    out = {
        "what": "global attention (S=32 workload) back to back; amd-smi socket power and gfx clock, "
                "mean of the readings after the first %.1f s" % settle,
        "calls": n, "samples": ns,
        "socket_power_w": round(watts, 1),
        "gfx_clock_mhz": round(mhz),
        "kernel_ms": round(kms, 4),
        "kernel_frac_of_bf16_peak": round(flop / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "frac_of_peak_at_this_clock": round(flop / (kms * 1e-3) / 1e12 / (PEAK_BF16_TFLOPS * mhz / 2400.0), 4),
        "mcycles_per_launch": round(kms * 1e-3 * mhz * 1e6 / 1e6, 3),
        "joules_per_launch": round(watts * call_ms * 1e-3, 3),
        "pj_per_flop": round(watts * call_ms * 1e-3 / flop * 1e12, 3),
    }
    # frame attention of the same tensors, and the global-attention backward
    fo = torch.empty_like(qd)
    ws_f = torch.empty(max(1, ffv.vggt_frame_attn_workspace(S, T, H, True)), dtype=torch.uint8, device=qd.device)
    frame_flop = attn_flops(T, T, H) * S
    r = _sustained_power(ffv, lambda: ffv.vggt_frame_attn(qd, kd, vd, out=fo, pos_yx=posd, rope_base=100.0,
                                                           workspace=ws_f),
                         ("frame",), seconds, settle)
    if r is not None:
        n, watts, mhz, ns, call_ms, kms = r
        out["frame"] = {"calls": n, "samples": ns, "socket_power_w": round(watts, 1), "gfx_clock_mhz": round(mhz),
                        "call_ms": round(call_ms, 4), "kernel_ms": round(kms, 4),
                        "joules_per_call": round(watts * call_ms * 1e-3, 4),
                        "pj_per_flop": round(watts * call_ms * 1e-3 / frame_flop * 1e12, 3)}
    import workload

    dout = torch.from_numpy(workload.normal_bf16(0xBAC4, tuple(qd.shape)).view(np.int16)).to(qd.device).view(
        torch.bfloat16)
    o, lse = ffv.vggt_global_attn_train(qd, kd, vd, pos_yx=posd)
    grads = tuple(torch.empty_like(qd) for _ in range(3))
    ws_b = torch.empty(max(1, int(ffv.lib().vggt_attn_backward_workspace(S, T, H, 1, 1, 0))), dtype=torch.uint8,
                       device=qd.device)
    bwd_flop = 2.5 * flop
    r = _sustained_power(ffv, lambda: ffv.vggt_global_attn_backward(qd, kd, vd, o, dout, lse, pos_yx=posd,
                                                                     workspace=ws_b, grads=grads),
                         ("bwd_dq", "bwd_dkdv"), seconds, settle)
    if r is not None:
        n, watts, mhz, ns, call_ms, kms = r
        out["backward"] = {"calls": n, "samples": ns, "socket_power_w": round(watts, 1),
                           "gfx_clock_mhz": round(mhz), "call_ms": round(call_ms, 4),
                           "kernels_ms": round(kms, 4),
                           "joules_per_call": round(watts * call_ms * 1e-3, 3),
                           "pj_per_flop": round(watts * call_ms * 1e-3 / bwd_flop * 1e12, 3),
                           "pj_per_executed_flop": round(watts * call_ms * 1e-3 / (bwd_flop * 7 / 5) * 1e12, 3)}
    return out


def bench_omega(ffv, dev, iters):
    """VGGT-Omega, 64 frames of 32x32 patches + 16 registers (N = 66560): global
    attention with the registers in, and the register-free form with the 4
    storage + 1 camera extra tokens (65536 + 5 tokens)."""
    import torch

    import workload

    wl = workload.WORKLOADS["omega-512-s64"]
    S, T, H = wl.S, wl.T, wl.H
    Ta, E = wl.gh * wl.gw, 5
    q, k, v = wl.qkv_bf16()

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    del q, k, v
    x = [to_dev(workload.normal_bf16(0x0E6A5 + i, (E, H, 64))) for i in range(3)]
    pd = torch.from_numpy(wl.positions()).to(dev)
    out = torch.empty_like(qd)
    xo = torch.empty_like(x[0])
    ws_g = torch.empty(max(1, ffv.vggt_global_attn_workspace(S, T, H, 0, True)), dtype=torch.uint8, device=dev)
    ws_e = torch.empty(max(1, int(ffv.lib().vggt_global_attn_ex_workspace(S, T, Ta, E, H, 0, ffv.PRE_ROPE, 0))),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ws_f = torch.empty(max(1, ffv.vggt_frame_attn_workspace(S, T, H, True)), dtype=torch.uint8, device=dev)
    calls = {
        "frame": lambda: ffv.vggt_frame_attn(qd, kd, vd, out=out, pos_yx=pd, workspace=ws_f),
        "global": lambda: ffv.vggt_global_attn(qd, kd, vd, out=out, pos_yx=pd, workspace=ws_g),
        "global_ex": lambda: ffv.vggt_global_attn_ex(qd, kd, vd, Ta, *x, out=out, xout=xo, pos_yx=pd,
                                                     workspace=ws_e),
    }
    flops = {"frame": attn_flops(T, T, H) * S, "global": attn_flops(S * T, S * T, H),
             "global_ex": attn_flops(S * Ta + E, S * Ta + E, H)}
    res = {"workload": f"{wl.name}: S={S} frames x T={T} (32x32 patches + 16 registers), H={H}, d=64, RoPE base "
                       f"100; global_ex = {Ta} patch tokens per frame + {E} extra tokens"}
    for name, fn in calls.items():
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        torch.cuda.synchronize()
        ffv.vggt_timer_start(2 * iters)
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        kern = [ms for _, ms in ffv.vggt_timer_stop()]
        call_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        kernel_ms = float(np.sum(kern)) / iters  # global_ex: frame-token and extra-token launches
        res[f"{name}_call_ms"] = round(call_ms, 4)
        res[f"{name}_kernel_ms"] = round(kernel_ms, 4)
        res[f"{name}_kernel_tflops"] = round(flops[name] / (kernel_ms * 1e-3) / 1e12, 2)
        res[f"{name}_kernel_frac_of_bf16_peak"] = round(flops[name] / (kernel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    res["ms_per_layer"] = round(res["frame_call_ms"] + res["global_call_ms"], 4)
    g = flops["global"] / (res["global_kernel_ms"] * 1e-3) / 1e12
    res["roofline"] = {
        "kernel": f"attn_fwd_bf16_kernel, global attention launch ({S * T} x {S * T} tokens, {H} heads of 64); "
                  f"4*N*N*H*64 flop per launch / mean kernel time from HIP events on its stream",
        "bound": "mfma",
        "achieved": round(g, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(g / PEAK_BF16_TFLOPS, 4),
        "traffic": profiled_traffic("omega-512-s64"),
    }
    return res


def bench_stream(ffv, dev, passes, warmup, chunk_frames=10):
    """FlashVGGT chunk-recursive attention on the 100-frame workload: per chunk
    of 10 frames, pool its K/V into descriptors, append them to the cache and
    attend the chunk's queries to every cached descriptor; plus the same result
    for all chunks in one launch over the full cache."""
    import torch

    import workload

    wl = workload.WORKLOADS["flashvggt-518-s100"]
    S, T, H, F = wl.S, wl.T, wl.H, chunk_frames
    ph, pw = wl.pool
    q, k, v = wl.qkv_bf16()

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    del q, k, v
    Dn = ffv.vggt_descriptor_count(T, wl.gh, wl.gw, ph, pw)
    nch = (S + F - 1) // F
    kp = torch.empty((F, Dn, H, 64), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    cache = ffv.DescriptorCache(S * Dn, H, torch.bfloat16, device=dev)
    out = torch.empty_like(qd)
    ws_bytes = max(ffv.vggt_descriptor_cache_attn_workspace(F * T, min(S, (c + 1) * F) * Dn, H, 0)
                   for c in range(nch))
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def one_pass():
        cache.used = 0
        for c in range(nch):
            f0, f1 = c * F, min(S, (c + 1) * F)
            ffv.vggt_descriptor_pool(kd[f0:f1], vd[f0:f1], wl.gh, wl.gw, wl.patch_begin, ph, pw,
                                     kd=kp[:f1 - f0], vd=vp[:f1 - f0])
            cache.append(kp[:f1 - f0], vp[:f1 - f0])
            cache.attend(qd[f0:f1], out=out[f0:f1], workspace=ws)

    for _ in range(warmup):
        one_pass()
        cache.attend_chunked(qd, Dn, F, out=out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * passes)]
    ffv.vggt_timer_start(passes * (nch + 1))
    for i in range(passes):
        ev[2 * i][0].record(stream)
        one_pass()
        ev[2 * i][1].record(stream)
        ev[2 * i + 1][0].record(stream)
        cache.attend_chunked(qd, Dn, F, out=out)
        ev[2 * i + 1][1].record(stream)
    torch.cuda.synchronize()
    kern = {}
    for kind, ms in ffv.vggt_timer_stop():
        kern.setdefault(kind, []).append(ms)
    pass_ms = float(np.median([a.elapsed_time(b) for a, b in ev[0::2]]))
    chunked_ms = float(np.median([a.elapsed_time(b) for a, b in ev[1::2]]))

    # the single-forward form of the same workload: pool every frame, then all 137400 queries
    # against all 36600 descriptors
    kall = torch.empty((S, Dn, H, 64), dtype=torch.bfloat16, device=dev)
    vall = torch.empty_like(kall)
    ws_x = torch.empty(max(1, ffv.vggt_descriptor_xattn_workspace(S, T, Dn, H, 0)), dtype=torch.uint8, device=dev)
    pool_ms = _median_ms(lambda: ffv.vggt_descriptor_pool(kd, vd, wl.gh, wl.gw, wl.patch_begin, ph, pw, kd=kall,
                                                          vd=vall), passes, flush=True)
    ffv.vggt_timer_start(passes)
    xattn_ms = _median_ms(lambda: ffv.vggt_descriptor_xattn(qd, kall, vall, out=out, workspace=ws_x), passes,
                          warm=0)
    xk = [ms for _, ms in ffv.vggt_timer_stop()]
    x_flops = attn_flops(S * T, S * Dn, H)
    pool_bytes = 2 * S * T * H * 64 * 2 + 2 * S * Dn * H * 64 * 2
    flops = sum(attn_flops(min(F, S - c * F) * T, min(S, (c + 1) * F) * Dn, H) for c in range(nch))
    cache_kernel_ms = float(np.sum(kern["cache"])) / passes
    chunked_kernel_ms = float(np.mean(kern["chunked"]))
    return {
        "workload": f"{wl.name}: S={S} frames x T={T}, H={H}, d=64, 2x2 descriptors ({Dn} per frame), "
                    f"chunks of {F} frames; pass = per chunk pool + cache append + attention to the cache",
        "attention_tflop_per_pass": round(flops / 1e12, 4),
        "pass_ms": round(pass_ms, 4),
        "pass_tflops": round(flops / (pass_ms * 1e-3) / 1e12, 2),
        "cache_attention_kernel_ms_per_pass": round(cache_kernel_ms, 4),
        "chunked_one_launch_ms": round(chunked_ms, 4),
        "chunked_one_launch_tflops": round(flops / (chunked_ms * 1e-3) / 1e12, 2),
        "chunked_kernel_ms": round(chunked_kernel_ms, 4),
        "chunked_kernel_frac_of_bf16_peak": round(flops / (chunked_kernel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "single_forward": {
            "pool_ms": round(pool_ms, 4),
            "pool_gbs": round(pool_bytes / (pool_ms * 1e-3) / 1e9, 1),
            "pool_frac_of_hbm_peak": round(pool_bytes / (pool_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "xattn_tflop": round(x_flops / 1e12, 3),
            "xattn_call_ms": round(xattn_ms, 4),
            "xattn_kernel_ms": round(float(np.mean(xk)), 4),
            "xattn_kernel_tflops": round(x_flops / (float(np.mean(xk)) * 1e-3) / 1e12, 2),
            "xattn_kernel_frac_of_bf16_peak": round(x_flops / (float(np.mean(xk)) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
    }


def _cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, q, k, v, pos, Dn, ph, pw, go, fo, xo, stride):
    """The float64 oracle, untuned, on every `stride`-th query row of each
    attention call of the step, plus the pooling of every frame (the
    cross-attention rows need all descriptors), timed on the host cores."""
    import torch

    import oracle

    S, T, H, N = wl.S, wl.T, wl.H, wl.N
    nthreads = oracle.default_threads()
    rows = np.arange(0, N, stride, dtype=np.int64)
    t0 = time.perf_counter()
    ref_f = oracle.frame_attn(q, k, v, S, T, pos=pos, base=100.0, rows=rows, nthreads=nthreads)
    ref_g = oracle.global_attn(q, k, v, S, T, pos=pos, base=100.0, rows=rows, nthreads=nthreads)
    kp = oracle.descriptor_pool(k, S, T, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    vp = oracle.descriptor_pool(v, S, T, wl.gh, wl.gw, wl.patch_begin, ph, pw)
    ref_x = oracle.descriptor_xattn(q[:, :, :, :].reshape(N, H, 64)[rows], kp, vp, nthreads=nthreads)
    secs = time.perf_counter() - t0
    sampled_flops = rows.size * (attn_flops(1, T) + attn_flops(1, N) + attn_flops(1, S * Dn))
    base = {
        "value": round(sampled_flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": nthreads,
        "host_threads": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"every {stride}th query row ({rows.size} of {N}) of frame, global and descriptor attention, "
                  f"all heads, plus full descriptor pooling; {secs:.1f} s",
    }

    def host(t):
        return oracle.to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(N, H, 64)[rows]

    par = {}
    for name, got, ref in (("frame", fo, ref_f), ("global", go, ref_g), ("xattn", xo, ref_x)):
        err = np.abs(host(got) - ref.reshape(rows.size, H, 64))
        r = ref.reshape(rows.size, H, 64)
        par[name] = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                     "nrmse": float(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(r ** 2)))}
    return base, par


if __name__ == "__main__":
    sys.exit(main())
