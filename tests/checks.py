"""Comparison bars of the parity tests (host-side numpy only, no GPU).

bf16 outputs against the float64 oracle, per output tensor:
  * max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3: the absolute
    bars stated for unit-normal Q/K/V;
  * NRMSE = sqrt(mean(err^2)) / sqrt(mean(ref^2)) <= 1e-2: the parity metric of
    the VGGT-JAX README (parity section), which scales with the output.  At
    N = 43968 the outputs are about 0.008 rms and 0.04 at most, so the absolute
    bars alone cannot see a lost 64-key tile (NRMSE 3.7e-2 there, see
    tests/test_oracle.py); the kernels measure 2-4e-3;
  * max |gpu - oracle| <= 0.25 rms(ref): no single element is off by a sizeable
    fraction of the output scale (a wrong row or head cannot hide in the mean).
fp32 debug outputs: NRMSE <= 1e-5.

Two GPU results that differ only in the order of their fp32 sums (key split
count, frame order, an equivalent launch form) are compared element by element
within a few bf16 units in the last place of the larger of the two, plus an
absolute floor far below any output scale.
"""
from __future__ import annotations

import numpy as np

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
BF16_NRMSE = 1e-2
BF16_MAX_OVER_RMS = 0.25
F32_NRMSE = 1e-5


def nrmse(got: np.ndarray, ref: np.ndarray) -> float:
    diff = got.reshape(ref.shape) - ref
    return float(np.sqrt(np.mean(diff ** 2)) / max(float(np.sqrt(np.mean(ref ** 2))), 1e-30))


def bf16_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got.reshape(ref.shape) - ref)
    rms = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "nrmse": nrmse(got, ref),
            "max_over_rms": float(err.max()) / rms}


def bf16_absolute_ok(e: dict) -> bool:
    """The absolute bars alone."""
    return e["max_abs"] <= BF16_MAX and e["mean_abs"] <= BF16_MEAN


def bf16_ok(e: dict) -> bool:
    return bf16_absolute_ok(e) and e["nrmse"] <= BF16_NRMSE and e["max_over_rms"] <= BF16_MAX_OVER_RMS


def check_bf16(got: np.ndarray, ref: np.ndarray, label: str) -> dict:
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    e = bf16_errors(got, ref)
    print(f"{label}: max_abs {e['max_abs']:.3e} mean_abs {e['mean_abs']:.3e} nrmse {e['nrmse']:.3e} "
          f"max/rms {e['max_over_rms']:.3e} (ref max {np.abs(ref).max():.3f})")
    assert bf16_ok(e), f"{label}: {e}"
    return e


def check_f32(got: np.ndarray, ref: np.ndarray, label: str) -> float:
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    r = nrmse(got, ref)
    print(f"{label}: nrmse {r:.3e} max_abs {np.abs(got.reshape(ref.shape) - ref).max():.3e}")
    assert r <= F32_NRMSE, f"{label}: nrmse {r:.3e}"
    return r


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 (8 significant bits) at |x| (normal range)."""
    mag = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(mag)) - 7)


def check_same_up_to_sum_order(a: np.ndarray, b: np.ndarray, label: str, ulps: float = 2.0,
                               floor: float = 2.0 ** -20) -> None:
    """a and b (float64 copies of bf16 results) agree element-wise within `ulps`
    bf16 ulps of the larger magnitude plus `floor`."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64).reshape(a.shape)
    tol = ulps * bf16_ulp(np.maximum(np.abs(a), np.abs(b))) + floor
    d = np.abs(a - b)
    worst = float((d / tol).max()) if d.size else 0.0
    same = float(np.mean(d == 0)) if d.size else 1.0
    print(f"{label}: max diff {d.max() if d.size else 0:.3e}, worst / tolerance {worst:.3f}, identical {same:.4f}")
    assert worst <= 1.0, f"{label}: differs beyond {ulps} bf16 ulps (worst ratio {worst:.3f})"
