"""Seeded synthetic inputs shared by the GPU library's tests/benchmark and the oracle.

This module holds no arithmetic of the attention method itself: it only draws
seeded normal numbers, rounds them to the storage dtype and lays out the
per-frame token positions and shapes of the workloads.

Workload shapes follow the pages:
  * VGGT-JAX README ("VGGT in JAX and Flax NNX"), attention kernel-trial table:
    tokens laid out [B, N, H=16, D=64]; a frame is its patch grid plus one
    camera and four register tokens (930 = 25*37 + 5 at 350x518, patch 14).
  * VGGT-Omega-1B-512-bf16 config article: 512 input, patch 16 -> 32x32 grid,
    16 register tokens appended after the patches, rope_base 100.
  * FlashVGGT README, Key Arguments: kv_downfactor 4 (a 2x2 window).

Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) used as a counter-based stream -- output n
(n = 1, 2, ...) of a stream with seed s is mix(s + n * 0x9E3779B97F4A7C15) --
turned into uniform (0, 1] doubles from the top 53 bits, then into normal pairs
by the Box-Muller transform (Box & Muller, 1958), rounded to float32 and then
to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import hashlib
import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SEED_BASE = 0x5EED0000


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start+1 .. start+count of the SplitMix64 stream with `seed`."""
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + n * GOLDEN
        return _mix64(z)


def _workers() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def normal_f64(seed: int, count: int, chunk: int = 1 << 21) -> np.ndarray:
    """`count` standard normal doubles: element 2j and 2j+1 come from the pair
    (u1, u2) = outputs (2j+1, 2j+2) of the stream, via Box-Muller.  Chunks are
    independent (counter-based stream), so they are filled by a thread pool."""
    out = np.empty(count, dtype=np.float64)
    npairs = (count + 1) // 2

    def fill(p0: int) -> None:
        p1 = min(npairs, p0 + chunk)
        r = splitmix64(seed, 2 * p0, 2 * (p1 - p0))
        u = ((r >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
        u1, u2 = u[0::2], u[1::2]
        rad = np.sqrt(-2.0 * np.log(u1))
        ang = 2.0 * np.pi * u2
        lo = 2 * p0
        hi = min(count, 2 * p1)
        z = np.empty(2 * (p1 - p0), dtype=np.float64)
        z[0::2] = rad * np.cos(ang)
        z[1::2] = rad * np.sin(ang)
        out[lo:hi] = z[: hi - lo]

    starts = range(0, npairs, chunk)
    if npairs <= chunk:
        for p0 in starts:
            fill(p0)
    else:
        with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, starts))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, shape) -> np.ndarray:
    """Seeded N(0,1) tensor as bf16 bit patterns (uint16) of the given shape."""
    n = int(np.prod(shape))
    return f32_to_bf16_bits(normal_f64(seed, n).astype(np.float32)).reshape(shape)


def normal_f32(seed: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return normal_f64(seed, n).astype(np.float32).reshape(shape)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------
# Token positions per frame, int32 [T, 2] = (row, col); tokens outside the
# patch grid sit at (0, 0).
# --------------------------------------------------------------------------

def positions(T: int, gh: int, gw: int, patch_begin: int) -> np.ndarray:
    pos = np.zeros((T, 2), dtype=np.int32)
    r, c = np.meshgrid(np.arange(gh, dtype=np.int32), np.arange(gw, dtype=np.int32), indexing="ij")
    pos[patch_begin : patch_begin + gh * gw, 0] = r.reshape(-1)
    pos[patch_begin : patch_begin + gh * gw, 1] = c.reshape(-1)
    return pos


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based workload number; seeds derive from it
    S: int              # frames
    gh: int             # patch grid rows
    gw: int             # patch grid cols
    n_special: int      # camera/register tokens per frame
    patch_begin: int    # index of the first patch token in a frame
    H: int = 16
    D: int = 64
    rope_base: float | None = 100.0
    pool: tuple[int, int] | None = None   # (ph, pw) window for descriptor pooling

    @property
    def T(self) -> int:
        return self.gh * self.gw + self.n_special

    @property
    def N(self) -> int:
        return self.S * self.T

    def seed(self, which: str) -> int:
        return SEED_BASE + 16 * self.index + {"q": 0, "k": 1, "v": 2}[which]

    def positions(self) -> np.ndarray:
        return positions(self.T, self.gh, self.gw, self.patch_begin)

    def qkv_bf16(self, S: int | None = None):
        """Q, K, V as bf16 bit patterns [S, T, H, D] (S defaults to the
        workload's frame count; a smaller S gives the leading frames)."""
        S = self.S if S is None else S
        shape = (S, self.T, self.H, self.D)
        return tuple(normal_bf16(self.seed(w), shape) for w in ("q", "k", "v"))

    def qkv_f32(self, S: int | None = None):
        S = self.S if S is None else S
        shape = (S, self.T, self.H, self.D)
        return tuple(normal_f32(self.seed(w), shape) for w in ("q", "k", "v"))


# The five workloads: (1) 4 frames of 224x224 at patch 14; (2) VGGT-1B, 8 frames
# of 518x518; (3) VGGT-1B at 32 frames; (4) VGGT-Omega-style 64 frames of
# 512x512 at patch 16 with 16 registers appended; (5) FlashVGGT-style 100 frames
# of 518x518 with 2x2 descriptor pooling and no RoPE.
WORKLOADS = {
    "vggt-224-s4": Workload("vggt-224-s4", 1, S=4, gh=16, gw=16, n_special=5, patch_begin=5),
    "vggt-518-s8": Workload("vggt-518-s8", 2, S=8, gh=37, gw=37, n_special=5, patch_begin=5),
    "vggt-518-s32": Workload("vggt-518-s32", 3, S=32, gh=37, gw=37, n_special=5, patch_begin=5),
    "omega-512-s64": Workload("omega-512-s64", 4, S=64, gh=32, gw=32, n_special=16, patch_begin=0),
    "flashvggt-518-s100": Workload("flashvggt-518-s100", 5, S=100, gh=37, gw=37, n_special=5,
                                   patch_begin=5, rope_base=None, pool=(2, 2)),
}
