"""Seeded synthetic inputs for the low-bit decode QMV workloads.

This module draws random numbers in the shapes, layouts and value
distributions of the decode workloads and nothing else: it never unpacks a
code, dequantizes a weight or forms a product.  Both sides of every parity
check (the CPU oracle and the HIP library) are fed from here.

Storage layouts (the readings used throughout the repository):

* ``u1`` / ``u2``: uint32 words ``[N][K*bits/32]``.  Codes are uniform over
  ``{0 .. 2^bits-1}`` and independent, which is exactly what uniformly random
  32-bit words give, so the words are drawn directly.
* ``t5``: uint8 ``[N][(K/gs) * ceil(gs/5)]``.  Each group of ``gs`` weights
  owns ``ceil(gs/5)`` bytes (13 for gs=64, 26 for gs=128); every full byte
  carries five base-3 digits, so it is uniform on ``[0, 243)``; the last byte
  of a group carries only ``gs mod 5`` digits and its unused digits are zero,
  so it is uniform on ``[0, 3^(gs mod 5))``.
* scales: fp16 ``[N][K/gs]`` uniform on [0.01, 0.05].  For 2-bit weights whose
  bias is implied as ``-1.5*scale`` the two low mantissa bits are cleared so
  that the implied bias is an exact fp16 number.
* biases: fp16 ``[N][K/gs]`` uniform on [-0.05, 0.05] (affine variant only;
  the symmetric and ternary variants store none).
* x: fp16 ``[M][K]`` standard normal.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass
from typing import Optional

import numpy as np

FORMATS = ("u1", "u2", "t5")

# The seven projection shapes (N x K) of a hidden=5120 decoder layer.
PROJECTION_SHAPES = {
    "q": (6144, 5120),
    "k": (1024, 5120),
    "v": (1024, 5120),
    "o": (5120, 6144),
    "gate": (17408, 5120),
    "up": (17408, 5120),
    "down": (5120, 17408),
}
LARGE_SHAPES = ("gate", "up", "down", "q", "o")


def seed_for(*key) -> int:
    """Stable 63-bit seed from any tuple of printable values."""
    h = hashlib.sha256(repr(tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") >> 1


def t5_bytes_per_group(group_size: int) -> int:
    return -(-group_size // 5)


def packed_row_bytes(fmt: str, K: int, group_size: int) -> int:
    if fmt == "u1":
        return K // 8
    if fmt == "u2":
        return K // 4
    if fmt == "t5":
        return (K // group_size) * t5_bytes_per_group(group_size)
    raise ValueError(f"unknown format {fmt!r}")


@dataclass
class QmvInputs:
    fmt: str
    M: int
    N: int
    K: int
    group_size: int
    variant: str  # "asym", "sym" (implied bias) or "t5" (implied bias)
    x: np.ndarray  # fp16 [M][K]
    w: np.ndarray  # uint32 [N][K*bits/32] or uint8 [N][row_bytes]
    scales: np.ndarray  # fp16 [N][K/gs]
    biases: Optional[np.ndarray]  # fp16 [N][K/gs] or None when implied

    @property
    def bits(self) -> int:
        return {"u1": 1, "u2": 2, "t5": 0}[self.fmt]


def draw_x(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def draw_scales(rng, N: int, G: int, trim_low_bits: int = 0) -> np.ndarray:
    s = rng.uniform(0.01, 0.05, size=(N, G)).astype(np.float16)
    if trim_low_bits:
        mask = np.uint16((0xFFFF << trim_low_bits) & 0xFFFF)
        s = (s.view(np.uint16) & mask).view(np.float16)
    return s


def draw_biases(rng, N: int, G: int) -> np.ndarray:
    return rng.uniform(-0.05, 0.05, size=(N, G)).astype(np.float16)


def draw_words(rng, N: int, K: int, bits: int) -> np.ndarray:
    words_per_row = K * bits // 32
    return rng.integers(0, 2**32, size=(N, words_per_row), dtype=np.uint64).astype(np.uint32)


def draw_t5_bytes(rng, N: int, K: int, group_size: int) -> np.ndarray:
    G = K // group_size
    gb = t5_bytes_per_group(group_size)
    tail_digits = group_size - 5 * (gb - 1)
    out = rng.integers(0, 243, size=(N, G, gb), dtype=np.int32)
    out[:, :, gb - 1] = rng.integers(0, 3**tail_digits, size=(N, G), dtype=np.int32)
    return out.astype(np.uint8).reshape(N, G * gb)


def make_inputs(fmt: str, M: int, N: int, K: int, group_size: int,
                variant: str = "asym", seed: int = 0) -> QmvInputs:
    """Draw one complete QMV input set.

    ``variant``: "asym" draws biases; "sym" stores none (bias implied as
    -scale*(2^bits-1)/2); for ``fmt == "t5"`` the bias is implied as -scale
    unless ``variant == "asym"`` asks for explicit biases.
    """
    if fmt not in FORMATS:
        raise ValueError(fmt)
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    rng = np.random.Generator(np.random.PCG64(seed_for("qmv", fmt, M, N, K, group_size, variant, seed)))
    G = K // group_size
    x = draw_x(rng, M, K)
    if fmt == "t5":
        w = draw_t5_bytes(rng, N, K, group_size)
    else:
        w = draw_words(rng, N, K, 1 if fmt == "u1" else 2)
    trim = 2 if (fmt == "u2" and variant == "sym") else 0
    scales = draw_scales(rng, N, G, trim)
    if variant == "asym":
        biases = draw_biases(rng, N, G)
    elif variant in ("sym", "t5"):
        biases = None
    else:
        raise ValueError(variant)
    return QmvInputs(fmt, M, N, K, group_size, variant, x, w, scales, biases)


def default_variant(fmt: str) -> str:
    return "t5" if fmt == "t5" else "asym"
