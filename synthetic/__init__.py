"""Seeded synthetic inputs, shared by the CPU oracle side and the GPU side.

This module draws random numbers and rounds them to the storage type. It holds
none of the attention arithmetic (no normalisation, rotation, masking or
softmax): both sides receive the exact same bytes from here and compute on their
own.

Generator: NumPy PCG64 seeded per workload, ``standard_normal`` in float32,
then round-to-nearest-even to bfloat16 where the workload stores bfloat16.
"""

from __future__ import annotations

import numpy as np

BASE_SEED = 20261202


def generator(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(gen: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits.

    Inputs are finite (drawn from a normal distribution), so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16."""
    return bf16_bits_to_f32(bf16_bits(x))


class Draw:
    """Sequential draws from one seeded stream, stored as float32 (already
    rounded to bfloat16 when ``bf16`` is set)."""

    def __init__(self, seed: int, bf16: bool):
        self.gen = generator(seed)
        self.bf16 = bf16

    def normal(self, shape, std: float = 1.0) -> np.ndarray:
        x = normal_f32(self.gen, shape, std)
        return bf16_round(x) if self.bf16 else x

    def uniform(self, lo: float, hi: float) -> float:
        """One float32 value uniform in [lo, hi) (bf16-rounded when ``bf16``)."""
        x = np.float32(self.gen.uniform(lo, hi))
        return float(bf16_round(np.array([x]))[0]) if self.bf16 else float(x)
