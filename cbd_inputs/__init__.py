"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds random-number generation and workload descriptions only;
it does no convolution arithmetic, so both the CPU oracle and the HIP path
can take their operands from it without sharing any of the method.

Generators (published definitions, implemented here from those definitions):
  * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): state advances by the golden-ratio increment,
    each output is the state passed through the two xor-shift-multiply
    finalisation rounds.
  * Uniform doubles take the top 53 bits of each 64-bit output.
  * Normal deviates use the Box-Muller transform (Box and Muller 1958),
    cosine branch only, with sigma the standard deviation.

Tensors are filled in the memory order of the declared layout; values are
then rounded to the problem dtype (fp32 by IEEE round-to-nearest-even, bf16
by torch's float32 -> bfloat16 conversion), so every consumer receives the
same host bits.
"""
from __future__ import annotations

import numpy as np

from .problems import GROUPED_SWEEP, PROBLEMS, Problem, problem_by_name, seed_for  # noqa: F401

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, count: int) -> np.ndarray:
    """`count` consecutive SplitMix64 outputs for the given 64-bit seed."""
    i = np.arange(1, count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _unit(seed: int, count: int) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (splitmix64(seed, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform(seed: int, shape) -> np.ndarray:
    """U[-1, 1) doubles of the given shape (row-major fill)."""
    n = int(np.prod(shape))
    return (2.0 * _unit(seed, n) - 1.0).reshape(shape)


def normal(seed: int, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) doubles by Box-Muller from 2*count uniforms."""
    n = int(np.prod(shape))
    u = _unit(seed, 2 * n)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    return (sigma * r * np.cos(2.0 * np.pi * u2)).reshape(shape)


def small_ints(seed: int, shape, lo: int = -2, hi: int = 2) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi], as doubles."""
    n = int(np.prod(shape))
    span = hi - lo + 1
    v = (splitmix64(seed, n) >> np.uint64(11)) % np.uint64(span)
    return (v.astype(np.int64) + lo).astype(np.float64).reshape(shape)


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round doubles to the operand dtype; returns float32 values that are
    exactly representable in `dtype` ('f32' or 'bf16')."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(a32).to(torch.bfloat16).to(torch.float32)
        return t.numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(dist: str, seed: int, shape, dtype: str) -> np.ndarray:
    """One operand: dist is 'u' (U[-1,1)), 'n<sigma>' (normal), or 'int'
    (small integers in [-2, 2], for exact-arithmetic runs)."""
    if dist == "u":
        a = uniform(seed, shape)
    elif dist == "int":
        a = small_ints(seed, shape)
    elif dist.startswith("n"):
        a = normal(seed, shape, float(dist[1:]))
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return to_dtype(a, dtype)
