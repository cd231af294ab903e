"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests
and the bench.  Holds none of the method's arithmetic: only random draws,
the input value distribution, and bit-level dtype conversion.

Recipe (same for every consumer, so both sides see identical bits):
  * ``numpy.random.Generator(PCG64(SeedSequence([42, cfg, t])))`` with t an
    integer tag per tensor (0 = Q, 1 = K, 2 = V, larger tags for extras);
  * ``standard_normal`` in float64 of the GLOBAL tensor shape;
  * optional per-(token, head) RMS normalisation over D: x / sqrt(mean(x^2)
    + 1e-6), weight 1 (the QK-norm that DiT attention layers apply);
  * cast to float32, then to bfloat16 with round-to-nearest-even when the
    workload is bf16.
Shards and KV chunks are slices of the global tensor.
"""

from __future__ import annotations

import numpy as np

SEED = 42


def rng(cfg: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, int(cfg), int(tag)])))


def normal(cfg: int, tag: int, shape, rms_norm: bool = False) -> np.ndarray:
    """float64 N(0,1) draws, optionally RMS-normalised over the last axis."""
    x = rng(cfg, tag).standard_normal(size=tuple(shape), dtype=np.float64)
    if rms_norm:
        x = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    NaN inputs keep a quiet NaN pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tensor(cfg: int, tag: int, shape, dtype: str, rms_norm: bool = False):
    """Return (bits, values_f64): the storage array the device gets
    (uint16 bf16 bits or float32) and the exact same values widened to
    float64 for the oracle."""
    x = normal(cfg, tag, shape, rms_norm).astype(np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "fp32":
        return x, x.astype(np.float64)
    raise ValueError("dtype must be 'bf16' or 'fp32'")


# Workload shapes (global tensors; see the design doc for the recipe per config).
CONFIGS = {
    1: dict(name="tiny ragged fp32 share", dtype="fp32", B=1, S=257, H=2, D=64,
            shards=[129, 128], rms=False),
    2: dict(name="FLUX.1-dev 1024x1024 Ulysses share", dtype="bf16", B=1, S=4608, H=24, D=128,
            shards=[2304, 2304], rms=True),
    3: dict(name="FLUX.1-dev 1008x1008 UAA share", dtype="bf16", B=1, S=4481, H=24, D=128,
            shards=[2241, 2240], rms=True),
    4: dict(name="Qwen-Image 1328x1328 Ring share", dtype="bf16", B=1, S=6986, H=24, D=128,
            shards=[3493, 3493], rms=True),
    5: dict(name="long-context causal zigzag share", dtype="bf16", B=1, S=32768, H=32, D=128,
            chunks=8, q_chunks=[1, 6], rms=False),
}
