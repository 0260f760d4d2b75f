"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds none of the reduce or gather arithmetic.  It only draws numbers and hands back raw
bit patterns (numpy unsigned views), so that the CPU oracle and the HIP path see identical input bits.

Value recipes follow the workloads the all-reduce and all-gather pages describe: floating-point rank
buffers drawn uniform on [-1, 1) or standard normal in fp32 and narrowed to bf16/fp16 by torch's CPU
conversion (round to nearest even); gather inputs are uniformly random bit patterns, so NaN and inf
encodings occur; FSDP-style parameter splits are log-uniform element counts rounded to multiples of 8.
Every rank buffer r of a workload with seed c is drawn from numpy ``SeedSequence([c, r])`` over PCG64.
"""
from __future__ import annotations

import math

import numpy as np

DTYPES = ("bf16", "fp16", "fp32", "int32")

BITS_DTYPE = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32, "int32": np.uint32}
ELEM_SIZE = {"bf16": 2, "fp16": 2, "fp32": 4, "int32": 4}


def rng_for(seed: int, r: int) -> np.random.Generator:
    """PCG64 stream for rank buffer ``r`` of the workload seeded ``seed``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, r])))


def _to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Narrow an fp32 draw to ``dtype`` with torch's CPU conversion and return the raw bits."""
    if dtype == "fp32":
        return x32.view(np.uint32).copy()
    import torch

    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(tdt)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rank_buffer(seed: int, r: int, n: int, dtype: str, dist: str = "uniform") -> np.ndarray:
    """One rank buffer of ``n`` elements as raw bits.

    ``dist`` is ``"uniform"`` (uniform on [-1, 1)) or ``"normal"`` (N(0, 1)), drawn in fp32.
    """
    if dtype not in ("bf16", "fp16", "fp32"):
        raise ValueError(f"floating rank buffers only, got {dtype}")
    g = rng_for(seed, r)
    if dist == "uniform":
        x = g.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    elif dist == "normal":
        x = g.standard_normal(n, dtype=np.float32)
    else:
        raise ValueError(dist)
    return _to_bits(x.astype(np.float32, copy=False), dtype)


def rank_buffers(seed: int, W: int, n: int, dtype: str, dist: str = "uniform") -> list[np.ndarray]:
    """``W`` independent rank buffers (one seed per rank)."""
    return [rank_buffer(seed, r, n, dtype, dist) for r in range(W)]


def random_bits(seed: int, r: int, n: int, dtype: str) -> np.ndarray:
    """Uniformly random bit patterns of the element width of ``dtype`` (NaN/inf encodings included)."""
    g = rng_for(seed, r)
    bd = BITS_DTYPE[dtype]
    info = np.iinfo(bd)
    return g.integers(0, int(info.max) + 1, size=n, dtype=bd)


def log_uniform_splits(seed: int, P: int, lo: int = 1024, hi: int = 4_194_304, mult: int = 8) -> np.ndarray:
    """``P`` element counts, log-uniform in [lo, hi], rounded to multiples of ``mult`` and clamped."""
    g = rng_for(seed, 1_000_003)
    u = g.uniform(math.log(lo), math.log(hi), size=P)
    e = np.rint(np.exp(u) / mult).astype(np.int64) * mult
    return np.clip(e, lo, hi).astype(np.uint64)


def gather_source(seed: int, W: int, T: int, dtype: str) -> np.ndarray:
    """Rank-major gathered buffer ``[W][T]`` of random bits, flattened (one seed per rank row)."""
    bd = BITS_DTYPE[dtype]
    out = np.empty(W * T, dtype=bd)
    for r in range(W):
        out[r * T:(r + 1) * T] = random_bits(seed, r, T, dtype)
    return out


# The named workloads: shapes and seeds (values come from the functions above).
W4_BF16_64KI = dict(seed=1, W=4, n=65_536, dtype="bf16", dist="uniform")
W8_BF16_16MIB = dict(seed=2, W=8, n=8_388_608, dtype="bf16", dist="normal")
SWEEP_BYTES_PER_RANK = [256 << 10, 1 << 20, 4 << 20, 16 << 20, 64 << 20, 256 << 20]
FSDP_SPLITS_W8_G4_P64 = dict(seed=4, W=8, G=4, P=64)
W8_FP32_512MIB = dict(seed=5, W=8, n=134_217_728, dtype="fp32", dist="uniform")
