"""Widening to fp32 and round-to-nearest-even narrowing, on raw bit views.  Test infrastructure only.

The pages never state how a bf16/fp16 rank value enters the fp32 sum or how the sum leaves it.  Reading
taken here: widening is exact (every bf16 and fp16 value is an fp32 value), narrowing is IEEE-754
round-to-nearest-even with subnormals kept and overflow to infinity; a NaN stays a NaN.
"""
from __future__ import annotations

import numpy as np

_BITS = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32}


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw bits of ``dtype`` -> float32 values (exact)."""
    if dtype == "bf16":
        # A bf16 is the upper half of an fp32 with the lower 16 fraction bits zero.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "fp32":
        return bits.view(np.float32).copy()
    raise ValueError(f"no floating widening for {dtype}")


def _narrow_bf16(x: np.ndarray) -> np.ndarray:
    u = x.view(np.uint32)
    hi = u >> np.uint32(16)
    lo = u & np.uint32(0xFFFF)
    # Round to nearest on the 16 dropped bits; on an exact half, round to the even upper half.
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint32(1)) == 1))
    r = hi + up.astype(np.uint32)  # a carry out of the fraction steps the exponent (to inf at the top)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, hi | np.uint32(0x0040), r)  # NaN: keep sign and payload top, set the quiet bit
    return r.astype(np.uint16)


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> raw bits of ``dtype`` by round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return _narrow_bf16(x)
    if dtype == "fp16":
        with np.errstate(over="ignore"):  # overflow to +-inf is the defined result
            return x.astype(np.float16).view(np.uint16)
    if dtype == "fp32":
        return x.view(np.uint32).copy()
    raise ValueError(f"no floating narrowing for {dtype}")
