"""Exact-rational IEEE-754 binary arithmetic, written from the standard, for pinning the oracle.

Values are decoded from raw bits into exact rationals (``fractions.Fraction``); a sum is formed exactly
and rounded once to a target format by round-to-nearest-even with gradual underflow and overflow to
infinity.  Nothing here uses hardware floating point, so it is independent of numpy's float32 ops and
of any conversion routine.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction


@dataclass(frozen=True)
class Fmt:
    name: str
    ebits: int
    mbits: int  # stored fraction bits

    @property
    def bias(self) -> int:
        return (1 << (self.ebits - 1)) - 1

    @property
    def emin(self) -> int:
        return 1 - self.bias

    @property
    def emax(self) -> int:
        return self.bias

    @property
    def p(self) -> int:
        return self.mbits + 1

    @property
    def width(self) -> int:
        return 1 + self.ebits + self.mbits


BF16 = Fmt("bf16", 8, 7)
FP16 = Fmt("fp16", 5, 10)
FP32 = Fmt("fp32", 8, 23)
FMTS = {"bf16": BF16, "fp16": FP16, "fp32": FP32}


@dataclass(frozen=True)
class Val:
    kind: str          # "num", "inf", "nan"
    neg: bool = False
    mag: Fraction = Fraction(0)  # magnitude for "num" (0 for a signed zero)


def decode(bits: int, f: Fmt) -> Val:
    neg = bool(bits >> (f.width - 1) & 1)
    e = bits >> f.mbits & ((1 << f.ebits) - 1)
    m = bits & ((1 << f.mbits) - 1)
    if e == (1 << f.ebits) - 1:
        return Val("nan") if m else Val("inf", neg)
    if e == 0:
        mag = Fraction(m, 1 << f.mbits) * Fraction(2) ** f.emin
    else:
        mag = Fraction((1 << f.mbits) + m, 1 << f.mbits) * Fraction(2) ** (e - f.bias)
    return Val("num", neg, mag)


def _floor_log2(q: Fraction) -> int:
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_mag(q: Fraction, f: Fmt) -> Val:
    """Round a positive magnitude to ``f`` (RNE); returns "num" or "inf" (positive)."""
    assert q > 0
    e = max(_floor_log2(q), f.emin)
    quantum = Fraction(2) ** (e - f.p + 1)
    m = q / quantum
    k = m.numerator // m.denominator
    rem = m - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    r = k * quantum
    maxfinite = (2 - Fraction(2) ** (1 - f.p)) * Fraction(2) ** f.emax
    if r > maxfinite:
        return Val("inf")
    return Val("num", False, r)


def round_signed(neg: bool, q: Fraction, f: Fmt) -> Val:
    """Round a nonzero exact value (sign, magnitude) to ``f``; underflow to zero keeps the sign."""
    v = round_mag(q, f)
    return Val(v.kind, neg, v.mag)


def convert(v: Val, f: Fmt) -> Val:
    """Round a value (from any format) to ``f``."""
    if v.kind != "num" or v.mag == 0:
        return v
    return round_signed(v.neg, v.mag, f)


def add(a: Val, b: Val, f: Fmt) -> Val:
    """IEEE addition a + b rounded to ``f`` (RNE)."""
    if a.kind == "nan" or b.kind == "nan":
        return Val("nan")
    if a.kind == "inf" and b.kind == "inf":
        return a if a.neg == b.neg else Val("nan")
    if a.kind == "inf":
        return a
    if b.kind == "inf":
        return b
    sa = -a.mag if a.neg else a.mag
    sb = -b.mag if b.neg else b.mag
    s = sa + sb
    if s == 0:
        # Exact zero sum: -0 only when both addends are -0 (round-to-nearest).
        both_neg_zero = a.mag == 0 and b.mag == 0 and a.neg and b.neg
        return Val("num", both_neg_zero, Fraction(0))
    return round_signed(s < 0, abs(s), f)


def encode(v: Val, f: Fmt) -> int | None:
    """Bits of a value that is exactly representable in ``f`` (None for NaN)."""
    sign = (1 << (f.width - 1)) if v.neg else 0
    if v.kind == "nan":
        return None
    if v.kind == "inf":
        return sign | (((1 << f.ebits) - 1) << f.mbits)
    if v.mag == 0:
        return sign
    fl = _floor_log2(v.mag)
    if fl < f.emin:  # subnormal: biased exponent field 0
        m = v.mag / Fraction(2) ** f.emin * (1 << f.mbits)
        assert m.denominator == 1, "value not representable"
        return sign | int(m)
    m = v.mag / Fraction(2) ** fl * (1 << f.mbits)
    assert m.denominator == 1, "value not representable"
    return sign | ((fl + f.bias) << f.mbits) | (int(m) - (1 << f.mbits))


def same(a: Val, b: Val) -> bool:
    """Bitwise-equal values, treating every NaN as equal to every NaN."""
    if a.kind == "nan" or b.kind == "nan":
        return a.kind == b.kind
    return a == b


def reduce_exact(cols: list[list[int]], src: str, dst: str) -> list[Val]:
    """Brute-force W-way sum: fp32 accumulation in rank order, each add rounded once, then narrowing.

    ``cols[i]`` holds the W raw bit patterns of element i (rank order).
    """
    fs, f32, fd = FMTS[src], FP32, FMTS[dst]
    out = []
    for col in cols:
        acc = convert(decode(col[0], fs), f32)
        for b in col[1:]:
            acc = add(acc, convert(decode(b, fs), f32), f32)
        out.append(convert(acc, fd))
    return out
