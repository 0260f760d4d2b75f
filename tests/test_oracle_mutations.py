"""The oracle's pins catch plausible mistakes.

Each case below is a copy of an oracle function with one planted mistake (a wrong accumulator start, a
reversed rank order, a dropped rank, a wider accumulator, a wrong rounding, a flushed subnormal, a wrong
offset in the gather placement).  It is patched in, on the CPU, for the pins named beside it, and at
least one of those pins must fail.  The pins themselves are the functions of tests/test_oracle.py; a
pin that would pass with a mistake in the oracle would not be pinning it."""
import numpy as np
import pytest

import oracle
import test_oracle as pins

# --------------------------------------------------------------------------------- reduce: mutants


def _widen(b, dtype):
    return oracle.widen(b, dtype)


def _sum(bufs, dtype, order=None, start=None, acc_dtype=np.float32, drop_last=False, ftz=False):
    order = list(range(len(bufs))) if order is None else order
    if drop_last:
        order = order[:-1]
    with np.errstate(over="ignore", invalid="ignore"):
        if start is None:
            acc = _widen(bufs[order[0]], dtype).astype(acc_dtype)
            rest = order[1:]
        else:
            acc = np.full(bufs[0].shape, start, dtype=acc_dtype)
            rest = order
        for r in rest:
            t = _widen(bufs[r], dtype).astype(acc_dtype)
            if ftz:
                t = np.where(np.abs(t) < np.float32(2.0 ** -126), acc_dtype(0), t)
            acc = np.add(acc, t, dtype=acc_dtype)
            if ftz:
                acc = np.where(np.abs(acc) < np.float32(2.0 ** -126), acc_dtype(0), acc).astype(acc_dtype)
    return acc.astype(np.float32)


def _narrow_truncate_bf16(x):
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _narrow_ties_up_bf16(x):
    u = x.view(np.uint32)
    hi, lo = u >> np.uint32(16), u & np.uint32(0xFFFF)
    r = hi + (lo >= 0x8000).astype(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    return np.where(nan, hi | np.uint32(0x40), r).astype(np.uint16)


def _narrow_nan_not_quieted(x, dtype):
    if dtype != "bf16":
        return oracle.narrow(x, dtype)
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    hi, lo = u >> np.uint32(16), u & np.uint32(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint32(1)) == 1))
    return (hi + up.astype(np.uint32)).astype(np.uint16)  # a NaN whose payload sits in the low half becomes inf


def _reduce_with(narrow_bf16=None, **kw):
    def f(bufs, dtype):
        if dtype not in ("bf16", "fp16", "fp32"):
            raise ValueError(dtype)
        acc = _sum(bufs, dtype, **kw)
        if dtype == "bf16" and narrow_bf16 is not None:
            return narrow_bf16(acc)
        return oracle.narrow(acc, dtype)
    return f


def _reversed(bufs, dtype):
    return oracle.narrow(_sum(bufs, dtype, order=list(range(len(bufs)))[::-1]), dtype)


# pins, called directly with their parameters
def _golden():
    for case in pins._golden_cases():
        pins.test_reduce_golden_closed_forms(case)


def _brute():
    for dtype in ("bf16", "fp16", "fp32"):
        for W in (2, 3, 8):
            pins.test_reduce_brute_force(dtype, W)


def _torch_loop():
    for dtype in ("bf16", "fp16", "fp32"):
        for W in (2, 3, 8):
            pins.test_reduce_matches_torch_cpu_loop(dtype, W)


def _equal_buffers():
    pins.test_reduce_equal_buffers_give_W_times_x("bf16", 8)


REDUCE_MUTANTS = {
    "accumulator starts at +0": (_reduce_with(start=0.0), [_golden]),
    "ranks summed in reverse order": (_reversed, [_golden, _brute]),
    "last rank dropped": (_reduce_with(drop_last=True), [_torch_loop, _equal_buffers]),
    "fp64 accumulation": (_reduce_with(acc_dtype=np.float64), [_brute]),
    "bf16 narrowing truncates": (_reduce_with(narrow_bf16=_narrow_truncate_bf16), [_golden, _torch_loop]),
    "bf16 ties round up": (_reduce_with(narrow_bf16=_narrow_ties_up_bf16), [_golden]),
    "subnormals flushed to zero": (_reduce_with(ftz=True), [_golden]),
}


@pytest.mark.parametrize("name", list(REDUCE_MUTANTS))
def test_reduce_pins_catch_planted_mistake(name, monkeypatch):
    mutant, catchers = REDUCE_MUTANTS[name]
    monkeypatch.setattr(oracle, "allreduce_sum_ref", mutant)
    caught = []
    for pin in catchers:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"


def test_narrowing_pin_catches_an_unquieted_nan(monkeypatch):
    monkeypatch.setattr(oracle, "narrow", _narrow_nan_not_quieted)
    with pytest.raises(AssertionError):
        pins.test_bf16_narrow_structured_sweep()


def test_unmutated_oracle_passes_the_same_pins():
    for pin in (_golden, _brute, _torch_loop, _equal_buffers):
        pin()
    pins.test_bf16_narrow_structured_sweep()


# --------------------------------------------------------------------------------- gather: mutants


def _gather_with(offsets="exclusive", block="m*G*E", src_stride="T", times_W=True, reverse_slots=False):
    def f(src, W, G, splits):
        if W < 1 or G < 1 or W % G != 0:
            raise ValueError("G")
        e = [int(v) for v in splits]
        T = sum(e)
        if src.shape != (W * T,):
            raise ValueError("size")
        out = np.zeros_like(src)
        O = 0
        for s, E in enumerate(e):
            Os = O + E if offsets == "inclusive" else O
            for m in range(W // G):
                base = (Os * W if times_W else Os) + (m * G * E if block == "m*G*E" else m * E)
                for g in range(G):
                    r = m * G + g
                    slot = G - 1 - g if reverse_slots else g
                    stride = T if src_stride == "T" else Os
                    dst = base + slot * E
                    piece = src[r * stride + Os:r * stride + Os + E]
                    k = max(0, min(len(piece), len(out) - dst))  # clipped: a wrong result, not a crash
                    out[dst:dst + k] = piece[:k]
            O += E
        return out
    return f


def _transpose():
    for args in ((8, 4, 5, 24), (4, 4, 3, 7), (2, 1, 6, 1)):
        pins.test_gather_equal_splits_is_transpose(*args)


def _inverse_map():
    pins.test_gather_inverse_map_from_output_side()


def _g_independent():
    pins.test_gather_independent_of_G()


GATHER_MUTANTS = {
    "inclusive O_s": (_gather_with(offsets="inclusive"), [_transpose, _inverse_map]),
    "node-block offset m*E_s": (_gather_with(block="m*E"), [_transpose, _g_independent]),
    "source row stride O_s instead of T": (_gather_with(src_stride="O"), [_transpose, _inverse_map]),
    "O_s not multiplied by W": (_gather_with(times_W=False), [_transpose, _inverse_map]),
    "slots in reverse order": (_gather_with(reverse_slots=True), [_inverse_map]),
}


@pytest.mark.parametrize("name", list(GATHER_MUTANTS))
def test_gather_pins_catch_planted_mistake(name, monkeypatch):
    mutant, catchers = GATHER_MUTANTS[name]
    monkeypatch.setattr(oracle, "allgather_param_contig_ref", mutant)
    caught = []
    for pin in catchers:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"


def test_unmutated_gather_passes_the_same_pins():
    for pin in (_transpose, _inverse_map, _g_independent):
        pin()
