"""Pins for the CPU oracle: it is checked against things other than itself.

* exact-rational IEEE arithmetic written from the standard (tests/ieee_exact.py) on brute-force inputs;
* hand-derived closed forms (tests/golden/ieee_reduce_cases.txt);
* an independent nearest-neighbour formulation of bf16 rounding and torch's CPU conversions;
* invariants of the gather (permutation, inverse map, transpose for equal splits, node-block size G).
"""
import os

import numpy as np
import pytest
import torch

import ieee_exact as ie
import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ieee_reduce_cases.txt")
BITS = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32}
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _bits_to_val(bits, dtype):
    return ie.decode(int(bits), ie.FMTS[dtype])


# ----------------------------------------------------------------------------------------------- numerics

def _bf16_nearest(u: np.ndarray) -> np.ndarray:
    """bf16 rounding by comparing distances to the two neighbouring bf16 values (float64, exact)."""
    u = u.astype(np.uint32)
    x = u.view(np.float32).astype(np.float64)
    sign = u & np.uint32(0x80000000)
    mag = u & np.uint32(0x7FFFFFFF)
    lo_bits = mag & np.uint32(0xFFFF0000)                  # toward zero
    lo = lo_bits.view(np.float32).astype(np.float64)
    hi_bits = lo_bits + np.uint32(0x10000)                 # next bf16 magnitude (may be inf)
    with np.errstate(over="ignore"):
        hi = hi_bits.view(np.float32).astype(np.float64)
    hi = np.where(hi_bits == 0x7F800000, 2.0 ** 128, hi)   # unbounded-exponent neighbour above max
    ax = np.abs(x)
    dlo, dhi = ax - lo, hi - ax
    even_lo = ((lo_bits >> 16) & 1) == 0
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ~even_lo)
    res = np.where(pick_hi, hi_bits, lo_bits) >> 16
    res = res | (sign >> 16)
    return res.astype(np.uint16)


def _is_nan32(u):
    return (u.astype(np.uint32) & 0x7FFFFFFF) > 0x7F800000


def _is_nan16(b, dtype):
    b = b.astype(np.uint32)
    if dtype == "bf16":
        return (b & 0x7FFF) > 0x7F80
    return (b & 0x7FFF) > 0x7C00


def test_bf16_narrow_structured_sweep():
    # Every one of the 65536 upper halves with the lower halves that decide rounding: 0, just below,
    # at and just above the half, the quarter points and the extremes.
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFE, 0xFFFF], np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    got = oracle.narrow(u.view(np.float32), "bf16")
    nan = _is_nan32(u)
    ref = _bf16_nearest(u)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(_is_nan16(got[nan], "bf16"))
    # torch's own bf16 conversion on the same values (finite inputs and infinities)
    tt = torch.from_numpy(u[~nan].view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[~nan], tt)


def test_bf16_narrow_random_and_exact():
    g = np.random.default_rng(7)
    u = g.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    got = oracle.narrow(u.view(np.float32), "bf16")
    nan = _is_nan32(u)
    assert np.array_equal(got[~nan], _bf16_nearest(u)[~nan])
    assert np.all(_is_nan16(got[nan], "bf16"))
    # exact-rational rounding on a sample
    for v in u[:3000]:
        want = ie.convert(ie.decode(int(v), ie.FP32), ie.BF16)
        g16 = oracle.narrow(np.array([v], np.uint32).view(np.float32), "bf16")[0]
        assert ie.same(ie.decode(int(g16), ie.BF16), want), hex(int(v))


def test_fp16_narrow_against_torch_and_exact():
    g = np.random.default_rng(11)
    # fp32 exponents around the fp16 range (subnormal, normal, overflow) with structured fractions
    exps = np.arange(127 - 30, 127 + 18, dtype=np.uint32)
    fr = np.concatenate([
        np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x7FFFFF], np.uint32),
        g.integers(0, 1 << 23, size=200, dtype=np.uint32),
    ])
    u = ((exps[:, None] << 23) | fr[None, :]).ravel()
    u = np.concatenate([u, u | np.uint32(0x80000000), g.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    got = oracle.narrow(u.view(np.float32), "fp16")
    nan = _is_nan32(u)
    tt = torch.from_numpy(u.view(np.float32)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[~nan], tt[~nan])
    assert np.all(_is_nan16(got[nan], "fp16"))
    for v in u[::97][:2500]:
        want = ie.convert(ie.decode(int(v), ie.FP32), ie.FP16)
        g16 = oracle.narrow(np.array([v], np.uint32).view(np.float32), "fp16")[0]
        assert ie.same(ie.decode(int(g16), ie.FP16), want), hex(int(v))


def _every_fp32_pattern(check, chunk_bits=23):
    """Run check(u) over all 2^32 fp32 bit patterns in chunks, on the host's cores (numpy releases the
    GIL inside its loops).  Returns the number of chunks checked."""
    from concurrent.futures import ThreadPoolExecutor
    step = 1 << chunk_bits

    def one(k):
        u = np.arange(k * step, (k + 1) * step, dtype=np.uint64).astype(np.uint32)
        check(u)
        return 1

    threads = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as ex:
        return sum(ex.map(one, range(1 << (32 - chunk_bits))))


@pytest.mark.slow
def test_bf16_narrow_every_fp32_pattern():
    """All 2^32 fp32 patterns: the oracle's integer rounding against the nearest-neighbour formulation
    (and torch's conversion on the non-NaN ones); NaNs stay NaN."""
    def check(u):
        got = oracle.narrow(u.view(np.float32), "bf16")
        nan = _is_nan32(u)
        ok = ~nan
        assert np.array_equal(got[ok], _bf16_nearest(u[ok])), hex(int(u[0]))
        tt = torch.from_numpy(u[ok].view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[ok], tt), hex(int(u[0]))
        assert np.all(_is_nan16(got[nan], "bf16")), hex(int(u[0]))

    assert _every_fp32_pattern(check) == 512


@pytest.mark.slow
def test_fp16_narrow_every_fp32_pattern():
    """All 2^32 fp32 patterns: the oracle's fp16 narrowing against torch's CPU conversion; NaNs stay NaN."""
    def check(u):
        got = oracle.narrow(u.view(np.float32), "fp16")
        nan = _is_nan32(u)
        tt = torch.from_numpy(u.view(np.float32)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[~nan], tt[~nan]), hex(int(u[0]))
        assert np.all(_is_nan16(got[nan], "fp16")), hex(int(u[0]))

    assert _every_fp32_pattern(check) == 512


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_widen_is_exact_for_every_pattern(dtype):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = oracle.widen(b, dtype).view(np.uint32)
    for i in range(0, 65536, 37):
        a = ie.decode(int(b[i]), ie.FMTS[dtype])
        c = ie.decode(int(w[i]), ie.FP32)
        assert ie.same(a, c), (dtype, hex(i))
    # and narrowing a widened value gives the value back (all non-NaN patterns)
    nn = ~_is_nan16(b, dtype)
    assert np.array_equal(oracle.narrow(oracle.widen(b, dtype), dtype)[nn], b[nn])


def test_fp32_add_is_ieee_rne():
    """The oracle's accumulation relies on numpy float32 addition; pin it to exact IEEE arithmetic."""
    g = np.random.default_rng(3)
    n = 4000
    # mixes of magnitudes: subnormals, close exponents (ties), far exponents, cancellations
    a = g.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    b = g.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    b[: n // 4] = a[: n // 4] ^ np.uint32(0x80000000)                       # exact cancellation
    b[n // 4: n // 2] = (a[n // 4: n // 2] & 0xFF800000) - np.uint32(24 << 23) & 0xFFFFFFFF  # ties
    a[n // 2: 3 * n // 4] &= np.uint32(0x807FFFFF)                          # subnormals
    b[n // 2: 3 * n // 4] &= np.uint32(0x807FFFFF)
    s = (a.view(np.float32) + b.view(np.float32)).view(np.uint32)
    for i in range(n):
        want = ie.add(ie.decode(int(a[i]), ie.FP32), ie.decode(int(b[i]), ie.FP32), ie.FP32)
        assert ie.same(ie.decode(int(s[i]), ie.FP32), want), (hex(int(a[i])), hex(int(b[i])))


# -------------------------------------------------------------------------------------------------- reduce

def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if not line or line.startswith("#"):
                continue
            dtype, W, ins, exp = line.split()
            cases.append((dtype, int(W), [int(x, 16) for x in ins.split(",")], exp))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: f"{c[0]}-{'-'.join(hex(x) for x in c[2])}")
def test_reduce_golden_closed_forms(case):
    dtype, W, ins, exp = case
    assert len(ins) == W
    bufs = [np.array([v], dtype=BITS[dtype]) for v in ins]
    out = oracle.allreduce_sum_ref(bufs, dtype)[0]
    if exp == "nan":
        assert _is_nan16(np.array([out]), dtype)[0] if dtype != "fp32" else _is_nan32(np.array([out]))[0]
    else:
        assert int(out) == int(exp, 16), (hex(int(out)), exp)
    # the brute-force IEEE model agrees with the hand derivation too
    want = ie.reduce_exact([ins], dtype, dtype)[0]
    got = ie.decode(int(out), ie.FMTS[dtype])
    assert ie.same(got, want)


def _special_patterns(dtype):
    f = ie.FMTS[dtype]
    sign = 1 << (f.width - 1)
    inf = ((1 << f.ebits) - 1) << f.mbits
    one = f.bias << f.mbits
    pats = [0, sign, 1, sign | 1, inf, sign | inf, inf | 1, one, sign | one, inf - 1, sign | (inf - 1),
            (1 << f.mbits) - 1, 1 << f.mbits, one | 1]
    return pats


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 16])
def test_reduce_brute_force(dtype, W):
    g = np.random.default_rng(100 + W)
    n = 48
    bd = BITS[dtype]
    width = ie.FMTS[dtype].width
    # random bit patterns restricted to moderate exponents, so sums are interesting, plus specials
    bufs = []
    for r in range(W):
        if dtype == "fp32":
            x = g.standard_normal(n).astype(np.float32) * np.float32(2.0 ** g.integers(-8, 8))
            b = x.view(np.uint32).copy()
        else:
            x = torch.from_numpy(g.standard_normal(n).astype(np.float32)).to(TORCH[dtype])
            b = x.view(torch.int16).numpy().view(np.uint16).copy()
        sp = _special_patterns(dtype)
        k = min(len(sp), n // 3)
        b[:k] = np.array(g.permutation(sp)[:k], dtype=bd)
        bufs.append(b.astype(bd))
    out = oracle.allreduce_sum_ref(bufs, dtype)
    cols = [[int(bufs[r][i]) for r in range(W)] for i in range(n)]
    want = ie.reduce_exact(cols, dtype, dtype)
    for i in range(n):
        assert ie.same(ie.decode(int(out[i]), ie.FMTS[dtype]), want[i]), (dtype, W, i, [hex(c) for c in cols[i]])
    assert out.dtype == bd and width in (16, 32)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("W", [2, 3, 5, 7, 8, 16])
def test_reduce_equal_buffers_give_W_times_x(dtype, W):
    # For bf16/fp16 inputs every partial sum k*x needs at most 11 + 4 significant bits, so it is exact
    # in fp32 and the result is the single rounding of W*x.
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[~_is_nan16(b, dtype)]
    out = oracle.allreduce_sum_ref([b] * W, dtype)
    for i in range(0, len(b), 211):
        v = ie.decode(int(b[i]), ie.FMTS[dtype])
        if v.kind == "inf":
            want = v
        elif v.mag == 0:
            want = v
        else:
            want = ie.round_signed(v.neg, v.mag * W, ie.FMTS[dtype])
        assert ie.same(ie.decode(int(out[i]), ie.FMTS[dtype]), want), hex(int(b[i]))


def test_reduce_equal_buffers_fp32_short_significands():
    # fp32 values with at most 20 significant bits: W*x for W <= 16 is exact in every partial sum.
    g = np.random.default_rng(5)
    x = (g.standard_normal(5000).astype(np.float32).view(np.uint32) & np.uint32(0xFFFFFFF0))
    for W in (3, 8, 13, 16):
        out = oracle.allreduce_sum_ref([x] * W, "fp32")
        want = (x.view(np.float32).astype(np.float64) * W).astype(np.float32).view(np.uint32)
        assert np.array_equal(out, want)


def test_reduce_exact_sum_construction():
    # Values k/256 with |k| < 128 are exact in bf16; sums of up to 16 of them are exact in fp32, so the
    # result is the single RNE rounding of the exact integer sum, whatever the order.
    g = np.random.default_rng(9)
    W, n = 16, 3000
    ks = g.integers(-127, 128, size=(W, n))
    bufs = [torch.from_numpy((ks[r] / 256.0).astype(np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16).copy() for r in range(W)]
    out = oracle.allreduce_sum_ref(bufs, "bf16")
    tot = ks.sum(axis=0)
    from fractions import Fraction
    for i in range(0, n, 7):
        q = Fraction(int(tot[i]), 256)
        want = ie.Val("num", False, Fraction(0)) if q == 0 else ie.round_signed(q < 0, abs(q), ie.BF16)
        assert ie.same(ie.decode(int(out[i]), ie.BF16), want)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_reduce_W1_is_identity(dtype):
    n = 65536 if dtype != "fp32" else 1 << 18
    if dtype == "fp32":
        b = np.random.default_rng(1).integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
        nan = _is_nan32(b)
    else:
        b = np.arange(n, dtype=np.uint32).astype(np.uint16)
        nan = _is_nan16(b, dtype)
    out = oracle.allreduce_sum_ref([b], dtype)
    assert np.array_equal(out[~nan], b[~nan])


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_reduce_matches_torch_cpu_loop(dtype, W):
    g = np.random.default_rng(W)
    n = 4096 + W
    ts = [torch.from_numpy(g.uniform(-1, 1, n).astype(np.float32)).to(TORCH[dtype]) for _ in range(W)]
    acc = ts[0].float()
    for t in ts[1:]:
        acc = acc + t.float()
    ref = acc.to(TORCH[dtype])
    ibits = torch.int16 if dtype != "fp32" else torch.int32
    ub = np.uint16 if dtype != "fp32" else np.uint32
    bufs = [t.view(ibits).numpy().view(ub).copy() for t in ts]
    out = oracle.allreduce_sum_ref(bufs, dtype)
    assert np.array_equal(out, ref.view(ibits).numpy().view(ub))


def _structured_partners16(dtype: str) -> np.ndarray:
    """4096 structured 16-bit partners: every exponent field with mantissas at 0 (powers of two), 1,
    the half-way points and the top, plus random mantissas, in both signs (subnormals, inf and NaN
    included)."""
    g = np.random.default_rng(4096)
    if dtype == "bf16":
        eb, mb = 8, 7
        fixed = [0, 1, 0x3F, 0x40, 0x41, 0x7F]
    else:
        eb, mb = 5, 10
        fixed = [0, 1, 0x1FF, 0x200, 0x201, 0x3FF]
    per_exp = 4096 // (2 << eb)
    mants = []
    for e in range(1 << eb):
        m = fixed + list(g.integers(0, 1 << mb, size=per_exp - len(fixed)))
        mants.append([(e << mb) | int(x) for x in m])
    v = np.array(mants, dtype=np.uint32).ravel()
    return np.concatenate([v, v | 0x8000]).astype(np.uint16)


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_reduce_W2_every_pattern_against_structured_partners(dtype):
    """W=2: each of the 65,536 patterns of x0 against 4,096 structured x1 (268M pairs) equals torch's
    CPU widen, fp32 add and narrow; NaN results compare by NaN-ness."""
    x0 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x1 = _structured_partners16(dtype)
    assert len(x1) == 4096 and len(np.unique(x1)) > 3500
    for k in range(0, 4096, 256):
        a = np.repeat(x0, 256)
        b = np.tile(x1[k:k + 256], 65536)
        got = oracle.allreduce_sum_ref([a, b], dtype)
        ta = torch.from_numpy(a.view(np.int16)).view(TORCH[dtype]).float()
        tb = torch.from_numpy(b.view(np.int16)).view(TORCH[dtype]).float()
        ref = (ta + tb).to(TORCH[dtype]).view(torch.int16).numpy().view(np.uint16)
        rn = _is_nan16(ref, dtype)
        assert np.array_equal(got[~rn], ref[~rn]), (dtype, k)
        assert np.all(_is_nan16(got[rn], dtype)), (dtype, k)


def test_reduce_rejects_int32():
    with pytest.raises(ValueError):
        oracle.allreduce_sum_ref([np.zeros(4, np.uint32)], "int32")


def test_threaded_oracle_equals_single():
    bufs = workloads.rank_buffers(2, 8, 100_003, "bf16", "normal")
    a = oracle.allreduce_sum_ref(bufs, "bf16")
    b = oracle.allreduce_sum_ref_threaded(bufs, "bf16", threads=4)
    assert np.array_equal(a, b)


# -------------------------------------------------------------------------------------------------- gather

def _tagged(W, T):
    return np.arange(W * T, dtype=np.uint32)


@pytest.mark.parametrize("W,G", [(1, 1), (4, 2), (8, 4), (8, 8)])
def test_gather_single_split_is_identity(W, G):
    T = 1000
    src = _tagged(W, T)
    assert np.array_equal(oracle.allgather_param_contig_ref(src, W, G, [T]), src)


@pytest.mark.parametrize("W,G,P,E", [(8, 4, 5, 24), (4, 4, 3, 7), (2, 1, 6, 1)])
def test_gather_equal_splits_is_transpose(W, G, P, E):
    src = np.random.default_rng(0).integers(0, 2 ** 16, size=W * P * E, dtype=np.uint16)
    out = oracle.allgather_param_contig_ref(src, W, G, [E] * P)
    want = np.transpose(src.reshape(W, P, E), (1, 0, 2)).ravel()
    assert np.array_equal(out, want)
    tw = torch.from_numpy(src.astype(np.int32)).view(W, P, E).permute(1, 0, 2).contiguous().view(-1).numpy()
    assert np.array_equal(out.astype(np.int32), tw)


def test_gather_inverse_map_from_output_side():
    """Tagged input: decode each output position back to (param, rank, element) independently."""
    W, G = 8, 4
    splits = [16, 0, 8, 40, 8, 24]
    T = sum(splits)
    src = _tagged(W, T)
    out = oracle.allgather_param_contig_ref(src, W, G, splits)
    pos = 0
    base = 0
    for E in splits:
        for r in range(W):
            for j in range(E):
                assert out[pos] == r * T + base + j, (pos, r, j)
                pos += 1
        base += E
    assert pos == W * T


def test_gather_is_a_bit_permutation_of_random_bits():
    W, G = 8, 4
    splits = workloads.log_uniform_splits(4, 12, lo=8, hi=4096)
    T = int(splits.sum())
    for dtype in ("bf16", "fp32"):
        src = workloads.gather_source(40, W, T, dtype)
        out = oracle.allgather_param_contig_ref(src, W, G, splits)
        assert np.array_equal(np.sort(out), np.sort(src))
        # and every NaN payload survives untouched (integer views only)
        assert out.tobytes() != src.tobytes() or len(splits) == 1


def test_gather_independent_of_G():
    W = 8
    splits = [8, 64, 1024, 0, 120, 8]
    T = sum(splits)
    src = workloads.gather_source(41, W, T, "fp16")
    outs = [oracle.allgather_param_contig_ref(src, W, G, splits) for G in (1, 2, 4, 8)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_gather_matches_torch_split_and_cat_copy_out():
    # FSDP's copy-out after a rank-major all-gather: split each rank's shard by the parameter sizes and
    # concatenate, per parameter, the W rank pieces.
    W, G = 8, 2
    splits = [int(v) for v in workloads.log_uniform_splits(5, 9, lo=8, hi=2048)]
    T = sum(splits)
    src = workloads.gather_source(42, W, T, "int32")
    t = torch.from_numpy(src.view(np.int32)).view(W, T)
    pieces = [t[r].split(splits) for r in range(W)]
    want = torch.cat([torch.cat([pieces[r][s] for r in range(W)]) for s in range(len(splits))])
    out = oracle.allgather_param_contig_ref(src, W, G, splits)
    assert np.array_equal(out.view(np.int32), want.numpy())


def test_gather_rejects_bad_G_and_size():
    with pytest.raises(ValueError):
        oracle.allgather_param_contig_ref(np.zeros(24, np.uint16), 8, 3, [3])
    with pytest.raises(ValueError):
        oracle.allgather_param_contig_ref(np.zeros(23, np.uint16), 8, 4, [3])


# ------------------------------------------------------------------------------------------------ workloads

def test_log_uniform_splits_recipe():
    e = workloads.log_uniform_splits(4, 64)
    assert e.dtype == np.uint64 and len(e) == 64
    assert np.all(e % 8 == 0) and e.min() >= 1024 and e.max() <= 4_194_304
    assert np.array_equal(e, workloads.log_uniform_splits(4, 64))


def test_rank_buffers_are_seeded_and_in_range():
    a = workloads.rank_buffers(1, 4, 1000, "bf16")
    b = workloads.rank_buffers(1, 4, 1000, "bf16")
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], a[1])
    v = oracle.widen(a[0], "bf16")
    assert v.min() >= -1.0 and v.max() <= 1.0


# ------------------------------------------------------------------------------------ next-step ops

@pytest.mark.parametrize("dtype,V", [("bf16", 8), ("fp16", 8), ("fp32", 4)])
def test_reduce_scatter_chunks_tile_the_message(dtype, V):
    # closed form: chunks are [c*C, (c+1)*C) with C a whole number of 16-byte packs, covering [0, n)
    # exactly once; for n a multiple of W*V every chunk is n/W long
    for n in (0, 1, 7, 8, 9, 63, 64, 65, 1000, 8_388_608, 8_388_611):
        for W in (1, 2, 3, 8, 16):
            spans = [oracle.reduce_scatter_chunk(n, W, dtype, r) for r in range(W)]
            assert spans[0][0] == 0 and spans[-1][1] == n
            for (a0, b0), (a1, b1) in zip(spans, spans[1:]):
                assert b0 == a1
            C = spans[0][1] - spans[0][0]
            if n > 0:
                assert C % V == 0 or C == n
                assert C >= n / W
            if n % (W * V) == 0:
                assert all(b - a == n // W for a, b in spans)


def test_reduce_scatter_shares_concatenate_to_the_all_reduce():
    W, n = 8, 100_003
    bufs = workloads.rank_buffers(60, W, n, "bf16", "normal")
    full = oracle.allreduce_sum_ref(bufs, "bf16")
    parts = [oracle.reduce_scatter_sum_ref(bufs, "bf16", r) for r in range(W)]
    assert np.array_equal(np.concatenate(parts), full)
    # each share only reads its own chunk: poisoning the rest of the inputs leaves it unchanged
    a, b = oracle.reduce_scatter_chunk(n, W, "bf16", 3)
    poisoned = [x.copy() for x in bufs]
    for x in poisoned:
        x[:a] = 0x7FC0
        x[b:] = 0x7FC0
    assert np.array_equal(oracle.reduce_scatter_sum_ref(poisoned, "bf16", 3), full[a:b])


def test_allgather_into_tensor_and_list_against_torch():
    W, T = 6, 1001
    shards = [workloads.random_bits(61, r, T, "fp16") for r in range(W)]
    want = torch.cat([torch.from_numpy(x.astype(np.int32)) for x in shards]).numpy()
    assert np.array_equal(oracle.allgather_into_tensor_ref(shards).astype(np.int32), want)
    outs = oracle.allgather_list_ref(shards)
    assert all(np.array_equal(o, x) and o is not x for o, x in zip(outs, shards))


def test_param_contig_from_shards_matches_split_and_cat():
    W, G = 8, 4
    splits = [int(v) for v in workloads.log_uniform_splits(62, 7, lo=8, hi=4096)]
    T = sum(splits)
    shards = [workloads.random_bits(62, r, T, "int32") for r in range(W)]
    pieces = [torch.from_numpy(x.view(np.int32)).split(splits) for x in shards]
    want = torch.cat([torch.cat([pieces[r][s] for r in range(W)]) for s in range(len(splits))]).numpy()
    assert np.array_equal(oracle.allgather_param_contig_shards_ref(shards, G, splits).view(np.int32), want)
