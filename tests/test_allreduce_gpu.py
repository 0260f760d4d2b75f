"""GPU parity of mr_allreduce_sum (one-shot and two-shot) against the CPU oracle, through the C ABI.

Bit-exact in both modes (NaN payloads compare by NaN-ness only)."""
import numpy as np
import pytest
import torch

import all_gather_amd as mr
import oracle
import workloads
from gpu_util import TORCH_DT, assert_reduce_equal, device, to_bits, to_dev

pytestmark = pytest.mark.gpu
# one-shot, and two-shot under the default (size-chosen) hand-off and each explicit one (per-tile
# flags, per-chunk barrier, grid barrier, last arriver of each tile group)
MODES = ("oneshot", "twoshot", "twoshot:tile", "twoshot:chunk", "twoshot:grid", "twoshot:last")
TWOSHOT_MODES = MODES[1:]


def _call(dbufs, out, mode):
    kind, _, sync = mode.partition(":")
    if sync:
        mr.set_option("twoshot_sync", sync)
    try:
        mr.allreduce_sum(dbufs, out, mode=kind)
    finally:
        if sync:
            mr.set_option("twoshot_sync", "auto")


def _run(dbufs, dtype, n, mode, out=None):
    if out is None:
        out = torch.empty(n, dtype=TORCH_DT[dtype], device=device())
    _call(dbufs, out, mode)
    torch.cuda.synchronize()
    return out


def _check_modes(bufs, dtype, what):
    n = len(bufs[0])
    want = oracle.allreduce_sum_ref(bufs, dtype)
    dbufs = [to_dev(b, dtype) for b in bufs]
    for mode in MODES:
        print(f"[case] {what} {mode}", flush=True)
        got = to_bits(_run(dbufs, dtype, n, mode))
        assert_reduce_equal(got, want, dtype, f"{what} {mode}")
    assert mr.workspace_check() == 0


def test_w4_bf16_64ki_uniform():
    c = workloads.W4_BF16_64KI
    _check_modes(workloads.rank_buffers(c["seed"], c["W"], c["n"], c["dtype"], c["dist"]), "bf16", "W=4 bf16 n=65,536")


def test_w8_bf16_16MiB_normal():
    c = workloads.W8_BF16_16MIB
    _check_modes(workloads.rank_buffers(c["seed"], c["W"], c["n"], c["dtype"], c["dist"]), "bf16", "W=8 bf16 16 MiB")


@pytest.mark.parametrize("W,n,dtype", [(8, 8_388_608 + 4_099, "bf16"), (5, 4_194_304 + 77, "fp32"),
                                       (8, 33_554_432 - 13, "fp16")])
def test_pipelined_oneshot_ragged(W, n, dtype):
    """Sizes in the pipelined one-shot's range (1 to 4 Mi packs of 16 bytes) with more tiles than resident
    workgroups, so workgroups walk several tiles and hold one tile's sums while the next loads, with a
    partial last tile and an element tail; every element against the oracle, both modes."""
    bufs = workloads.rank_buffers(200 + W, W, n, dtype, "uniform")
    _check_modes(bufs, dtype, f"pipelined range {dtype} W={W} n={n}")


def test_pipelined_oneshot_every_W():
    """The pipelined one-shot is a separate build for every W up to 8: each runs just under 4 Mi packs
    (the top of its range, several tiles per resident workgroup at any occupancy) with a ragged element
    tail, one-shot only, every element against the oracle."""
    for W in range(1, 9):
        dtype = ("fp32", "bf16", "fp16")[W % 3]
        V = 4 if dtype == "fp32" else 8
        n = (4 << 20) * V - (V * W + 3)
        bufs = workloads.rank_buffers(700 + W, W, n, dtype, "uniform")
        want = oracle.allreduce_sum_ref(bufs, dtype)
        print(f"[case] pipelined one-shot W={W} {dtype} n={n}", flush=True)
        got = to_bits(_run([to_dev(b, dtype) for b in bufs], dtype, n, "oneshot"))
        assert_reduce_equal(got, want, dtype, f"pipelined one-shot W={W} {dtype} n={n}")
        del bufs, want, got
        torch.cuda.empty_cache()


def test_xcd_twoshot_wide_units_every_W():
    """The XCD-local two-shot is a separate build for every W up to 8; at 16 MiB per rank buffer it runs
    on wide units, under the last arriver (the default) and under per-tile flags with copier workgroups.
    W = 5 and 8 run there in other tests; these are the rest, with a ragged element tail."""
    for W in (2, 3, 4, 6, 7):
        n = 8_388_608 + 2 * W + 1
        bufs = workloads.rank_buffers(740 + W, W, n, "bf16", "uniform")
        want = oracle.allreduce_sum_ref(bufs, "bf16")
        dbufs = [to_dev(b, "bf16") for b in bufs]
        for mode in ("twoshot", "twoshot:tile"):
            print(f"[case] XCD two-shot W={W} n={n} {mode}", flush=True)
            got = to_bits(_run(dbufs, "bf16", n, mode))
            assert_reduce_equal(got, want, "bf16", f"XCD two-shot W={W} {mode}")
        del dbufs
        torch.cuda.empty_cache()
    assert mr.workspace_check() == 0


def test_w16_large_every_mode():
    """W = 16, the largest rank count, at about 8 MiB per rank buffer: the one-shot's wide tiles of one
    pack per lane (W > 8) over many tiles, and every two-shot hand-off on chunk tiles (the XCD-local
    units are for W <= 8), with a ragged element tail."""
    bufs = workloads.rank_buffers(716, 16, 4_194_304 + 13, "bf16", "normal")
    _check_modes(bufs, "bf16", "W=16 bf16 n=4,194,317")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8, 11, 16])
def test_dtypes_W_and_ragged_sizes(dtype, W):
    for n in (1, 7, 8, 9, 1000, 4096 * W + 3, 300_007):
        bufs = workloads.rank_buffers(100 + W, W, n, dtype, "uniform")
        _check_modes(bufs, dtype, f"{dtype} W={W} n={n}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_random_bit_patterns_specials(dtype):
    # uniformly random bits: NaNs, infinities, subnormals, signed zeros and overflow all occur
    W, n = 8, 200_003
    bufs = [workloads.random_bits(7, r, n, dtype) for r in range(W)]
    _check_modes(bufs, dtype, f"random bits {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_structured_special_values(dtype):
    g = np.random.default_rng(3)
    bd = np.uint16 if dtype != "fp32" else np.uint32
    if dtype == "bf16":
        pats = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3F80,
                0xBF80, 0x3380, 0x3B80, 0x3F81]
    else:
        pats = [0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000,
                0xFF800000, 0x7FC00000, 0x3F800000, 0xBF800000, 0x33800000]
    W, n = 4, 16 ** 3
    bufs = [np.array(g.choice(pats, size=n), dtype=bd) for _ in range(W)]
    _check_modes(bufs, dtype, f"specials {dtype}")


def test_in_place_out_is_an_input():
    W, n = 8, 100_000
    bufs = workloads.rank_buffers(11, W, n, "bf16", "normal")
    want = oracle.allreduce_sum_ref(bufs, "bf16")
    for mode in MODES:
        for k in (0, 5):
            dbufs = [to_dev(b, "bf16") for b in bufs]
            _call(dbufs, dbufs[k], mode)
            torch.cuda.synchronize()
            assert_reduce_equal(to_bits(dbufs[k]), want, "bf16", f"in place k={k} {mode}")


def test_repeated_input_pointer():
    n = 50_001
    b = workloads.rank_buffer(12, 0, n, "fp16", "uniform")
    want = oracle.allreduce_sum_ref([b, b, b], "fp16")
    d = to_dev(b, "fp16")
    for mode in MODES:
        assert_reduce_equal(to_bits(_run([d, d, d], "fp16", n, mode)), want, "fp16", mode)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_unaligned_views(dtype):
    W, n = 5, 70_001
    es = 2 if dtype == "bf16" else 4
    bufs = workloads.rank_buffers(13, W, n + 16, dtype, "uniform")
    dev_full = [to_dev(b, dtype) for b in bufs]
    # (a) every pointer shifted by the same element offset: 16-byte body plus element-wise head
    for off in (1, 3):
        views = [d[off:off + n] for d in dev_full]
        want = oracle.allreduce_sum_ref([b[off:off + n] for b in bufs], dtype)
        for mode in MODES:
            outbuf = torch.empty(n + 16, dtype=TORCH_DT[dtype], device=device())
            out = outbuf[off:off + n]
            _call(views, out, mode)
            torch.cuda.synchronize()
            assert_reduce_equal(to_bits(out), want, dtype, f"same phase off={off} {mode}")
    # (b) pointers with different 16-byte phases: element-wise path
    offs = [r % (16 // es) for r in range(W)]
    views = [dev_full[r][offs[r]:offs[r] + n] for r in range(W)]
    want = oracle.allreduce_sum_ref([bufs[r][offs[r]:offs[r] + n] for r in range(W)], dtype)
    for mode in MODES:
        got = to_bits(_run(views, dtype, n, mode))
        assert_reduce_equal(got, want, dtype, f"mixed phases {mode}")


def test_oneshot_equals_twoshot_and_is_deterministic():
    W, n = 8, 1_048_579
    bufs = [workloads.random_bits(14, r, n, "bf16") for r in range(W)]
    dbufs = [to_dev(b, "bf16") for b in bufs]
    ref = to_bits(_run(dbufs, "bf16", n, "oneshot"))
    out = torch.empty(n, dtype=torch.bfloat16, device=device())
    for i in range(60):
        mode = MODES[i % len(MODES)]
        _call(dbufs, out, mode)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), ref), f"launch {i} ({mode}) differs"
    assert mr.workspace_check() == 0


@pytest.mark.parametrize("sync", ["tile", "chunk", "grid", "last", "tile:wide_pair", "tile:wide_pair:3",
                                  "last:wide_pair", "last:wide_pair:3"])
def test_twoshot_stale_stage_is_never_read(sync):
    """Two input sets alternate on one caller-owned workspace, so when a call starts its stage still
    holds the previous call's (different) sums: a phase-2 copy that ran ahead of its phase-1 producer
    would surface as a mismatch.  The last case shifts every pointer by 3 elements (a common 6-byte
    phase: 16-byte body after an element-wise head), so the XCD-local kernel's units start 6 bytes
    past a 16-byte boundary of out."""
    W, n = 8, 4_194_304 + 24
    sync, _, shape = sync.partition(":")
    shape, _, off = shape.partition(":")
    off = int(off or 0)
    sets = [workloads.rank_buffers(15 + k, W, n, "bf16", "normal") for k in range(2)]
    wants = [oracle.allreduce_sum_ref(b, "bf16") for b in sets]
    dsets = []
    for s_ in sets:
        views = []
        for b in s_:
            full = torch.empty(n + 8, dtype=torch.bfloat16, device=device())
            full[off:off + n].copy_(to_dev(b, "bf16"))
            views.append(full[off:off + n])
        dsets.append(views)
    ws = torch.empty(mr.workspace_bytes(W, n, "bf16"), dtype=torch.uint8, device=device())
    mr.set_workspace(ws)
    mr.set_option("twoshot_sync", sync)
    mr.set_option("tile_shape", shape or "auto")
    try:
        outs = [torch.empty(n + 8, dtype=torch.bfloat16, device=device())[off:off + n] for _ in range(2)]
        for i in range(200):
            k = i % 2
            outs[k].fill_(0)
            mr.allreduce_sum(dsets[k], outs[k], mode="twoshot")
            if i % 20 in (0, 1) or i >= 198:
                torch.cuda.synchronize()
                assert_reduce_equal(to_bits(outs[k]), wants[k], "bf16", f"{sync} launch {i}")
        assert mr.workspace_check() == 0
    finally:
        mr.set_option("tile_shape", "auto")
        mr.set_option("twoshot_sync", "auto")
        mr.set_workspace(None)


@pytest.mark.parametrize("sync", ["tile", "chunk", "grid", "last"])
def test_twoshot_poisoned_stage_stress(sync):
    """Before every launch, a fill on the launch stream overwrites the whole stage (and out) with 0xFF
    bytes, a NaN in every element; 80 launches per tile shape, at sizes whose grids differ (under the
    last arriver, auto takes XCD-local units of 1 KiB and 4 KiB at the two auto sizes), must all
    match the oracle bit for bit.  A phase-2 copy that ran ahead of its producer, or a phase-1 tile
    that was never written, would publish the poison."""
    W = 8
    cases = [("narrow", 30_011), ("medium", 1_000_003), ("wide", 4_194_304 + 8), ("auto", 2_500_001),
             ("auto", 300_017), ("wide_pair", 8_388_608 + 24)]
    n_max = max(n for _, n in cases)
    ws = torch.empty(mr.workspace_bytes(W, n_max, "bf16"), dtype=torch.uint8, device=device())
    flags_cap = ws.numel() >> 8
    stage_off = 16384 + ((flags_cap * 4 + 255) // 256) * 256
    mr.set_workspace(ws)
    mr.set_option("twoshot_sync", sync)
    try:
        for shape, n in cases:
            print(f"[case] poisoned stage {sync} {shape} n={n}", flush=True)
            mr.set_option("tile_shape", shape)
            bufs = workloads.rank_buffers(70 + n % 97, W, n, "bf16", "uniform")
            want = torch.from_numpy(oracle.allreduce_sum_ref(bufs, "bf16").view(np.int16)).to(device())
            dbufs = [to_dev(b, "bf16") for b in bufs]
            out = torch.empty(n, dtype=torch.bfloat16, device=device())
            bad = torch.zeros((), dtype=torch.int64, device=device())
            for _ in range(80):
                ws[stage_off:].fill_(0xFF)
                out.view(torch.int16).fill_(-1)
                mr.allreduce_sum(dbufs, out, mode="twoshot")
                bad += (out.view(torch.int16) != want).sum()
            assert int(bad) == 0, f"{sync} {shape} n={n}: {int(bad)} poisoned or wrong elements"
            assert mr.workspace_check() == 0
    finally:
        mr.set_option("tile_shape", "auto")
        mr.set_option("twoshot_sync", "auto")
        mr.set_workspace(None)


def test_caller_workspace_too_small():
    W, n = 8, 1_000_000
    bufs = [to_dev(b, "bf16") for b in workloads.rank_buffers(17, W, n, "bf16", "uniform")]
    out = torch.empty(n, dtype=torch.bfloat16, device=device())
    with pytest.raises(mr.MRError) as ei:  # cannot even hold the barrier words
        mr.set_workspace(torch.empty(4096, dtype=torch.uint8, device=device()))
    assert ei.value.status == -1
    small = torch.empty(1 << 16, dtype=torch.uint8, device=device())
    mr.set_workspace(small)
    try:
        with pytest.raises(mr.MRError) as ei:
            mr.allreduce_sum(bufs, out, mode="twoshot")
        assert ei.value.status == -4
    finally:
        mr.set_workspace(None)
    mr.allreduce_sum(bufs, out, mode="twoshot")  # library-owned workspace again
    torch.cuda.synchronize()
    assert mr.workspace_check() == 0


def test_bounded_wait_reports_and_recovers():
    """With a spin limit of 0, a grid-barrier phase-2 workgroup that starts while the last phase-1
    tiles still run gives up at its first poll: the call finishes, the workspace error word says so,
    mr_workspace_check clears it, and the next call is correct."""
    W, n = 8, 8_388_608
    bufs = workloads.rank_buffers(18, W, n, "bf16", "normal")
    want = oracle.allreduce_sum_ref(bufs, "bf16")
    dbufs = [to_dev(b, "bf16") for b in bufs]
    out = torch.empty(n, dtype=torch.bfloat16, device=device())
    mr.allreduce_sum(dbufs, out, mode="twoshot")  # a library-owned workspace exists and is clean
    assert mr.workspace_check() == 0
    mr.set_option("twoshot_sync", "grid")
    mr.set_option("spin_limit", 0)
    try:
        mr.allreduce_sum(dbufs, out, mode="twoshot")
        flags = mr.workspace_check()
    finally:
        mr.set_option("spin_limit", 1 << 22)
        mr.set_option("twoshot_sync", "auto")
    assert flags & 1, "a phase-2 wait should have given up"
    for mode in ("twoshot:tile", "twoshot:grid"):
        out.fill_(0)
        _call(dbufs, out, mode)
        torch.cuda.synchronize()
        assert_reduce_equal(to_bits(out), want, "bf16", f"after recovery {mode}")
    assert mr.workspace_check() == 0


def test_xcd_twoshot_timeouts_recompute_and_leave_no_flag_set():
    """XCD-local two-shot with a spin limit of 0: a copier whose unit is not yet published gives up at
    once, claims the flag and recomputes the unit from the rank buffers.  The output must still match
    the oracle, the error word may only carry the 'recomputed' bits (never bit 0), and after the launch
    every flag word of the caller-owned workspace is zero again, so a late producer's release cannot
    satisfy the next launch; the next launch (normal spin limit) is correct too."""
    W, n = 8, 8_388_608 + 40
    sets = [workloads.rank_buffers(90 + k, W, n, "bf16", "normal") for k in range(2)]
    wants = [oracle.allreduce_sum_ref(b, "bf16") for b in sets]
    dsets = [[to_dev(b, "bf16") for b in s] for s in sets]
    nbytes = mr.workspace_bytes(W, n, "bf16")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device())
    flags_cap = nbytes >> 8
    mr.set_workspace(ws)
    mr.set_option("twoshot_sync", "tile")
    mr.set_option("tile_shape", "wide_pair")
    try:
        outs = [torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(2)]
        for rep in range(6):
            k = rep % 2
            mr.set_option("spin_limit", 0 if k == 0 else 1 << 22)
            outs[k].view(torch.int16).fill_(-1)
            mr.allreduce_sum(dsets[k], outs[k], mode="twoshot")
            torch.cuda.synchronize()
            assert_reduce_equal(to_bits(outs[k]), wants[k], "bf16", f"rep {rep} spin {'0' if k == 0 else 'default'}")
            leftover = int((ws[16384:16384 + 4 * flags_cap].view(torch.int32) != 0).sum())
            assert leftover == 0, f"rep {rep}: {leftover} flag words left set"
            err = int(ws[:16384].view(torch.int32)[(3 * 16 * 64 + 64):(3 * 16 * 64 + 65)].item())
            assert err & 1 == 0, f"rep {rep}: error word {err:#x}"
        flags = mr.workspace_check()
        assert flags & 1 == 0
        print(f"[case] error word after the spin-0 launches: {flags:#x}", flush=True)
    finally:
        mr.set_option("spin_limit", 1 << 22)
        mr.set_option("tile_shape", "auto")
        mr.set_option("twoshot_sync", "auto")
        mr.set_workspace(None)


def test_twoshot_on_two_streams_concurrently():
    W, n = 8, 2_097_152 + 8
    sets = [workloads.rank_buffers(16 + k, W, n, "bf16", "uniform") for k in range(2)]
    wants = [oracle.allreduce_sum_ref(b, "bf16") for b in sets]
    dsets = [[to_dev(b, "bf16") for b in s] for s in sets]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(30):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                _call(dsets[k], outs[k], TWOSHOT_MODES[rep % len(TWOSHOT_MODES)])
    torch.cuda.synchronize()
    for k in range(2):
        assert_reduce_equal(to_bits(outs[k]), wants[k], "bf16", f"stream {k}")
        assert mr.workspace_check(streams[k]) == 0


def test_cross_stream_consumer_waits_on_event():
    """The reduce runs on a side stream with per-rep inputs; a consumer on the main stream waits on an
    event recorded after it and reads the output (the overlap pattern of FSDP's all-gather hook)."""
    W, n = 8, 1_000_003
    side = torch.cuda.Stream()
    out = torch.empty(n, dtype=torch.bfloat16, device=device())
    for rep in range(4):
        bufs = workloads.rank_buffers(30 + rep, W, n, "bf16", "normal")
        want = oracle.allreduce_sum_ref(bufs, "bf16")
        dbufs = [to_dev(b, "bf16") for b in bufs]
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            _call(dbufs, out, MODES[rep % len(MODES)])
            ev = torch.cuda.Event()
            ev.record(side)
        torch.cuda.current_stream().wait_event(ev)
        copy = out.clone()  # consumer on the main stream
        torch.cuda.synchronize()
        assert_reduce_equal(to_bits(copy), want, "bf16", f"rep {rep}")


@pytest.mark.parametrize("per_rank", workloads.SWEEP_BYTES_PER_RANK, ids=lambda b: f"{b >> 10}KiB")
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_w8_size_sweep(dtype, per_rank):
    es = 2 if dtype == "bf16" else 4
    n = per_rank // es
    bufs = workloads.rank_buffers(3, 8, n, dtype, "uniform")
    dbufs = [to_dev(b, dtype) for b in bufs]
    if n <= 32 * 2 ** 20:
        want = oracle.allreduce_sum_ref(bufs, dtype)
        idx = None
    else:  # sampled outputs: the oracle on 2^20 strided columns
        idx = np.linspace(0, n - 1, 1 << 20).astype(np.int64)
        want = oracle.allreduce_sum_ref([b[idx] for b in bufs], dtype)
    del bufs
    for mode in MODES:
        print(f"[case] size sweep {dtype} per-rank {per_rank >> 10} KiB {mode}", flush=True)
        got = to_bits(_run(dbufs, dtype, n, mode))
        assert_reduce_equal(got if idx is None else got[idx], want, dtype, f"{dtype} {per_rank} {mode}")
    del dbufs
    torch.cuda.empty_cache()
    assert mr.workspace_check() == 0


def test_twoshot_realigned_path_large():
    """Element-aligned pointers with different 16-byte phases take the realigned 16-byte path: a large
    call (past 32 MiB per rank buffer, so the default hand-off is no longer the last arriver) checked
    on sampled outputs, one-shot and two-shot under the hand-offs that then apply."""
    W, n = 8, 20_000_003
    bufs = workloads.rank_buffers(19, W, n + 8, "bf16", "uniform")
    offs = [r % 8 for r in range(W)]
    dev_full = [to_dev(b, "bf16") for b in bufs]
    views = [dev_full[r][offs[r]:offs[r] + n] for r in range(W)]
    idx = np.linspace(0, n - 1, 1 << 18).astype(np.int64)
    want = oracle.allreduce_sum_ref([bufs[r][offs[r]:offs[r] + n][idx] for r in range(W)], "bf16")
    for mode in ("oneshot", "twoshot:tile", "twoshot:chunk"):
        got = to_bits(_run(views, "bf16", n, mode))
        assert_reduce_equal(got[idx], want, "bf16", f"realigned path {mode}")
    assert mr.workspace_check() == 0


def test_w8_fp32_512MiB_alone_and_beside_a_gemm():
    """W=8 fp32 rank buffers of 134,217,728 elements (512 MiB each), uniform[-1,1): sampled outputs
    against the oracle, alone and while bf16 8192^3 GEMMs run on a second stream."""
    c = workloads.W8_FP32_512MIB
    W, n = c["W"], c["n"]
    idx = np.linspace(0, n - 1, 1 << 20).astype(np.int64)
    dbufs, cols = [], []
    for r in range(W):  # one rank at a time keeps host memory near 1 GiB
        b = workloads.rank_buffer(c["seed"], r, n, "fp32", c["dist"])
        cols.append(b[idx].copy())
        dbufs.append(to_dev(b, "fp32"))
        del b
    want = oracle.allreduce_sum_ref(cols, "fp32")
    out = torch.empty(n, dtype=torch.float32, device=device())
    for mode in ("oneshot", "twoshot:tile"):
        out.zero_()
        got = to_bits(_run(dbufs, "fp32", n, mode))
        assert_reduce_equal(got[idx], want, "fp32", f"W=8 fp32 512 MiB {mode}")
    # beside a GEMM on another stream (default priority)
    g = torch.Generator(device=device())
    g.manual_seed(5)
    a = (torch.randn(8192, 8192, device=device(), generator=g) * 0.02).to(torch.bfloat16)
    bm = (torch.randn(8192, 8192, device=device(), generator=g) * 0.02).to(torch.bfloat16)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(6):
            cgemm = torch.matmul(a, bm)
    idx_dev = torch.from_numpy(idx).to(device())
    for mode in MODES:  # every hand-off must make progress while GEMM workgroups hold the CUs
        out.zero_()
        _call(dbufs, out, mode)
        got = to_bits(out.index_select(0, idx_dev))  # waits for this stream only; the GEMMs go on
        assert_reduce_equal(got, want, "fp32", f"W=8 fp32 512 MiB {mode} under GEMM")
        with torch.cuda.stream(side):
            for _ in range(2):
                cgemm = torch.matmul(a, bm)
    torch.cuda.synchronize()
    assert torch.isfinite(cgemm.float()).all()
    assert mr.workspace_check() == 0
    del dbufs, out, a, bm, cgemm
    torch.cuda.empty_cache()


def _structured_partners(dtype, count=64):
    g = np.random.default_rng(21)
    if dtype == "bf16":
        base = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080, 0x3F80, 0xBF80, 0x3B80, 0xBB80,
                0x3380, 0xB380, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3F00, 0x4000, 0xC000, 0x3C00, 0x0100]
    else:
        base = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x8400, 0x3C00, 0xBC00, 0x1000, 0x9000,
                0x1400, 0x9400, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00, 0x7E00, 0x3800, 0x4000, 0xC000, 0x4C00, 0x4800]
    extra = g.integers(0, 65536, size=count - len(base), dtype=np.uint32)
    return np.array(base + list(extra), dtype=np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_every_16bit_pattern_against_structured_partners(dtype):
    """All 65,536 input patterns, each summed with 64 structured partners (signed zeros, subnormal
    edges, rounding ties, largest finite, infinities, NaN): the hardware conversions and adds agree
    with the oracle bit for bit, in both modes; W=3 adds the negated partner (exact cancellation)."""
    part = _structured_partners(dtype)
    x0 = np.tile(np.arange(65536, dtype=np.uint32).astype(np.uint16), len(part))
    x1 = np.repeat(part, 65536)
    x2 = x1 ^ np.uint16(0x8000)
    for bufs in ([x0, x1], [x1, x0, x2]):
        _check_modes(bufs, dtype, f"16-bit sweep {dtype} W={len(bufs)}")


@pytest.mark.parametrize("shape", ["wide", "medium", "narrow", "wide_pair"])
def test_every_tile_shape_in_every_mode(shape):
    """Each forced tile shape (one-shot lanes x packs, two-shot phase-1 tile) gives the oracle's bits,
    on sizes that leave partial tiles, partial chunks and unaligned edges."""
    mr.set_option("tile_shape", shape)
    try:
        for dtype in ("bf16", "fp32"):
            for W, n in ((8, 1_000_003), (3, 65_541), (16, 300_007), (8, 4_194_304 + 8)):
                bufs = workloads.rank_buffers(60 + W, W, n, dtype, "uniform")
                _check_modes(bufs, dtype, f"{shape} {dtype} W={W} n={n}")
    finally:
        mr.set_option("tile_shape", "auto")


def test_rank_buffers_beyond_2GiB():
    """W=3 bf16 rank buffers of 2^30 + 12,347 elements (just over 2 GiB each), so byte offsets pass 2^31 in
    every kernel: one-shot wide tiles, wide pairs, two-shot.  Finite random bit patterns (exponent's top
    bit cleared); sampled outputs, the first and last 4096 included, against the oracle."""
    W, n = 3, (1 << 30) + 12_347
    bufs = [workloads.random_bits(91, r, n, "bf16") & np.uint16(0xBFFF) for r in range(W)]
    idx = np.unique(np.concatenate([np.arange(4096), np.arange(n - 4096, n),
                                    np.linspace(0, n - 1, 1 << 20).astype(np.int64)]))
    want = oracle.allreduce_sum_ref([b[idx] for b in bufs], "bf16")
    dbufs = [to_dev(b, "bf16") for b in bufs]
    del bufs
    out = torch.empty(n, dtype=torch.bfloat16, device=device())
    try:
        for mode, shape in (("oneshot", "auto"), ("oneshot", "wide_pair"), ("twoshot", "auto")):
            print(f"[case] beyond 2 GiB {mode} shape={shape}", flush=True)
            out.view(torch.int16).fill_(-1)
            mr.set_option("tile_shape", shape)
            try:
                _run(dbufs, "bf16", n, mode, out)
            finally:
                mr.set_option("tile_shape", "auto")
            got = out.view(torch.int16)[torch.from_numpy(idx).to(device())].cpu().numpy().view(np.uint16)
            assert_reduce_equal(got, want, "bf16", f"beyond 2 GiB {mode} {shape}")
        assert mr.workspace_check() == 0
    finally:
        del dbufs, out
        torch.cuda.empty_cache()


@pytest.mark.parametrize("write", [1, 2])
def test_stream_mix_probe_writes_the_xor(write):
    """The bench's ceiling probe computes what it claims (the XOR of its K streams) on both schedules,
    with a ragged tail, so its rate is that of the full access pattern."""
    import ctypes

    L = mr.lib()
    f = L.mrx_stream_mix
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_void_p]
    nwords = 3 * 1024 * 1024 + 37  # more tiles than resident workgroups, and a partial last tile
    g = torch.Generator(device=device())
    g.manual_seed(write)
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (4 * nwords,), dtype=torch.int32, device=device(), generator=g)
            for _ in range(8)]
    out = torch.full((4 * nwords,), -1, dtype=torch.int32, device=device())
    ptrs = (ctypes.c_void_p * 8)(*[b.data_ptr() for b in bufs])
    print(f"[case] stream_mix write={write} words={nwords}", flush=True)
    assert f(ptrs, 8, out.data_ptr(), 16 * nwords, write, torch.cuda.current_stream().cuda_stream or None) == 0
    want = bufs[0].clone()
    for b in bufs[1:]:
        want ^= b
    torch.cuda.synchronize()
    assert torch.equal(out, want)
