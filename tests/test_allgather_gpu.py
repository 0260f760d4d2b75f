"""GPU parity of mr_allgather_param_contig against the CPU oracle, through the C ABI.  Bit-exact."""
import numpy as np
import pytest
import torch

import all_gather_amd as mr
import oracle
import workloads
from gpu_util import TORCH_DT, device, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _gather(src_bits, W, G, splits, dtype):
    src = to_dev(src_bits, dtype)
    out = torch.empty_like(src)
    out.view(torch.uint8).fill_(0xA5)
    mr.allgather_param_contig(src, W, G, splits, out)
    torch.cuda.synchronize()
    return to_bits(out)


def _check(src_bits, W, G, splits, dtype, what):
    print(f"[case] {what}", flush=True)
    want = oracle.allgather_param_contig_ref(src_bits, W, G, splits)
    got = _gather(src_bits, W, G, splits, dtype)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:8].tolist()}"


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32", "int32"])
def test_fsdp_splits_random_bits(dtype):
    c = workloads.FSDP_SPLITS_W8_G4_P64
    splits = workloads.log_uniform_splits(c["seed"], c["P"])
    T = int(splits.sum())
    src = workloads.gather_source(c["seed"], c["W"], T, dtype)
    _check(src, c["W"], c["G"], splits, dtype, f"FSDP splits W=8 G=4 P=64 {dtype} T={T}")


def test_G_does_not_change_the_output():
    W = 8
    splits = [int(x) for x in workloads.log_uniform_splits(50, 20, lo=8, hi=100_000)]
    T = sum(splits)
    src = workloads.gather_source(50, W, T, "fp16")
    outs = [_gather(src, W, G, splits, "fp16") for G in (1, 2, 4, 8)]
    want = oracle.allgather_param_contig_ref(src, W, 4, splits)
    for o in outs:
        assert np.array_equal(o, want)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_and_empty_splits(dtype):
    # odd element counts give pieces whose source and destination 16-byte phases differ
    W, G = 6, 3
    splits = [0, 1, 7, 8, 9, 4095, 4096, 4097, 0, 8191, 16385, 3, 100_001]
    T = sum(splits)
    src = workloads.gather_source(51, W, T, dtype)
    _check(src, W, G, splits, dtype, f"ragged {dtype}")


def test_single_split_and_single_rank():
    src = workloads.gather_source(52, 4, 10_000, "int32")
    _check(src, 4, 2, [10_000], "int32", "P=1")
    src = workloads.gather_source(53, 1, 777, "bf16")
    _check(src, 1, 1, [100, 600, 77], "bf16", "W=1")


def test_more_params_than_one_launch():
    W, G = 8, 4
    splits = [int(x) for x in workloads.log_uniform_splits(54, 300, lo=8, hi=20_000)]
    T = sum(splits)
    src = workloads.gather_source(54, W, T, "bf16")
    _check(src, W, G, splits, "bf16", "P=300 (3 launches)")


def test_unaligned_base_pointers():
    W, G = 4, 2
    splits = [64, 1000, 24, 8]
    T = sum(splits)
    src = workloads.gather_source(55, W, T + 8, "bf16")[: W * T + 8]
    full = to_dev(src, "bf16")
    for so, do in ((1, 1), (1, 0), (3, 5)):
        s = full[so:so + W * T]
        ob = torch.empty(W * T + 8, dtype=torch.bfloat16, device=device())
        o = ob[do:do + W * T]
        mr.allgather_param_contig(s, W, G, splits, o)
        torch.cuda.synchronize()
        want = oracle.allgather_param_contig_ref(src[so:so + W * T], W, G, splits)
        assert np.array_equal(to_bits(o), want), (so, do)


def test_over_2GiB_int32_68M_per_rank():
    """Eight ranks of 68,157,440 int32 elements: the gathered buffer is 2.18 GB, past 2^31 bytes, so a
    32-bit byte offset anywhere would misplace data."""
    W, G = 8, 4
    splits = [33_554_432, 33_554_432, 1_048_576]
    T = sum(splits)
    src = np.arange(W * T, dtype=np.uint32)  # every element tagged with its own index
    print(f"[case] 68M int32 per rank, {W * T * 4 / 1e9:.2f} GB", flush=True)
    dsrc = torch.arange(W * T, dtype=torch.int32, device=device())
    out = torch.empty_like(dsrc)
    mr.allgather_param_contig(dsrc, W, G, splits, out)
    torch.cuda.synchronize()
    want = oracle.allgather_param_contig_ref(src, W, G, splits)
    got = to_bits(out)
    assert np.array_equal(got, want)
    del dsrc, out
    torch.cuda.empty_cache()


def test_gather_on_side_stream_with_event_consumer():
    W, G = 8, 4
    splits = [int(x) for x in workloads.log_uniform_splits(56, 16, lo=1024, hi=2_000_000)]
    T = sum(splits)
    side = torch.cuda.Stream()
    out = torch.empty(W * T, dtype=torch.float32, device=device())
    for rep in range(3):
        src = workloads.gather_source(60 + rep, W, T, "fp32")
        want = oracle.allgather_param_contig_ref(src, W, G, splits)
        dsrc = to_dev(src, "fp32")
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            mr.allgather_param_contig(dsrc, W, G, splits, out)
            ev = torch.cuda.Event()
            ev.record(side)
        torch.cuda.current_stream().wait_event(ev)
        copy = out.clone()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(copy), want), rep


def test_more_split_sets_than_cached_plans():
    """Twelve distinct split sets, each gathered twice from fresh buffers: the host keeps a few launch
    plans per thread, and every call, hit or miss, must bind its own pointers."""
    W, G = 8, 4
    for rep in range(2):
        for k in range(12):
            splits = [1000 + 8 * k, 24 + k, 4096, 7 * k]
            T = sum(splits)
            print(f"[case] plan cache rep={rep} k={k} T={T}", flush=True)
            src = workloads.gather_source(200 + 12 * rep + k, W, T, "bf16")
            out = torch.empty(W * T, dtype=torch.bfloat16, device=device())
            mr.allgather_param_contig(to_dev(src, "bf16"), W, G, splits, out)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(out), oracle.allgather_param_contig_ref(src, W, G, splits)), (rep, k)


@pytest.mark.parametrize("dtype,E", [("fp32", 4099), ("fp32", 420_349), ("bf16", 4097), ("bf16", 262_147)])
def test_equal_splits_with_unaligned_sizes(dtype, E):
    """64 equal splits whose byte size is not a multiple of 16: segments take every combination of
    source and destination 16-byte (and, for bf16, 4-byte) phase, so the word-copy paths run at scale."""
    W, G, P = 8, 4, 64
    splits = [E] * P
    T = E * P
    print(f"[case] equal unaligned splits {dtype} E={E}", flush=True)
    src = workloads.gather_source(400 + E % 97, W, T, dtype)
    out = torch.empty(W * T, dtype=TORCH_DT[dtype], device=device())
    mr.allgather_param_contig(to_dev(src, dtype), W, G, splits, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_param_contig_ref(src, W, G, splits))


_SLOT_REUSE_CHILD = r"""
import torch
import all_gather_amd as mr
W, G = 8, 4
def run(splits):
    T = sum(splits)
    src = torch.arange(W * T, dtype=torch.int32, device="cuda:0").to(torch.int16).view(torch.bfloat16)
    out = torch.empty_like(src)
    mr.allgather_param_contig(src, W, G, splits, out)
    torch.cuda.synchronize()
run([3, 5])                        # odd sizes: pieces out of 16-byte phase (realign build)
for k in range(7):
    run([8 * (k + 2), 16])         # fill the other cached-plan slots with aligned plans
run([64, 128])                     # aligned, and lands in the first plan's slot
"""


def test_reused_plan_slot_keeps_no_stale_phase_bits():
    """A plan computed into a reused cache slot must not inherit the previous plan's phase bits, which
    would send an all-aligned gather to the slower realign build.  The launch trace names the build."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MR_TRACE="1", PYTHONPATH=root)
    print("[case] plan slot reuse (child process, MR_TRACE=1)", flush=True)
    r = subprocess.run([sys.executable, "-c", _SLOT_REUSE_CHILD], cwd=root, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[mr] gather")]
    assert len(lines) == 9, r.stderr[-2000:]
    assert "realign=1" in lines[0]
    assert all("realign=0" in ln for ln in lines[1:]), lines


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32", "int32"])
def test_sdma_engines_match_the_oracle(dtype):
    """mr_allgather_param_contig_sdma gives the oracle's bits on the FSDP-style splits, on ragged splits with
    empty and odd pieces, and with one parameter (a single merged copy), with every piece on the engines,
    with the small parameters on the compute-unit kernel (below 8 KiB and 1 MiB pieces), and with every
    parameter on the kernel; the output is read back both by the host and by a kernel (torch compare)."""
    n_eng = mr.sdma_engines()
    print(f"[case] SDMA engines: {n_eng}", flush=True)
    assert n_eng > 0, f"no SDMA engines offered for device-local copies (HSA status {mr.lib().mr_last_hip_error()})"
    c = workloads.FSDP_SPLITS_W8_G4_P64
    cases = [("fsdp", c["W"], c["G"], [int(x) for x in workloads.log_uniform_splits(c["seed"], c["P"])]),
             ("ragged", 6, 3, [0, 1, 7, 8, 9, 4095, 4096, 4097, 0, 8191, 16385, 3, 100_001]),
             ("one param", 8, 8, [3_000_017])]
    for name, W, G, splits in cases:
        T = sum(splits)
        print(f"[case] sdma {name} {dtype} W={W} G={G} P={len(splits)} T={T}", flush=True)
        src_bits = workloads.gather_source(60 + len(splits), W, T, dtype)
        want = oracle.allgather_param_contig_ref(src_bits, W, G, splits)
        src = to_dev(src_bits, dtype)
        ref = torch.empty_like(src)
        mr.allgather_param_contig(src, W, G, splits, ref)  # the kernel path, compared on the device
        it = torch.int16 if src.element_size() == 2 else torch.int32
        out = torch.empty_like(src)
        prev = mr.get_option("sdma_cu_below")
        try:
            for cu_below in (0, 8192, 1 << 20, 2 ** 32 - 1):
                print(f"[case] sdma {name} {dtype} cu_below={cu_below}", flush=True)
                mr.set_option("sdma_cu_below", cu_below)
                out.view(torch.uint8).fill_(0xA5)
                torch.cuda.synchronize()
                mr.allgather_param_contig_sdma(src, W, G, splits, out)
                bad = np.flatnonzero(to_bits(out) != want)
                assert bad.size == 0, f"sdma {name} {dtype} {cu_below}: {bad.size} mismatches, first at {bad[:8].tolist()}"
                assert torch.equal(out.view(it), ref.view(it)), f"sdma {name} {dtype} {cu_below}: differs from the kernel"
        finally:
            mr.set_option("sdma_cu_below", prev)


def test_sdma_gather_waits_for_earlier_stream_work():
    """The engines are not ordered by the stream, so the copy-engine gather waits for the stream's earlier
    work before its copies start: here the source and the output are both written by kernels enqueued
    just before the call, with no host synchronisation in between (FSDP-style splits, bf16, every piece
    on the engines and the default split)."""
    c = workloads.FSDP_SPLITS_W8_G4_P64
    W, G = c["W"], c["G"]
    splits = [int(x) for x in workloads.log_uniform_splits(c["seed"], c["P"])]
    T = sum(splits)
    src_bits = workloads.gather_source(77, W, T, "bf16")
    want = oracle.allgather_param_contig_ref(src_bits, W, G, splits)
    staged = to_dev(src_bits, "bf16")
    src = torch.empty_like(staged)
    out = torch.empty_like(staged)
    prev = mr.get_option("sdma_cu_below")
    try:
        for cu_below in (0, prev):
            print(f"[case] sdma after stream work cu_below={cu_below}", flush=True)
            mr.set_option("sdma_cu_below", cu_below)
            src.view(torch.int16).fill_(0)
            torch.cuda.synchronize()
            src.copy_(staged)                      # about 0.1 ms of kernel work, still running at the call
            out.view(torch.int16).fill_(-1)        # a fill that must land before the copies, not after
            mr.allgather_param_contig_sdma(src, W, G, splits, out)
            bad = np.flatnonzero(to_bits(out) != want)
            assert bad.size == 0, f"cu_below={cu_below}: {bad.size} mismatches, first at {bad[:8].tolist()}"
    finally:
        mr.set_option("sdma_cu_below", prev)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fsdp_splits_of_any_size(dtype):
    """The FSDP-style workload with split sizes not rounded to 8 elements: most pieces take the realigning
    16-byte copy, in whole 16 KiB tiles and in partial ones, at the full size."""
    c = workloads.FSDP_SPLITS_W8_G4_P64
    splits = workloads.log_uniform_splits(c["seed"], c["P"], mult=1)
    T = int(splits.sum())
    src = workloads.gather_source(c["seed"] + 1, c["W"], T, dtype)
    _check(src, c["W"], c["G"], splits, dtype, f"FSDP splits of any size W=8 G=4 P=64 {dtype} T={T}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tiles_crossing_one_rank_boundary(dtype):
    """Splits whose rank pieces are 16 to 40 KiB, all whole 16-byte packs, so many whole tiles cross one
    rank boundary at many different pack offsets (the straight-line two-rank copy), beside tiles crossing
    none or several; from a rank-major source and from separate shards, every element against the oracle."""
    W, G = 8, 2
    es = 2 if dtype == "bf16" else 4
    splits = [(16384 + 16 * 37 * k) // es for k in range(40)]
    T = sum(splits)
    print(f"[case] two-rank tiles {dtype} T={T}", flush=True)
    src = workloads.gather_source(430, W, T, dtype)
    want = oracle.allgather_param_contig_ref(src, W, G, splits)
    assert np.array_equal(_gather(src, W, G, splits, dtype), want)
    shards = [src[r * T:(r + 1) * T] for r in range(W)]
    out = torch.empty(W * T, dtype=TORCH_DT[dtype], device=device())
    mr.allgather_param_contig_shards([to_dev(s, dtype) for s in shards], G, splits, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), want)
