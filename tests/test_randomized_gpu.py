"""Seeded random combinations of every argument the entry points take, each checked against the CPU
oracle through the C ABI: for the sum-reduce W, n (tiny, ragged and multi-tile), dtype, mode, two-shot
hand-off, tile shape and a per-pointer element offset (which mixes 16-byte phases); for the gathers W,
G, P, split sizes (empty ones included), dtype, entry point (the copy-engine gather with a random split
between engines and kernel included) and base offsets."""
import numpy as np
import pytest
import torch

import all_gather_amd as mr
import oracle
import workloads
from gpu_util import TORCH_DT, assert_reduce_equal, device, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _view(host_bits, dtype, off):
    """A device tensor holding host_bits that starts `off` elements into its allocation."""
    full = np.zeros(len(host_bits) + off, dtype=host_bits.dtype)
    full[off:] = host_bits
    return to_dev(full, dtype)[off:]


@pytest.mark.parametrize("block", range(6))
def test_random_reduce_cases(block):
    rng = np.random.default_rng(9000 + block)
    for case in range(20):
        W = int(rng.integers(1, 17))
        n = int(rng.choice([1, 2, 7, 9, 63, 1000, 65_537, 300_001, 1_500_007]))
        dtype = str(rng.choice(["bf16", "fp16", "fp32"]))
        mode = str(rng.choice(["oneshot", "twoshot"]))
        sync = str(rng.choice(["auto", "tile", "chunk", "grid", "last"]))
        shape = str(rng.choice(["auto", "wide", "medium", "narrow", "wide_pair"]))
        aligned = rng.random() < 0.6
        offs = [0] * (W + 1) if aligned else [int(x) for x in rng.integers(0, 9, size=W + 1)]
        what = f"block {block} case {case}: W={W} n={n} {dtype} {mode} sync={sync} shape={shape} offs={offs}"
        print(f"[case] {what}", flush=True)
        bufs = workloads.rank_buffers(int(rng.integers(1 << 30)), W, n, dtype, "normal")
        dbufs = [_view(b, dtype, offs[r]) for r, b in enumerate(bufs)]
        out = _view(np.zeros(n, dtype=bufs[0].dtype), dtype, offs[W])
        mr.set_option("twoshot_sync", sync)
        mr.set_option("tile_shape", shape)
        try:
            mr.allreduce_sum(dbufs, out, mode=mode)
            torch.cuda.synchronize()
        finally:
            mr.set_option("twoshot_sync", "auto")
            mr.set_option("tile_shape", "auto")
        assert_reduce_equal(to_bits(out), oracle.allreduce_sum_ref(bufs, dtype), dtype, what)
    assert mr.workspace_check() == 0


@pytest.mark.parametrize("block", range(6))
def test_random_gather_cases(block):
    rng = np.random.default_rng(9100 + block)
    for case in range(16):
        G = int(rng.choice([1, 2, 3, 4, 8]))
        W = G * int(rng.choice([1, 2, 3]))
        P = int(rng.integers(1, 140))
        splits = [int(x) for x in rng.choice([0, 1, 3, 8, 100, 1023, 4096, 20_001], size=P)]
        T = sum(splits)
        dtype = str(rng.choice(["bf16", "fp16", "fp32", "int32"]))
        entry = str(rng.choice(["rank_major", "shards", "into_tensor", "list", "sdma"]))
        if entry == "sdma" and mr.sdma_engines() == 0:
            entry = "rank_major"
        cu_below = int(rng.choice([0, 64, 8192, 1 << 20, 2 ** 32 - 1]))  # the SDMA gather's kernel part
        if entry in ("into_tensor", "list"):
            splits, P = [T], 1
        off = int(rng.integers(0, 5))
        what = f"block {block} case {case}: {entry} W={W} G={G} P={P} T={T} {dtype} off={off}" + (
            f" cu_below={cu_below}" if entry == "sdma" else "")
        print(f"[case] {what}", flush=True)
        src = workloads.gather_source(int(rng.integers(1 << 30)), W, T, dtype)
        shards = [src[r * T:(r + 1) * T] for r in range(W)]
        out = _view(np.zeros(W * T, dtype=src.dtype), dtype, off)
        if entry == "rank_major":
            mr.allgather_param_contig(_view(src, dtype, off), W, G, splits, out)
            want = oracle.allgather_param_contig_ref(src, W, G, splits)
        elif entry == "sdma":
            prev = mr.get_option("sdma_cu_below")
            mr.set_option("sdma_cu_below", cu_below)
            try:
                mr.allgather_param_contig_sdma(_view(src, dtype, off), W, G, splits, out)
            finally:
                mr.set_option("sdma_cu_below", prev)
            want = oracle.allgather_param_contig_ref(src, W, G, splits)
        elif entry == "shards":
            mr.allgather_param_contig_shards([_view(x, dtype, off + r % 3) for r, x in enumerate(shards)], G,
                                             splits, out)
            want = oracle.allgather_param_contig_shards_ref(shards, G, splits)
        elif entry == "into_tensor":
            mr.allgather_into_tensor([_view(x, dtype, r % 2) for r, x in enumerate(shards)], out)
            want = oracle.allgather_into_tensor_ref(shards)
        else:
            outs = [_view(np.zeros(T, dtype=src.dtype), dtype, (off + r) % 4) for r in range(W)]
            mr.allgather_list([_view(x, dtype, r % 2) for r, x in enumerate(shards)], outs)
            torch.cuda.synchronize()
            for o, w in zip(outs, oracle.allgather_list_ref(shards)):
                assert np.array_equal(to_bits(o), w), what
            continue
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), want), what
