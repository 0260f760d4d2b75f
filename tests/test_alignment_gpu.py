"""Any alignment: rank buffers, outputs and shards at odd byte offsets (off the element grid) and at
mixed 16-byte phases, through the C ABI with raw pointers into byte buffers, against the CPU oracle.

Off-grid pointers take byte accesses only (reduce: one element per lane, each element read and written
one byte at a time; gathers: planned and copied in bytes); element-aligned pointers in different 16-byte
phases take the realigned 16-byte path.  Reduce results are compared bit for bit (NaN by NaN-ness), the
gathers bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import all_gather_amd as mr
import oracle
import workloads
from gpu_util import assert_reduce_equal, device

pytestmark = pytest.mark.gpu

NPBITS = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32, "int32": np.uint32}


class ByteBuf:
    """A device byte buffer holding `nbytes` at byte offset `off` (plus slack on both sides)."""

    def __init__(self, nbytes, off):
        self.t = torch.empty(nbytes + 64, dtype=torch.uint8, device=device())
        self.t.fill_(0xA5)
        self.off, self.n = off, nbytes

    @property
    def ptr(self):
        return self.t.data_ptr() + self.off

    def put(self, bits):
        raw = np.ascontiguousarray(bits).view(np.uint8)
        self.t[self.off:self.off + raw.size].copy_(torch.from_numpy(raw.copy()))

    def get(self, dtype):
        raw = self.t[self.off:self.off + self.n].cpu().numpy().copy()
        return raw.view(NPBITS[dtype])


def _stream():
    return torch.cuda.current_stream().cuda_stream or None


def _reduce(bufs_bits, dtype, offs, out_off, mode, sync="auto"):
    W, n = len(bufs_bits), len(bufs_bits[0])
    es = np.dtype(NPBITS[dtype]).itemsize
    ins = []
    for b, o in zip(bufs_bits, offs):
        bb = ByteBuf(n * es, o)
        bb.put(b)
        ins.append(bb)
    out = ByteBuf(n * es, out_off)
    ptrs = (ctypes.c_void_p * W)(*[b.ptr for b in ins])
    mr.set_option("twoshot_sync", sync)
    try:
        st = mr.lib().mr_allreduce_sum(ptrs, W, n, mr.DTYPE_CODE[dtype], out.ptr, mr.MODE_CODE[mode], _stream())
    finally:
        mr.set_option("twoshot_sync", "auto")
    assert st == 0, mr.STATUS.get(st, st)
    torch.cuda.synchronize()
    return out.get(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["oneshot", "twoshot", "twoshot:tile", "twoshot:chunk", "twoshot:grid"])
def test_reduce_at_odd_byte_offsets(dtype, mode):
    kind, _, sync = mode.partition(":")
    rng = np.random.default_rng(5)
    for W, n in ((1, 7), (3, 1), (3, 70_001), (8, 300_003)):
        bufs = workloads.rank_buffers(40 + W, W, n, dtype, "normal")
        want = oracle.allreduce_sum_ref(bufs, dtype)
        offs = [int(x) for x in rng.integers(0, 16, size=W)]
        offs[0] |= 1  # at least one input off the element grid
        for out_off in (3, 8):
            print(f"[case] odd offsets {dtype} {mode} W={W} n={n} offs={offs} out+{out_off}", flush=True)
            got = _reduce(bufs, dtype, offs, out_off, kind, sync or "auto")
            assert_reduce_equal(got, want, dtype, f"{mode} W={W} n={n} offs={offs} out+{out_off}")
    if kind == "twoshot":
        assert mr.workspace_check() == 0


@pytest.mark.parametrize("mode", ["oneshot", "twoshot", "twoshot:tile", "twoshot:chunk"])
def test_reduce_at_odd_byte_offsets_large(mode):
    """The byte path at 8 MiB per rank buffer (its two-shot plan needs a flag per 1024-element tile of
    every chunk, so this also checks the workspace sizing), outputs sampled against the oracle."""
    kind, _, sync = mode.partition(":")
    W, n = 8, 4_194_304 + 5
    bufs = workloads.rank_buffers(47, W, n, "bf16", "uniform")
    idx = np.linspace(0, n - 1, 1 << 16).astype(np.int64)
    want = oracle.allreduce_sum_ref([b[idx] for b in bufs], "bf16")
    offs = [1, 2, 7, 0, 4, 9, 15, 3]
    print(f"[case] odd offsets large {mode} W={W} n={n}", flush=True)
    got = _reduce(bufs, "bf16", offs, 5, kind, sync or "auto")
    assert_reduce_equal(got[idx], want, "bf16", f"odd offsets large {mode}")
    if kind == "twoshot":
        assert mr.workspace_check() == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_reduce_mixed_phases_realigned(dtype):
    """Element-aligned pointers, every rank at its own 16-byte phase (the realigned 16-byte path), in
    both modes, at sizes with partial tiles and a ragged tail."""
    es = np.dtype(NPBITS[dtype]).itemsize
    for W, n in ((2, 1_000), (8, 1_000_003), (16, 65_541), (8, 8_388_608 + 24)):
        bufs = workloads.rank_buffers(50 + W, W, n, dtype, "uniform")
        want = oracle.allreduce_sum_ref(bufs, dtype)
        offs = [(r * es * 3) % 16 for r in range(W)]
        for out_off in (0, 16 - es):
            for mode in ("oneshot", "twoshot"):
                print(f"[case] mixed phases {dtype} {mode} W={W} n={n} out+{out_off}", flush=True)
                got = _reduce(bufs, dtype, offs, out_off, mode)
                assert_reduce_equal(got, want, dtype, f"mixed {mode} W={W} n={n} out+{out_off}")
    assert mr.workspace_check() == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_gathers_at_odd_byte_offsets(dtype):
    es = np.dtype(NPBITS[dtype]).itemsize
    W, G = 8, 4
    splits = [0, 1, 7, 8, 9, 4095, 4096, 4097, 16385, 3, 100_001]
    T = sum(splits)
    src_bits = workloads.gather_source(70, W, T, dtype)
    want = oracle.allgather_param_contig_ref(src_bits, W, G, splits)
    sp = (ctypes.c_uint64 * len(splits))(*splits)
    L = mr.lib()
    for so, oo in ((1, 0), (0, 3), (5, 11), (es, 1)):
        print(f"[case] gather {dtype} src+{so} out+{oo}", flush=True)
        src = ByteBuf(W * T * es, so)
        src.put(src_bits)
        out = ByteBuf(W * T * es, oo)
        assert L.mr_allgather_param_contig(src.ptr, W, G, sp, len(splits), mr.DTYPE_CODE[dtype], out.ptr, _stream()) == 0
        torch.cuda.synchronize()
        assert np.array_equal(out.get(dtype), want), f"param_contig src+{so} out+{oo}"
        prev = mr.get_option("sdma_cu_below")
        for cu_below in (0, 256 << 10):  # every piece on the engines; the smaller parameters on the kernel
            mr.set_option("sdma_cu_below", cu_below)
            out2 = ByteBuf(W * T * es, oo)
            try:
                assert L.mr_allgather_param_contig_sdma(src.ptr, W, G, sp, len(splits), mr.DTYPE_CODE[dtype],
                                                        out2.ptr, _stream()) == 0
            finally:
                mr.set_option("sdma_cu_below", prev)
            assert np.array_equal(out2.get(dtype), want), f"sdma src+{so} out+{oo} cu_below={cu_below}"
    # from separate shards at odd offsets: param-contiguous, rank-major and list outputs
    shards_bits = [src_bits[r * T:(r + 1) * T] for r in range(W)]
    shards = []
    for r in range(W):
        b = ByteBuf(T * es, (3 * r + 1) % 16)
        b.put(shards_bits[r])
        shards.append(b)
    sptr = (ctypes.c_void_p * W)(*[b.ptr for b in shards])
    out = ByteBuf(W * T * es, 7)
    assert L.mr_allgather_param_contig_shards(sptr, W, G, sp, len(splits), mr.DTYPE_CODE[dtype], out.ptr, _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.get(dtype), want), "param_contig_shards at odd offsets"
    out = ByteBuf(W * T * es, 9)
    assert L.mr_allgather_into_tensor(sptr, W, T, mr.DTYPE_CODE[dtype], out.ptr, _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.get(dtype), src_bits), "all_gather_into_tensor at odd offsets"
    outs = [ByteBuf(T * es, (5 * r + 2) % 16) for r in range(W)]
    optr = (ctypes.c_void_p * W)(*[o.ptr for o in outs])
    assert L.mr_allgather_list(sptr, W, T, mr.DTYPE_CODE[dtype], optr, _stream()) == 0
    torch.cuda.synchronize()
    for r in range(W):
        assert np.array_equal(outs[r].get(dtype), shards_bits[r]), f"list output rank {r}"
