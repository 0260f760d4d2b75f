"""GPU parity of the reduce-scatter share and the shard-list all-gathers against the CPU oracle."""
import numpy as np
import pytest
import torch

import all_gather_amd as mr
import oracle
import workloads
from gpu_util import TORCH_DT, assert_reduce_equal, device, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,W,n", [("bf16", 8, 8_388_608), ("bf16", 3, 100_003), ("fp16", 5, 65_541),
                                       ("fp32", 16, 1_000_001), ("fp32", 8, 7)])
def test_reduce_scatter_every_rank(dtype, W, n):
    bufs = workloads.rank_buffers(70 + W, W, n, dtype, "normal")
    dbufs = [to_dev(b, dtype) for b in bufs]
    for rank in range(W):
        off, cnt = mr.reduce_scatter_chunk(n, W, dtype, rank)
        assert (off, off + cnt) == oracle.reduce_scatter_chunk(n, W, dtype, rank)
        if cnt == 0:
            continue
        out = torch.empty(cnt, dtype=TORCH_DT[dtype], device=device())
        mr.reduce_scatter_sum(dbufs, rank, out)
        torch.cuda.synchronize()
        assert_reduce_equal(to_bits(out), oracle.reduce_scatter_sum_ref(bufs, dtype, rank), dtype, f"rank {rank}")


def test_reduce_scatter_in_place_into_own_chunk():
    W, n = 4, 40_000
    bufs = workloads.rank_buffers(75, W, n, "bf16", "uniform")
    dbufs = [to_dev(b, "bf16") for b in bufs]
    rank = 2
    off, cnt = mr.reduce_scatter_chunk(n, W, "bf16", rank)
    out = dbufs[rank][off:off + cnt]
    mr.reduce_scatter_sum(dbufs, rank, out)
    torch.cuda.synchronize()
    assert_reduce_equal(to_bits(out), oracle.reduce_scatter_sum_ref(bufs, "bf16", rank), "bf16", "in place")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32", "int32"])
def test_allgather_into_tensor_and_list(dtype):
    W, T = 8, 3_000_017
    shards = [workloads.random_bits(76, r, T, dtype) for r in range(W)]
    dshards = [to_dev(x, dtype) for x in shards]
    out = torch.empty(W * T, dtype=TORCH_DT[dtype], device=device())
    mr.allgather_into_tensor(dshards, out)
    outs = [torch.empty(T, dtype=TORCH_DT[dtype], device=device()) for _ in range(W)]
    mr.allgather_list(dshards, outs)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_into_tensor_ref(shards))
    for o, want in zip(outs, oracle.allgather_list_ref(shards)):
        assert np.array_equal(to_bits(o), want)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_param_contig_from_shards_fsdp_splits(dtype):
    c = workloads.FSDP_SPLITS_W8_G4_P64
    W, G = c["W"], c["G"]
    splits = [int(x) for x in workloads.log_uniform_splits(c["seed"], c["P"])]
    T = sum(splits)
    shards = [workloads.random_bits(c["seed"], r, T, dtype) for r in range(W)]
    dshards = [to_dev(x, dtype) for x in shards]
    out = torch.empty(W * T, dtype=TORCH_DT[dtype], device=device())
    mr.allgather_param_contig_shards(dshards, G, splits, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_param_contig_shards_ref(shards, G, splits))
    # and it equals the rank-major path's output
    src = torch.cat(dshards)
    out2 = torch.empty_like(out)
    mr.allgather_param_contig(src, W, G, splits, out2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))


def test_param_contig_from_shards_ragged_and_many_params():
    W, G = 6, 2
    splits = [int(x) for x in workloads.log_uniform_splits(77, 200, lo=1, hi=5000, mult=1)] + [0, 3]
    T = sum(splits)
    shards = [workloads.random_bits(77, r, T, "bf16") for r in range(W)]
    dshards = [to_dev(x, "bf16") for x in shards]
    out = torch.empty(W * T, dtype=torch.bfloat16, device=device())
    mr.allgather_param_contig_shards(dshards, G, splits, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_param_contig_shards_ref(shards, G, splits))


def test_empty_inputs_are_no_ops():
    """n = 0 and T = 0 through every entry point: success, nothing written, the stream still works."""
    W = 8
    empty = [torch.empty(0, dtype=torch.bfloat16, device=device()) for _ in range(W)]
    out0 = torch.empty(0, dtype=torch.bfloat16, device=device())
    for mode in ("oneshot", "twoshot"):
        mr.allreduce_sum(empty, out0, mode=mode)
    mr.reduce_scatter_sum(empty, 3, out0)
    mr.allgather_into_tensor(empty, out0)
    mr.allgather_list(empty, [torch.empty(0, dtype=torch.bfloat16, device=device()) for _ in range(W)])
    mr.allgather_param_contig_shards(empty, 4, [0, 0, 0], out0)
    mr.allgather_param_contig(out0, W, 4, [0, 0], out0)
    # a sentinel output next to the empty calls stays untouched, and real work still runs afterwards
    sentinel = torch.full((64,), 7, dtype=torch.int32, device=device())
    torch.cuda.synchronize()
    assert bool((sentinel == 7).all())
    bufs = workloads.rank_buffers(303, W, 1000, "bf16", "uniform")
    out = torch.empty(1000, dtype=torch.bfloat16, device=device())
    mr.allreduce_sum([to_dev(b, "bf16") for b in bufs], out, mode="twoshot")
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allreduce_sum_ref(bufs, "bf16"))
    assert mr.workspace_check() == 0


def test_binding_rejects_mismatched_extents():
    """The library takes raw pointers and cannot see extents, so the binding refuses tensors whose sizes,
    dtypes or layout disagree with the call, before anything is enqueued."""
    d, bf = device(), torch.bfloat16
    W = 4
    sentinel = torch.full((64,), 7, dtype=torch.int32, device=d)
    bufs = [torch.zeros(100, dtype=bf, device=d) for _ in range(W)]
    out = torch.zeros(100, dtype=bf, device=d)
    short = torch.zeros(99, dtype=bf, device=d)
    strided = torch.zeros(200, dtype=bf, device=d)[::2]
    bad_calls = {
        "allreduce short rank buffer": lambda: mr.prepare_allreduce(bufs[:-1] + [short], out),
        "allreduce short out": lambda: mr.allreduce_sum(bufs, short),
        "allreduce dtype": lambda: mr.allreduce_sum(bufs, out.float()),
        "allreduce strided": lambda: mr.allreduce_sum(bufs[:-1] + [strided], out),
        "reduce-scatter out size": lambda: mr.prepare_reduce_scatter(bufs, 0, short),
        "reduce-scatter short rank buffer": lambda: mr.reduce_scatter_sum(bufs[:-1] + [short], 0, out[:32]),
    }
    src = torch.zeros(W * 10, dtype=bf, device=d)
    shards = [torch.zeros(10, dtype=bf, device=d) for _ in range(W)]
    full = torch.empty(W * 10, dtype=bf, device=d)
    bad_calls.update({
        "param-contig splits != T": lambda: mr.prepare_allgather_param_contig(src, W, 2, [4, 5], full),
        "param-contig short out": lambda: mr.allgather_param_contig(src, W, 2, [4, 6], full[:-1]),
        "param-contig negative split": lambda: mr.allgather_param_contig(src, W, 2, [-1, 11], full),
        "param-contig no splits": lambda: mr.allgather_param_contig(src, W, 2, [], full),
        "param-contig W=0": lambda: mr.allgather_param_contig(src, 0, 1, [10], full),
        "shards splits != T": lambda: mr.allgather_param_contig_shards(shards, 2, [4, 5], full),
        "shards short out": lambda: mr.prepare_allgather_shards(shards, full[:-1], 2, [4, 6]),
        "into-tensor short out": lambda: mr.allgather_into_tensor(shards, full[:-1]),
        "into-tensor short shard": lambda: mr.allgather_into_tensor(shards[:-1] + [shards[0][:9]], full),
        "into-tensor no shards": lambda: mr.allgather_into_tensor([], full),
        "list short output": lambda: mr.allgather_list(shards, [torch.empty(9, dtype=bf, device=d)] * W),
        "list output count": lambda: mr.allgather_list(shards, [full[:10]] * (W - 1)),
    })
    for what, call in bad_calls.items():
        print(f"[case] binding check: {what}", flush=True)
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    assert bool((sentinel == 7).all())
    assert bool((out == 0).all())


def test_gathers_at_large_rank_counts():
    """Rank counts far above 8: a rank-major scatter with W = 1000 (125 node-blocks of G = 8), and the
    shard gathers at MR_MAX_TABLE_W = 64 ranks (param-contiguous, rank-major and list outputs), every element
    against the oracle; 65 shards are refused with nothing written."""
    import ctypes

    W, G = 1000, 8
    splits = [3, 17, 64, 0, 129, 8]
    T = sum(splits)
    print(f"[case] rank-major scatter W={W} G={G} T={T}", flush=True)
    src = workloads.gather_source(780, W, T, "bf16")
    out = torch.empty(W * T, dtype=torch.bfloat16, device=device())
    mr.allgather_param_contig(to_dev(src, "bf16"), W, G, splits, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_param_contig_ref(src, W, G, splits))

    W, G = 64, 16
    splits = [7, 4096, 33, 1000]
    T = sum(splits)
    print(f"[case] shard gathers W={W} G={G} T={T}", flush=True)
    shards = [workloads.random_bits(781, r, T, "fp32") for r in range(W)]
    dshards = [to_dev(x, "fp32") for x in shards]
    out = torch.empty(W * T, dtype=torch.float32, device=device())
    mr.allgather_param_contig_shards(dshards, G, splits, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_param_contig_shards_ref(shards, G, splits))
    mr.allgather_into_tensor(dshards, out)
    outs = [torch.empty(T, dtype=torch.float32, device=device()) for _ in range(W)]
    mr.allgather_list(dshards, outs)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), oracle.allgather_into_tensor_ref(shards))
    for o, want in zip(outs, oracle.allgather_list_ref(shards)):
        assert np.array_equal(to_bits(o), want)

    extra = dshards + [dshards[0].clone()]
    big = torch.zeros(65 * T, dtype=torch.float32, device=device())
    ptrs = (ctypes.c_void_p * 65)(*[x.data_ptr() for x in extra])
    rc = mr.lib().mr_allgather_into_tensor(ptrs, 65, T, mr.DTYPE_CODE["fp32"], big.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == -1, rc  # MR_ERR_INVALID_ARG
    assert int(torch.count_nonzero(big)) == 0
