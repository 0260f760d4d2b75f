"""mr_allreduce_sum_noalloc (two-shot workspace in the library's device array) against mr_allreduce_sum,
through the C ABI: bit-identical output on two calls in a row, the second with a smaller input, in both
modes and for bf16 and fp32; a rank buffer over the limit is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import all_gather_amd as mr
import workloads
from gpu_util import TORCH_DT, device, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["twoshot", "oneshot"])
def test_noalloc_matches_allreduce_sum(dtype, mode):
    W = 8
    es = 2 if dtype == "bf16" else 4
    # first call at the limit (wide XCD-local units: 16 KiB each), the second smaller and ragged (4 KiB
    # units), so the array holds the first call's stage and words
    sizes = [mr.NOALLOC_MAX_BYTES // es - (8 if es == 2 else 0), 1_000_003]
    for i, n in enumerate(sizes):
        print(f"[case] noalloc {mode} {dtype} call {i} n={n}", flush=True)
        bufs = [to_dev(b, dtype) for b in workloads.rank_buffers(80 + i, W, n, dtype, "normal")]
        want = torch.empty(n, dtype=TORCH_DT[dtype], device=device())
        got = torch.empty_like(want)
        got.view(torch.uint8).fill_(0xFF)
        mr.allreduce_sum(bufs, want, mode=mode)
        mr.allreduce_sum_noalloc(bufs, got, mode=mode)
        torch.cuda.synchronize()
        a, b = to_bits(got), to_bits(want)
        bad = np.flatnonzero(a != b)
        assert bad.size == 0, f"{mode} {dtype} call {i}: {bad.size} elements differ, first at {bad[:8].tolist()}"


def test_noalloc_refuses_rank_buffers_over_the_limit():
    n = mr.NOALLOC_MAX_BYTES // 2 + 8  # bf16, 16 bytes over
    bufs = [torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(2)]
    out = torch.empty_like(bufs[0])
    with pytest.raises(mr.MRError) as ei:
        mr.allreduce_sum_noalloc(bufs, out, mode="twoshot")
    assert ei.value.status == -4


def test_noalloc_graph_replays():
    """A captured allocation-free call (after one eager call on the device has set the array up), replayed
    three times with new inputs and eager work between the replays: every replay matches mr_allreduce_sum."""
    W, n = 8, 4_000_037
    s = torch.cuda.Stream()
    dbufs = [torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(W)]
    got = torch.empty(n, dtype=torch.bfloat16, device=device())
    want = torch.empty_like(got)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mr.allreduce_sum_noalloc(dbufs, got, mode="twoshot")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mr.allreduce_sum_noalloc(dbufs, got, mode="twoshot")
    for rep in range(3):
        print(f"[case] noalloc graph replay {rep}", flush=True)
        for d, b in zip(dbufs, workloads.rank_buffers(140 + rep, W, n, "bf16", "normal")):
            d.copy_(to_dev(b, "bf16"))
        got.view(torch.uint8).fill_(0xFF)
        mr.allreduce_sum(dbufs, want, mode="twoshot")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = np.flatnonzero(to_bits(got) != to_bits(want))
        assert bad.size == 0, f"replay {rep}: {bad.size} elements differ, first at {bad[:8].tolist()}"
    del g
