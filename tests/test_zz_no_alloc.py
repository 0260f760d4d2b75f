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
    # first call at the limit (16 MiB bf16 takes the XCD-local units, 32 MiB fp32 too), the second smaller
    # and ragged (the last-arriver hand-off), so the array holds the first call's stage and words
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
