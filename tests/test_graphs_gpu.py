"""The entry points captured into a HIP graph replay correctly, again and again.

Each op is captured once on a stream that already ran it (so the two-shot workspace exists and no
allocation happens under capture), then the graph is replayed several times with fresh inputs copied
into the captured buffers between replays, eager work and synchronisations in between; every replay is
checked against the CPU oracle.  The two-shot barrier words and flags re-arm themselves inside each
launch, which is what lets a captured two-shot replay without host-side resets."""
import numpy as np
import pytest
import torch

import all_gather_amd as mr
import oracle
import workloads
from gpu_util import assert_reduce_equal, device, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _capture(fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


@pytest.mark.parametrize("mode", ["oneshot", "twoshot", "twoshot:tile", "twoshot:chunk", "twoshot:grid", "twoshot:last"])
def test_allreduce_graph_replays(mode):
    W, n = 8, 2_000_003
    kind, _, sync = mode.partition(":")
    s = torch.cuda.Stream()
    dbufs = [torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(W)]
    out = torch.empty(n, dtype=torch.bfloat16, device=device())
    if sync:
        mr.set_option("twoshot_sync", sync)
    try:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            mr.allreduce_sum(dbufs, out, mode=kind)  # warm: creates this stream's workspace
        torch.cuda.synchronize()
        g = _capture(lambda: mr.allreduce_sum(dbufs, out, mode=kind), s)
        for rep in range(5):
            bufs = workloads.rank_buffers(80 + rep, W, n, "bf16", "normal")
            for d, b in zip(dbufs, bufs):
                d.copy_(to_dev(b, "bf16"))
            out.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_reduce_equal(to_bits(out), oracle.allreduce_sum_ref(bufs, "bf16"), "bf16", f"{mode} replay {rep}")
        if kind == "twoshot":
            assert mr.workspace_check(s) == 0
    finally:
        mr.set_option("twoshot_sync", "auto")


def test_gathers_and_reduce_scatter_graph_replays():
    W, G = 8, 4
    splits = [8, 4096, 100_000, 24, 777_776]
    T = sum(splits)
    s = torch.cuda.Stream()
    src = torch.empty(W * T, dtype=torch.float16, device=device())
    shards = [torch.empty(T, dtype=torch.float16, device=device()) for _ in range(W)]
    out_pc = torch.empty_like(src)
    out_sh = torch.empty_like(src)
    outs_list = [torch.empty(T, dtype=torch.float16, device=device()) for _ in range(W)]
    rs_bufs = [torch.empty(T, dtype=torch.float16, device=device()) for _ in range(W)]
    off, cnt = mr.reduce_scatter_chunk(T, W, "fp16", 5)
    rs_out = torch.empty(cnt, dtype=torch.float16, device=device())

    def ops():
        mr.allgather_param_contig(src, W, G, splits, out_pc)
        mr.allgather_param_contig_shards(shards, G, splits, out_sh)
        mr.allgather_list(shards, outs_list)
        mr.reduce_scatter_sum(rs_bufs, 5, rs_out)

    g = _capture(ops, s)
    for rep in range(4):
        hsrc = workloads.gather_source(90 + rep, W, T, "fp16")
        hsh = [workloads.random_bits(95 + rep, r, T, "fp16") for r in range(W)]
        hrs = workloads.rank_buffers(99 + rep, W, T, "fp16", "uniform")
        src.copy_(to_dev(hsrc, "fp16"))
        for d, h in zip(shards, hsh):
            d.copy_(to_dev(h, "fp16"))
        for d, h in zip(rs_bufs, hrs):
            d.copy_(to_dev(h, "fp16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out_pc), oracle.allgather_param_contig_ref(hsrc, W, G, splits)), rep
        assert np.array_equal(to_bits(out_sh), oracle.allgather_param_contig_shards_ref(hsh, G, splits)), rep
        for o, h in zip(outs_list, hsh):
            assert np.array_equal(to_bits(o), h), rep
        assert_reduce_equal(to_bits(rs_out), oracle.reduce_scatter_sum_ref(hrs, "fp16", 5), "fp16", f"rs {rep}")


def test_twoshot_graph_replays_after_the_workspace_grew():
    """A graph captured with the stream's first (small) workspace is replayed after an eager call on the
    same stream grew the workspace: the replaced buffer stays alive, so the replay still reads and
    writes valid memory and gives the oracle's bits."""
    W, n_small, n_big = 8, 300_001, 6_000_017
    s = torch.cuda.Stream()
    small = [torch.empty(n_small, dtype=torch.bfloat16, device=device()) for _ in range(W)]
    out_small = torch.empty(n_small, dtype=torch.bfloat16, device=device())
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mr.allreduce_sum(small, out_small, mode="twoshot")  # first use: allocates the small workspace
    torch.cuda.synchronize()
    g = _capture(lambda: mr.allreduce_sum(small, out_small, mode="twoshot"), s)
    big_host = workloads.rank_buffers(86, W, n_big, "bf16", "normal")
    big = [to_dev(b, "bf16") for b in big_host]
    out_big = torch.empty(n_big, dtype=torch.bfloat16, device=device())
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mr.allreduce_sum(big, out_big, mode="twoshot")  # grows this stream's workspace
    torch.cuda.synchronize()
    assert_reduce_equal(to_bits(out_big), oracle.allreduce_sum_ref(big_host, "bf16"), "bf16", "grown call")
    for rep in range(3):
        bufs = workloads.rank_buffers(87 + rep, W, n_small, "bf16", "normal")
        for d, b in zip(small, bufs):
            d.copy_(to_dev(b, "bf16"))
        out_small.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_reduce_equal(to_bits(out_small), oracle.allreduce_sum_ref(bufs, "bf16"), "bf16", f"replay {rep}")
    assert mr.workspace_check(s) == 0
    del g
    mr.set_workspace(None, stream=s)  # frees the live and the replaced buffers of this stream


@pytest.mark.parametrize("mode", ["twoshot", "twoshot:tile", "twoshot:last", "twoshot:chunk"])
def test_graphs_captured_on_one_stream_replay_together(mode):
    """Two two-shot calls captured into two graphs on the same capture stream (torch.cuda.graph's default
    shares one), replayed at the same time on two different streams with different inputs.  Each
    capture has its own workspace, so the replays cannot hand each other's workgroups tickets, flags or
    stage bytes; every replay must match the oracle, and the capture workspaces' error words (read by
    mr_workspace_check on the capture stream) must stay clear."""
    W, n = 8, 8_388_608 + 16
    kind, _, sync = mode.partition(":")
    cap = torch.cuda.Stream()
    sets = [[torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(W)] for _ in range(2)]
    outs = [torch.empty(n, dtype=torch.bfloat16, device=device()) for _ in range(2)]
    if sync:
        mr.set_option("twoshot_sync", sync)
    try:
        graphs = [_capture(lambda k=k: mr.allreduce_sum(sets[k], outs[k], mode=kind), cap) for k in range(2)]
        run = [torch.cuda.Stream(), torch.cuda.Stream()]
        for rep in range(4):
            wants = []
            for k in range(2):
                bufs = workloads.rank_buffers(120 + 2 * rep + k, W, n, "bf16", "normal")
                for d, b in zip(sets[k], bufs):
                    d.copy_(to_dev(b, "bf16"))
                outs[k].fill_(0)
                wants.append(oracle.allreduce_sum_ref(bufs, "bf16"))
            torch.cuda.synchronize()
            for k in range(2):
                with torch.cuda.stream(run[k]):
                    graphs[k].replay()
            torch.cuda.synchronize()
            for k in range(2):
                assert_reduce_equal(to_bits(outs[k]), wants[k], "bf16", f"{mode} rep {rep} graph {k}")
        assert mr.workspace_check(cap) == 0
        del graphs
        torch.cuda.synchronize()
        mr.set_workspace(None, cap)  # frees the capture workspaces of the stream
    finally:
        mr.set_option("twoshot_sync", "auto")


_PIPE_CAPTURE_CHILD = r"""
import torch
import all_gather_amd as mr
import oracle
import workloads
from gpu_util import assert_reduce_equal, to_bits, to_dev
W, n = 8, 8_388_608 + 5
dbufs = [torch.empty(n, dtype=torch.bfloat16, device="cuda:0") for _ in range(W)]
out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
torch.cuda.synchronize()
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):
    mr.allreduce_sum(dbufs, out, mode="oneshot")
for rep in range(3):
    bufs = workloads.rank_buffers(140 + rep, W, n, "bf16", "normal")
    want = oracle.allreduce_sum_ref(bufs, "bf16")
    for d, b in zip(dbufs, bufs):
        d.copy_(to_dev(b, "bf16"))
    out.fill_(0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert_reduce_equal(to_bits(out), want, "bf16", f"replay {rep}")
    out.fill_(0)
    mr.allreduce_sum(dbufs, out, mode="oneshot")
    torch.cuda.synchronize()
    assert_reduce_equal(to_bits(out), want, "bf16", f"eager call after replay {rep}")
print("replays ok", flush=True)
"""


def test_pipelined_oneshot_first_called_under_capture():
    """A fresh process whose first pipelined one-shot (W=8 bf16, 16 MiB per rank) is made under HIP graph
    capture, so the kernel's resident-grid lookup runs during the capture; the graph is replayed three
    times with new inputs, an eager call after each, and every result is checked against the oracle.
    The launch trace confirms the pipelined shape was chosen."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MR_TRACE="1", PYTHONPATH=os.pathsep.join([root, os.path.join(root, "tests")]))
    print("[case] pipelined one-shot first called under capture (child process, MR_TRACE=1)", flush=True)
    r = subprocess.run([sys.executable, "-c", _PIPE_CAPTURE_CHILD], cwd=root, env=env, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "replays ok" in r.stdout
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[mr] allreduce oneshot")]
    assert lines and all("shape=4" in ln for ln in lines), lines
