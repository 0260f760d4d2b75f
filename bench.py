"""Benchmark of the W-way sum-reduce and the param-contiguous scatter on one MI355X.

Headline: achieved HBM GB/s (and fraction of the 8.0e12 B/s peak) of the one-shot W=8 bf16 sum-reduce
at 16 MiB per rank buffer (n = 8,388,608), bytes per call W*n*s read + n*s written = 150,994,944.

A step is one mr_allreduce_sum call over one batch of W rank buffers.  The inputs are resident in HBM
before timing starts and the caches do not hold them: the steps rotate over several disjoint buffer
sets whose total (>= 864 MiB) is far beyond the 256 MB last-level cache, so every step streams from
HBM.  Timing: HIP events on the stream the kernels are launched on, around exactly K steps, with a
device synchronisation on both sides.  The same run also times two-shot (both byte counts), the
param-contiguous scatter on the FSDP-style split workload, the cache-resident one-shot, a size sweep of
256 KiB .. 256 MiB per rank, and the CPU oracle on the host cores; one JSON line goes to stdout,
progress to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E, 8.0e12 B/s
PROFILE_PMC = os.path.join(ROOT, "profiles", "oneshot_pipe_bf16_w8_16MiB_pmc.txt")
# the reduce kernels and the header that picks their launch shapes
KERNEL_SRC = (os.path.join(ROOT, "all_gather_amd", "csrc", "reduce_kernels.hip"),
              os.path.join(ROOT, "all_gather_amd", "csrc", "mr_internal.h"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(paths=None) -> str:
    """sha256 (first 16 hex digits) of the reduce kernels' source (or of `paths`) with comments and blank
    space taken out, so that a change to the code, not to its comments, marks the committed counters as
    stale."""
    h = hashlib.sha256()
    for path in paths or KERNEL_SRC:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(algo_bytes: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; None otherwise."""
    if not os.path.exists(PROFILE_PMC):
        return None, "no counter summary"
    txt = open(PROFILE_PMC).read()
    m = re.search(r"^kernel_source_sha256_16:\s*(\S+)", txt, re.M)
    t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", txt, re.M)
    if not m or not t:
        return None, "counter summary incomplete"
    if m.group(1) != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return int(t.group(1)), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def time_steps(calls, K, W_, stream):
    import torch

    for i in range(W_):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)  # ms


def _overlap(torch, stream, side, call, R, gemm, G):
    """Time R calls alone on `stream`, G GEMMs alone on `side`, then both at once (the GEMM window is
    opened first).  Returns seconds per call and per GEMM, alone and together.  A synchronous call (the
    copy-engine gather returns only when its copies are complete) is timed by the same events: the
    second is recorded after the last call has returned."""
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def op_run():
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(R):
            call()
        e1.record(stream)
        return e0, e1

    def gemm_run():
        e0, e1 = ev(), ev()
        with torch.cuda.stream(side):
            e0.record(side)
            for _ in range(G):
                gemm()
            e1.record(side)
        return e0, e1

    call(); gemm(); torch.cuda.synchronize()
    r0, r1 = op_run(); torch.cuda.synchronize()
    t_op = r0.elapsed_time(r1) / R * 1e-3
    g0, g1 = gemm_run(); torch.cuda.synchronize()
    t_gemm = g0.elapsed_time(g1) / G * 1e-3
    side.wait_stream(stream)
    g0, g1 = gemm_run()
    r0, r1 = op_run()
    torch.cuda.synchronize()
    return t_op, t_gemm, r0.elapsed_time(r1) / R * 1e-3, g0.elapsed_time(g1) / G * 1e-3


def copy_ceiling(mr, torch, dev, stream, reps=40):
    """Secondary ceiling: GB/s (read + write bytes) of a plain 256 MiB device-to-device copy made by this
    library's gather kernel (all_gather_into_tensor of one shard: 16-byte non-temporal loads and
    stores), timed the same way on the same GPU.  The runtime's own blit copy is slower (about
    5.3 TB/s), so it would understate the ceiling."""
    a = torch.empty(1 << 26, dtype=torch.int32, device=dev).fill_(1)
    b = torch.empty_like(a)
    call = mr.prepare_allgather_shards([a], b)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    del a, b
    torch.cuda.empty_cache()
    return 2 * (1 << 28) / t / 1e9


def stream_mix_ceiling(mr, torch, sets, n, s, stream, K, warmup):
    """Same-run ceilings of the one-shot's access pattern on its own buffer sets: the library's probe
    kernel (mrx_stream_mix, not part of the mr.h ABI) streams the 8 rank buffers and writes the XOR of
    them to out with the one-shot's lane layout, on the one-shot's schedule (a persistent grid of
    resident workgroups, each issuing a tile's loads before storing the previous tile's XOR), once
    more with one tile per workgroup, and once without the write.  Returns GB/s counting every byte
    moved (9 and 8 times the per-rank bytes)."""
    import ctypes

    L = mr.lib()
    f = L.mrx_stream_mix
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_void_p]
    res = {}
    for name, write in (("reads8_write1_pipelined", 2), ("reads8_write1", 1), ("reads8_only", 0)):
        calls = []
        for bufs, out in sets:
            ptrs = (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
            args = (ptrs, len(bufs), out.data_ptr(), n * s, write, stream.cuda_stream or None)
            calls.append(lambda a=args, keep=ptrs: _probe_ok(f(*a)))
        ms = time_steps(calls, K, warmup, stream)
        t = ms / K * 1e-3
        nbytes = (len(sets[0][0]) + (1 if write else 0)) * n * s
        res[name] = {"us": t * 1e6, "GBps": nbytes / t / 1e9, "bytes": nbytes}
    return res


def _same_bytes_copy(mr, prepared, K, warmup, stream, nbytes, gbs):
    """A plain copy of exactly the bytes a prepared gather moves, on its own source and output buffers,
    made by the same kernel (all_gather_into_tensor of one shard) and timed the same way."""
    calls = [mr.prepare_allgather_shards([c.keepalive[1]], c.keepalive[2]) for c in prepared]
    ms = time_steps(calls, K, max(2, warmup // 10), stream)
    t = ms / K * 1e-3
    copy = nbytes / t / 1e9
    return {"copy_same_bytes_us": t * 1e6, "copy_same_bytes_GBps": copy, "frac_of_copy_same_bytes": gbs / copy}


def _with_option(mr, name, value, call):
    """`call` made with option `name` set to `value`, and the option's previous value restored after it."""
    def run():
        prev = mr.get_option(name)
        mr.set_option(name, value)
        try:
            call()
        finally:
            mr.set_option(name, prev)
    return run


def _probe_ok(rc):
    if rc != 0:
        raise RuntimeError(f"mrx_stream_mix failed: {rc}")


def contention_leg(mr, torch, dev, stream, gather_sets, gather_bytes, sdma_legs=()):
    """Ops alone and beside bf16 8192^3 GEMMs on a second stream (default priority): W=8 fp32 one-shot
    and two-shot at 512 MiB per rank, and the param-contiguous scatter at the FSDP-style splits.  GB/s of the op and
    TFLOP/s of the GEMM, alone and together."""
    W, n = 8, 134_217_728
    algo = (W + 1) * n * 4
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    bufs = [torch.rand(n, device=dev, generator=g) * 2 - 1 for _ in range(W)]
    out = torch.empty(n, dtype=torch.float32, device=dev)
    a = (torch.randn(8192, 8192, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(8192, 8192, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    flop = 2.0 * 8192 ** 3
    gemm = lambda: torch.matmul(a, b, out=c)
    res = {"note": "op window overlaps the GEMM stream; GEMM figure averaged over its own window"}
    legs = [("reduce_oneshot_fp32_512MiB", mr.prepare_allreduce(bufs, out, "oneshot"), algo, 20, 24),
            ("reduce_twoshot_fp32_512MiB", mr.prepare_allreduce(bufs, out, "twoshot"), algo, 20, 24),
            ("scatter_fsdp_splits_bf16", gather_sets[0], gather_bytes, 100, 24)]
    for name, call in sdma_legs:
        legs.append((name, call, gather_bytes, 12, 24))
    for name, call, nbytes, R, G in legs:
        t_op, t_gemm, t_op_c, t_gemm_c = _overlap(torch, stream, side, call, R, gemm, G)
        r = {"op_GBps_alone": nbytes / t_op / 1e9, "op_GBps_with_gemm": nbytes / t_op_c / 1e9,
             "op_us_alone": t_op * 1e6, "op_us_with_gemm": t_op_c * 1e6, "bytes_per_op": nbytes,
             "gemm_TFLOPs_alone": flop / t_gemm / 1e12, "gemm_TFLOPs_with_op": flop / t_gemm_c / 1e12}
        res[name] = r
        log(f"[bench] contention {name}: {r['op_us_alone']:.1f} us ({r['op_GBps_alone']:.0f} GB/s) alone, "
            f"{r['op_us_with_gemm']:.1f} us ({r['op_GBps_with_gemm']:.0f} GB/s) beside GEMM; GEMM "
            f"{r['gemm_TFLOPs_alone']:.0f} TFLOP/s alone, {r['gemm_TFLOPs_with_op']:.0f} beside")
    del bufs, out, a, b, c
    torch.cuda.empty_cache()
    return res


SWEEP_KIB = (256, 1024, 4096, 16384, 65536, 262144)  # bytes per rank buffer, 256 KiB .. 256 MiB
SWEEP_MODES = ("oneshot", "twoshot", "twoshot:grid")  # two-shot under its default hand-off and the grid barrier


def sweep_leg(mr, torch, dev):
    """W=8 sum-reduce over per-rank sizes 256 KiB .. 256 MiB, bf16 and fp32, uniform[-1,1) inputs:
    one-shot, and two-shot under its default (size-chosen) hand-off and with the grid barrier.  Each size rotates over
    enough disjoint buffer sets to keep >= 512 MiB in flight (twice the last-level cache); sizes up to
    1 MiB per rank are timed as HIP-graph replays so that launch cost does not hide the kernel."""
    W = 8
    side = torch.cuda.Stream()
    rows = []
    for dtype, tdt, s in (("bf16", torch.bfloat16, 2), ("fp32", torch.float32, 4)):
        for kib in SWEEP_KIB:
            n = kib * 1024 // s
            per_set = (W + 1) * n * s
            S = max(1, min(256, -(-(512 << 20) // per_set)))
            g = torch.Generator(device=dev)
            g.manual_seed(3000 + kib)
            inp = (torch.rand(S * W * n, device=dev, generator=g) * 2 - 1).to(tdt)
            outs = torch.empty(S * n, dtype=tdt, device=dev)
            sets = [([inp[(k * W + r) * n:(k * W + r + 1) * n] for r in range(W)], outs[k * n:(k + 1) * n])
                    for k in range(S)]
            launches = max(20, min(2000, (4 << 30) // per_set))
            use_graph = kib <= 1024
            row = {"dtype": dtype, "KiB_per_rank": kib, "n": n, "bytes": per_set, "buffer_sets": S,
                   "timing": "hip graph replay" if use_graph else "eager launches"}
            for mode in SWEEP_MODES:
                kind, _, sync = mode.partition(":")
                mr.set_option("twoshot_sync", sync or "auto")
                calls = [mr.prepare_allreduce(b, o, kind, stream=side) for b, o in sets]
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    for c in calls:  # warm: also sizes this stream's two-shot workspace
                        c()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                if use_graph:
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph, stream=side):
                        for c in calls:
                            c()
                    reps = max(1, launches // S)
                    with torch.cuda.stream(side):  # replay() launches on the current stream
                        graph.replay()
                        torch.cuda.synchronize()
                        e0.record(side)
                        for _ in range(reps):
                            graph.replay()
                        e1.record(side)
                    torch.cuda.synchronize()
                    count = reps * S
                    del graph
                else:
                    e0.record(side)
                    for i in range(launches):
                        calls[i % S]()
                    e1.record(side)
                    torch.cuda.synchronize()
                    count = launches
                t = e0.elapsed_time(e1) / count * 1e-3
                row[mode] = {"us": round(t * 1e6, 3), "GBps": round(per_set / t / 1e9, 1),
                             "frac": round(per_set / t / 1e9 / PEAK_GBS, 4), "launches": count}
                if kind == "twoshot":
                    row[mode]["GBps_actual_bytes"] = round((W + 3) * n * s / t / 1e9, 1)
                    row[mode]["barrier_error_word"] = mr.workspace_check(side)
            mr.set_option("twoshot_sync", "auto")
            rows.append(row)
            log(f"[bench] sweep {dtype} {kib:>6d} KiB/rank ({row['timing']}): " + ", ".join(
                f"{m} {row[m]['us']:.2f} us {row[m]['GBps']:.0f} GB/s" for m in SWEEP_MODES))
            del sets, inp, outs
            torch.cuda.empty_cache()
    return rows


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=6, help="disjoint buffer sets rotated through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip the secondary paths")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 256 KiB .. 256 MiB size sweep")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (reference for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the reduce and scatter kernels run on a single MI355X "
              "(the rank buffers are W separate allocations on it). --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import all_gather_amd as mr
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    mr.lib()

    c = workloads.W8_BF16_16MIB
    W, n, dtype = c["W"], c["n"], c["dtype"]
    s = 2
    algo = (W + 1) * n * s  # 150,994,944
    log(f"[bench] inputs: W={W} n={n} {dtype} N(0,1), {args.sets} buffer sets")
    host = workloads.rank_buffers(c["seed"], W, n, dtype, c["dist"])
    base = [torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in host]
    sets = []
    for k in range(args.sets):
        bufs = [b.clone() for b in base]
        out = torch.empty(n, dtype=torch.bfloat16, device=dev)
        sets.append((bufs, out))
    torch.cuda.synchronize()

    # ---- correctness of what is timed: sampled outputs against the oracle
    import oracle

    one = [mr.prepare_allreduce(b, o, "oneshot") for b, o in sets]
    one[0]()
    torch.cuda.synchronize()
    idx = np.linspace(0, n - 1, 1 << 16).astype(np.int64)
    want = oracle.allreduce_sum_ref([b[idx] for b in host], dtype)
    got = sets[0][1].view(torch.int16).cpu().numpy().view(np.uint16)[idx]
    verified = bool(np.array_equal(got, want))
    log(f"[bench] sampled parity vs oracle: {verified}")

    if args.calibrate:
        # a plain copy of known size: 268,435,456 bytes read and written per launch
        a = torch.empty(1 << 28, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---- headline: one-shot, rotating sets (HBM-resident inputs, cold caches)
    K = args.steps
    ms = time_steps(one, K, args.warmup, stream)
    t_launch = ms / K * 1e-3
    gbs = algo / t_launch / 1e9
    log(f"[bench] oneshot: {ms / K * 1e3:.2f} us/launch, {gbs:.1f} GB/s ({gbs / PEAK_GBS:.1%} of peak)")
    traffic, traffic_src = traffic_from_profile(algo)
    copy_gbs = copy_ceiling(mr, torch, dev, stream)
    log(f"[bench] plain 256 MiB copy (gather kernel, one shard) on the same GPU: {copy_gbs:.1f} GB/s")
    smix = stream_mix_ceiling(mr, torch, sets, n, s, stream, K, args.warmup)
    mix_gbs = smix["reads8_write1_pipelined"]["GBps"]
    log(f"[bench] stream-mix probe on the same buffers: 8 reads + 1 write {smix['reads8_write1_pipelined']['us']:.2f} us "
        f"({mix_gbs:.1f} GB/s) on the one-shot's schedule, {smix['reads8_write1']['us']:.2f} us "
        f"({smix['reads8_write1']['GBps']:.1f} GB/s) one tile per workgroup; 8 reads only "
        f"{smix['reads8_only']['us']:.2f} us ({smix['reads8_only']['GBps']:.1f} GB/s)")

    paths = {}
    if not args.only_headline:
        # secondary legs: a failure in one of them is recorded in the line instead of losing the
        # headline measured above
        try:
            # cache-resident one-shot: the same set every step (labelled: not an HBM figure)
            ms_w = time_steps(one[:1], K, args.warmup, stream)
            paths["oneshot_cache_resident"] = {"us": ms_w / K * 1e3, "GBps_algorithmic": algo / (ms_w / K * 1e-3) / 1e9,
                                               "note": "one buffer set reused; served partly from cache, not HBM"}
            # reduce-scatter: rank 0's 1/W share, rotating sets
            off, cnt = mr.reduce_scatter_chunk(n, W, dtype, 0)
            rs_out = [torch.empty(cnt, dtype=torch.bfloat16, device=dev) for _ in sets]
            rs = [mr.prepare_reduce_scatter(b, 0, o) for (b, _), o in zip(sets, rs_out)]
            ms_rs = time_steps(rs, K, args.warmup, stream)
            t_rs = ms_rs / K * 1e-3
            rs_bytes = (W + 1) * cnt * s
            paths["reduce_scatter_rank0"] = {"us": t_rs * 1e6, "GBps": rs_bytes / t_rs / 1e9, "bytes": rs_bytes,
                                             "elements": cnt}
            log(f"[bench] reduce_scatter (rank 0 share, {cnt} elements): {t_rs * 1e6:.2f} us/launch, "
                f"{rs_bytes / t_rs / 1e9:.1f} GB/s")
            # two-shot, rotating sets, under the default hand-off (at this size the last arriver on XCD-local
            # units) and under each other one
            two = [mr.prepare_allreduce(b, o, "twoshot") for b, o in sets]
            actual2 = (W + 3) * n * s
            kernels = {"auto": "twoshot_xcd<last arriver> (XCD-local units, the default at this size)",
                       "tile": "twoshot_xcd<copier workgroups> (XCD-local units)",
                       "chunk": "twoshot_vec<chunk barrier>", "grid": "twoshot_vec<grid barrier>"}
            for sync in ("auto", "tile", "chunk", "grid"):
                mr.set_option("twoshot_sync", sync)
                two[0]()
                torch.cuda.synchronize()
                ms2 = time_steps(two, K, args.warmup, stream)
                t2 = ms2 / K * 1e-3
                paths[f"twoshot_{sync}"] = {"us": t2 * 1e6, "GBps_metric_bytes": algo / t2 / 1e9,
                                            "GBps_actual_bytes": actual2 / t2 / 1e9, "actual_bytes": actual2,
                                            "frac_actual_bytes": actual2 / t2 / 1e9 / PEAK_GBS,
                                            "kernel": kernels[sync],
                                            "barrier_error_word": mr.workspace_check()}
                log(f"[bench] twoshot ({sync}): {t2 * 1e6:.2f} us/launch, {algo / t2 / 1e9:.1f} GB/s (metric bytes), "
                    f"{actual2 / t2 / 1e9:.1f} GB/s (actual)")
            mr.set_option("twoshot_sync", "auto")
            # reference: the same two phases as two launches (one-shot into a stage tensor, then a plain copy
            # of it into out by the gather kernel), same rotating sets -- what the in-kernel hand-off is
            # measured against
            stages = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in sets]
            two_launch = []
            for (b, o), stg in zip(sets, stages):
                red = mr.prepare_allreduce(b, stg, "oneshot")
                cp = mr.prepare_allgather_shards([stg], o)
                two_launch.append(lambda red=red, cp=cp: (red(), cp()))
            ms_tl = time_steps(two_launch, K, args.warmup, stream)
            t_tl = ms_tl / K * 1e-3
            paths["twoshot_two_launch_reference"] = {"us": t_tl * 1e6, "GBps_actual_bytes": actual2 / t_tl / 1e9,
                                                     "note": "one-shot into a stage tensor, then a copy kernel; two "
                                                             "launches per step, no in-kernel hand-off"}
            log(f"[bench] two-launch reference (one-shot into a stage, then a copy): {t_tl * 1e6:.2f} us/step")
            del stages, two_launch
            # param-contiguous scatter: W=8, G=4, P=64 log-uniform splits, bf16 random bits
            c4 = workloads.FSDP_SPLITS_W8_G4_P64
            splits = [int(x) for x in workloads.log_uniform_splits(c4["seed"], c4["P"])]
            T = sum(splits)
            gsets = []
            for k in range(2):
                src = torch.randint(-32768, 32767, (c4["W"] * T,), dtype=torch.int16, device=dev).view(torch.bfloat16)
                gsets.append(mr.prepare_allgather_param_contig(src, c4["W"], c4["G"], splits, torch.empty_like(src)))
            gbytes = 2 * c4["W"] * T * 2
            Kg = max(20, K // 10)
            msg = time_steps(gsets, Kg, max(2, args.warmup // 10), stream)
            tg = msg / Kg * 1e-3
            paths["param_contig"] = {"us": tg * 1e6, "GBps": gbytes / tg / 1e9, "bytes": gbytes, "W": c4["W"],
                                     "G": c4["G"], "P": c4["P"], "T": T, "dtype": "bf16",
                                     "frac": gbytes / tg / 1e9 / PEAK_GBS}
            paths["param_contig"].update(_same_bytes_copy(mr, gsets, Kg, args.warmup, stream, gbytes, gbytes / tg / 1e9))
            log(f"[bench] param_contig: {tg * 1e6:.1f} us/launch, {gbytes / tg / 1e9:.1f} GB/s ({gbytes} B); plain copy of "
                f"the same bytes {paths['param_contig']['copy_same_bytes_GBps']:.1f} GB/s")
            # the same gather on the SDMA copy engines (synchronous calls; no compute units), if the device
            # offers engines for its own memory
            sdma_legs = []
            if mr.sdma_engines() > 0:
                cu_below = mr.get_option("sdma_cu_below")
                sdma_sets = [mr.prepare_allgather_param_contig_sdma(c.keepalive[1], c4["W"], c4["G"], splits,
                                                                    c.keepalive[2]) for c in gsets]
                engines_only = [_with_option(mr, "sdma_cu_below", 0, c) for c in sdma_sets]
                big = [E for E in splits if E * 2 >= cu_below]
                split_note = (f"parameters with pieces of {cu_below} B and more on the engines "
                              f"({c4['W'] * sum(-(-E * 2 // (8 << 20)) for E in big)} copies, cut at 8 MiB), the other "
                              f"{c4['P'] - len(big)} parameters ({c4['W'] * 2 * (T - sum(big))} B) on one "
                              f"compute-unit launch beside them")
                Ks = 10
                for key, sets_, note in (("param_contig_sdma", sdma_sets, split_note),
                                         ("param_contig_sdma_engines_only", engines_only, "every piece on the engines")):
                    mss = time_steps(sets_, Ks, 2, stream)
                    ts = mss / Ks * 1e-3
                    paths[key] = {"us": ts * 1e6, "GBps": gbytes / ts / 1e9, "bytes": gbytes, "dtype": "bf16",
                                  "engines": mr.sdma_engines(), "sdma_cu_below": cu_below if sets_ is sdma_sets else 0,
                                  "note": "SDMA copy engines through the HSA runtime; synchronous calls, host-observed "
                                          "time per call; " + note}
                    log(f"[bench] {key} ({mr.sdma_engines()} SDMA engines): {ts * 1e6:.1f} us/call, "
                        f"{gbytes / ts / 1e9:.1f} GB/s")
                sdma_legs = [("scatter_fsdp_splits_bf16_sdma", sdma_sets[0]),
                             ("scatter_fsdp_splits_bf16_sdma_engines_only", engines_only[0])]
            else:
                paths["param_contig_sdma"] = {"skipped": "no SDMA engines offered for device-local copies"}
            # the same splits in fp32 (4-byte elements: twice the bytes of the bf16 case)
            fsets = []
            for k in range(2):
                src = torch.randint(-2 ** 31, 2 ** 31 - 1, (c4["W"] * T,), dtype=torch.int32, device=dev).view(torch.float32)
                fsets.append(mr.prepare_allgather_param_contig(src, c4["W"], c4["G"], splits, torch.empty_like(src)))
            fbytes = 2 * c4["W"] * T * 4
            msf = time_steps(fsets, Kg, max(2, args.warmup // 10), stream)
            tf = msf / Kg * 1e-3
            paths["param_contig_fp32"] = {"us": tf * 1e6, "GBps": fbytes / tf / 1e9, "bytes": fbytes, "W": c4["W"],
                                          "G": c4["G"], "P": c4["P"], "T": T, "dtype": "fp32",
                                          "frac": fbytes / tf / 1e9 / PEAK_GBS}
            paths["param_contig_fp32"].update(_same_bytes_copy(mr, fsets, Kg, args.warmup, stream, fbytes, fbytes / tf / 1e9))
            log(f"[bench] param_contig fp32: {tf * 1e6:.1f} us/launch, {fbytes / tf / 1e9:.1f} GB/s "
                f"({fbytes / tf / 1e9 / PEAK_GBS:.1%} of peak)")
            del fsets
            torch.cuda.empty_cache()
            # log-uniform splits of any element count (not rounded to 8): most pieces sit at a source
            # 16-byte phase other than their destination's, so the realigning build runs
            splits_any = [int(x) for x in workloads.log_uniform_splits(c4["seed"], c4["P"], mult=1)]
            Ta = sum(splits_any)
            asets = []
            for k in range(2):
                src = torch.randint(-32768, 32767, (c4["W"] * Ta,), dtype=torch.int16, device=dev).view(torch.bfloat16)
                asets.append(mr.prepare_allgather_param_contig(src, c4["W"], c4["G"], splits_any, torch.empty_like(src)))
            abytes = 2 * c4["W"] * Ta * 2
            msa = time_steps(asets, Kg, max(2, args.warmup // 10), stream)
            ta = msa / Kg * 1e-3
            paths["param_contig_any_size"] = {"us": ta * 1e6, "GBps": abytes / ta / 1e9, "bytes": abytes, "W": c4["W"],
                                              "G": c4["G"], "P": c4["P"], "T": Ta, "dtype": "bf16",
                                              "unaligned_splits": sum(E % 8 != 0 for E in splits_any),
                                              "frac": abytes / ta / 1e9 / PEAK_GBS}
            log(f"[bench] param_contig any-size splits: {ta * 1e6:.1f} us/launch, {abytes / ta / 1e9:.1f} GB/s")
            del asets
            torch.cuda.empty_cache()
            # the same gathers written straight from W separate shard buffers
            shard_sets = []
            for k in range(2):
                shards = [torch.randint(-32768, 32767, (T,), dtype=torch.int16, device=dev).view(torch.bfloat16)
                          for _ in range(c4["W"])]
                shard_sets.append((shards, torch.empty(c4["W"] * T, dtype=torch.bfloat16, device=dev)))
            for name, kw in (("allgather_into_tensor", {}), ("param_contig_shards", {"G": c4["G"], "splits": splits})):
                calls = [mr.prepare_allgather_shards(sh, o, **kw) for sh, o in shard_sets]
                msx = time_steps(calls, Kg, max(2, args.warmup // 10), stream)
                tx = msx / Kg * 1e-3
                paths[name] = {"us": tx * 1e6, "GBps": gbytes / tx / 1e9, "bytes": gbytes, "W": c4["W"], "T": T}
                log(f"[bench] {name}: {tx * 1e6:.1f} us/launch, {gbytes / tx / 1e9:.1f} GB/s")
            del shard_sets
            torch.cuda.empty_cache()
            paths["contention"] = contention_leg(mr, torch, dev, stream, gsets, gbytes, sdma_legs)
            del gsets, sdma_legs
            torch.cuda.empty_cache()
            if not args.no_sweep:
                paths["sweep_w8"] = sweep_leg(mr, torch, dev)
        except Exception as e:  # noqa: BLE001 -- reported, not hidden
            paths["error"] = f"{type(e).__name__}: {e}"
            log(f"[bench] secondary legs stopped: {paths['error']}")

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on the full headline workload (one call is the whole sample: about 0.07 s), median of
        # 3 runs single-threaded, then the same oracle over disjoint index ranges on every core this
        # process may run on (per-element rank order unchanged, so the bits are the same), median of 3
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.allreduce_sum_ref(host, dtype)
            times.append(time.perf_counter() - t0)
        med = float(np.median(times))
        nthr = max(1, len(os.sched_getaffinity(0)))
        ttimes = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.allreduce_sum_ref_threaded(host, dtype, nthr)
            ttimes.append(time.perf_counter() - t0)
        tmed = float(np.median(ttimes))
        cpu = {"value": algo / tmed / 1e9, "unit": "GB/s", "cores": nthr, "kind": "oracle",
               "sample": f"the full workload (W=8 x 8,388,608 bf16, one call), split over disjoint index ranges "
                         f"on every core this process may run on ({nthr}), median of 3 runs ({tmed:.3f} s)",
               "cpu_model": cpu_model(),
               "single_thread": {"value": algo / med / 1e9, "unit": "GB/s", "cores": 1, "seconds": med,
                                 "sample": "the same workload, numpy single-threaded, median of 3"}}
        log(f"[bench] cpu oracle: {med:.3f} s per call, {algo / med / 1e9:.2f} GB/s; "
            f"{nthr} threads: {tmed:.3f} s, {algo / tmed / 1e9:.2f} GB/s ({cpu['cpu_model']})")

    rec = {
        "metric": "achieved HBM GB/s (and % of peak) for W=8 bf16 all-reduce at 16 MB/rank, 1 GPU",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one-shot W-way sum-reduce, W=8 bf16 rank buffers of n=8,388,608 (16 MiB), "
                               "N(0,1) inputs, fp32 accumulation in rank order",
                   "W": W, "n": n, "mode": "oneshot", "accumulate": "fp32", "buffer_sets": args.sets,
                   "bytes_per_step": algo},
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "verified_vs_oracle": verified,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "oneshot_pipe<Bf16, 8>", "bytes_per_launch": algo,
                     "avg_launch_us": round(t_launch * 1e6, 3), "traffic_source": traffic_src,
                     "traffic_GBps": round(traffic / t_launch / 1e9, 1) if traffic else None,
                     "stream_mix_ceiling_GBps": round(mix_gbs, 1),
                     "stream_mix_ceiling_kernel": "mrx_stream_mix write=2: the one-shot's 8 rank buffers read and "
                                                  "their XOR written to out, same lane layout, same persistent "
                                                  "pipelined schedule, same rotating sets",
                     "frac_of_stream_mix_ceiling": round(gbs / mix_gbs, 4),
                     "stream_mix_one_tile_per_workgroup_GBps": round(smix["reads8_write1"]["GBps"], 1),
                     "reads_only_GBps": round(smix["reads8_only"]["GBps"], 1),
                     "copy_ceiling_GBps": round(copy_gbs, 1),
                     "copy_ceiling_kernel": "param_contig<4, false>: all_gather_into_tensor of one 256 MiB shard",
                     "frac_of_copy_ceiling": round(gbs / copy_gbs, 4)},
        "cpu_baseline": cpu,
        "paths": paths,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
