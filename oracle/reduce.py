"""W-way elementwise sum-reduce oracle.  Test infrastructure only.

Definition (custom all-reduce, one-shot and two-shot alike): for every element i,
    a = widen(x_0[i]);  a = fl32(a + widen(x_r[i])) for r = 1 .. W-1;  out[i] = narrow(a)
where fl32 is binary32 addition with round-to-nearest-even.  One-shot (page "Question and suggestions
about custom allreduce", the quoted one-shot block schedule) and two-shot (the same page's question on
reduce-scatter then gather; page "triton_multimem_all_reduce.py", the per-rank slice of 128-bit packs)
compute the same values; two-shot only changes which worker computes which slice, so one oracle serves
both.  The accumulation order and precision are not on the pages; fp32 in rank order 0..W-1 is the
reading taken.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .numerics import narrow, widen

FLOAT_DTYPES = ("bf16", "fp16", "fp32")


def allreduce_sum_ref(bufs: list[np.ndarray], dtype: str) -> np.ndarray:
    """Sum W rank buffers of raw ``dtype`` bits elementwise; returns raw bits of ``dtype``."""
    if dtype not in FLOAT_DTYPES:
        raise ValueError(f"the all-reduce is defined for floating types only, not {dtype}")
    if len(bufs) < 1:
        raise ValueError("need at least one rank buffer")
    n = bufs[0].shape[0]
    for b in bufs:
        if b.shape != (n,):
            raise ValueError("rank buffers must have the same length")
    acc = widen(bufs[0], dtype)
    with np.errstate(over="ignore", invalid="ignore"):  # inf and NaN are legitimate results
        for r in range(1, len(bufs)):
            acc = np.add(acc, widen(bufs[r], dtype), dtype=np.float32)
    return narrow(acc, dtype)


def allreduce_sum_ref_threaded(bufs: list[np.ndarray], dtype: str, threads: int | None = None) -> np.ndarray:
    """The same oracle over disjoint index ranges in a thread pool.

    Each element's rank order is unchanged, so the bits equal ``allreduce_sum_ref``.  Used only to time
    the CPU baseline on several cores.
    """
    n = bufs[0].shape[0]
    threads = threads or len(os.sched_getaffinity(0))
    out = np.empty(n, dtype=bufs[0].dtype)
    edges = np.linspace(0, n, threads + 1).astype(np.int64)

    def part(k: int) -> None:
        a, b = int(edges[k]), int(edges[k + 1])
        out[a:b] = allreduce_sum_ref([x[a:b] for x in bufs], dtype)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(part, range(threads)))
    return out


def reduce_scatter_chunk(n: int, W: int, dtype: str, rank: int) -> tuple[int, int]:
    """Element range [start, stop) of rank ``rank``'s share of an n-element reduce-scatter.

    Two-shot's reduce-scatter hands chunk c to owner c.  The pages leave the chunk length open when W
    does not divide n (the Triton page's per-rank slice is cdiv(numel/8, W) 128-bit packs and is not
    masked); the reading taken: C = ceil(n/W) rounded up to a whole 16-byte pack, chunk c =
    [c*C, min((c+1)*C, n)), so trailing chunks may be short or empty.
    """
    V = 16 // {"bf16": 2, "fp16": 2, "fp32": 4}[dtype]
    per = -(-n // W)
    C = -(-per // V) * V
    start = min(rank * C, n)
    return start, min(start + C, n)


def reduce_scatter_sum_ref(bufs: list[np.ndarray], dtype: str, rank: int) -> np.ndarray:
    """Rank ``rank``'s share of the reduce-scatter: the W-way sum over its chunk only."""
    n = bufs[0].shape[0]
    a, b = reduce_scatter_chunk(n, len(bufs), dtype, rank)
    return allreduce_sum_ref([x[a:b] for x in bufs], dtype)
