"""Python binding of libmr, the MI355X W-way sum-reduce and param-contiguous gather library.

A thin ctypes layer over the C ABI declared in include/mr.h: it turns torch tensors into device
pointers, sizes and the current HIP stream, calls the entry point of the same name and raises on a
non-zero status.  Every step of the computation runs in the HIP kernels of libmr.so; there is no
fallback.  If libmr.so has not been built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmr.so")

MR_OK = 0
STATUS = {
    0: "MR_OK",
    -1: "MR_ERR_INVALID_ARG",
    -2: "MR_ERR_DTYPE",
    -3: "MR_ERR_ALIAS",
    -4: "MR_ERR_WORKSPACE",
    -5: "MR_ERR_HIP",
    -6: "MR_ERR_ENGINE",
}
DTYPE_CODE = {"bf16": 0, "fp16": 1, "fp32": 2, "int32": 3}
MODE_CODE = {"oneshot": 0, "twoshot": 1}
OPTION_CODE = {"twoshot_sync": 0, "spin_limit": 1, "tile_shape": 2, "sdma_cu_below": 3}
TWOSHOT_SYNC = {"tile": 0, "chunk": 1, "grid": 2, "last": 3, "auto": 4}
TILE_SHAPE = {"auto": 0, "wide": 1, "medium": 2, "narrow": 3, "wide_pair": 4}
MAX_W = 16
MAX_PARAMS_PER_LAUNCH = 128
MAX_TABLE_W = 64

# Exported symbols of include/mr.h, with ctypes signatures.
_SIGS = {
    "mr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mr_last_hip_error": (ctypes.c_int, []),
    "mr_version": (ctypes.c_int, []),
    "mr_allreduce_sum": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "mr_allreduce_sum_noalloc": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                                                ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "mr_allgather_param_contig": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_uint64), ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p]),
    "mr_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_size_t, ctypes.c_int]),
    "mr_set_workspace": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]),
    "mr_workspace_check": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]),
    "mr_reduce_scatter_chunk": (ctypes.c_int, [ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "mr_reduce_scatter_sum": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "mr_allgather_into_tensor": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                                                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "mr_allgather_list": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                                         ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
    "mr_allgather_param_contig_shards": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int,
                                                        ctypes.POINTER(ctypes.c_uint64), ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_void_p, ctypes.c_void_p]),
    "mr_allgather_param_contig_sdma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                      ctypes.POINTER(ctypes.c_uint64), ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_void_p, ctypes.c_void_p]),
    "mr_sdma_engines": (ctypes.c_int, []),
    "mr_set_option": (ctypes.c_int, [ctypes.c_int, ctypes.c_int64]),
    "mr_get_option": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]),
}
EXPORTS = tuple(_SIGS)

_lib = None


class MRError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """Load libmr.so (once).  Raises if it is missing: the product path has no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != MR_OK:
        raise MRError(status, what)


def _torch():
    import torch

    return torch


def dtype_name(t) -> str:
    torch = _torch()
    return {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32", torch.int32: "int32"}[t.dtype]


def _stream_handle(stream) -> int | None:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


def _dev_tensor(t, what: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous device tensor")


def _splits_array(splits: Sequence[int]):
    sp = [int(x) for x in splits]
    if not sp or min(sp) < 0:
        raise ValueError("splits must be a non-empty list of non-negative element counts")
    return (ctypes.c_uint64 * len(sp))(*sp), sum(sp)


def _same(tensors, ref, what: str, numel: int) -> None:
    """Every tensor is a contiguous device tensor of ref's dtype holding exactly ``numel`` elements."""
    for t in tensors:
        _dev_tensor(t, what)
        if t.dtype != ref.dtype or t.numel() != numel:
            raise ValueError(f"{what} must hold {numel} elements of {ref.dtype}")


def _prepared(name: str, f, args, keep):
    def call() -> None:
        st = f(*args)
        if st != MR_OK:
            raise MRError(st, name)

    call.keepalive = keep
    return call


# Each prepare_* checks that every tensor is a contiguous device tensor of the sizes the call implies
# (the library takes raw pointers and cannot check extents) and marshals the arguments once; the
# returned no-argument callable enqueues that same call (tight timing loops, graph capture).  The
# plain functions are one prepared call.

def prepare_allreduce(bufs: Sequence, out, mode: str = "oneshot", stream=None):
    """Pre-marshalled mr_allreduce_sum: out = elementwise fp32 sum (rank order) of the tensors ``bufs``."""
    _dev_tensor(out, "out")
    _same(bufs, out, "rank buffer", out.numel())
    ptrs = (ctypes.c_void_p * max(len(bufs), 1))(*[b.data_ptr() for b in bufs])
    args = (ptrs, len(bufs), out.numel(), DTYPE_CODE[dtype_name(out)], out.data_ptr(), MODE_CODE[mode],
            _stream_handle(stream))
    return _prepared("mr_allreduce_sum", lib().mr_allreduce_sum, args, (ptrs, list(bufs), out))


def allreduce_sum(bufs: Sequence, out, mode: str = "oneshot", stream=None):
    """out = elementwise fp32 sum (rank order 0..W-1) of the W same-shape, same-dtype tensors ``bufs``."""
    prepare_allreduce(bufs, out, mode, stream)()
    return out


NOALLOC_MAX_BYTES = 32 << 20


def prepare_allreduce_noalloc(bufs: Sequence, out, mode: str = "oneshot", stream=None):
    """Pre-marshalled mr_allreduce_sum_noalloc (two-shot workspace inside the library; never allocates)."""
    _dev_tensor(out, "out")
    _same(bufs, out, "rank buffer", out.numel())
    ptrs = (ctypes.c_void_p * max(len(bufs), 1))(*[b.data_ptr() for b in bufs])
    args = (ptrs, len(bufs), out.numel(), DTYPE_CODE[dtype_name(out)], out.data_ptr(), MODE_CODE[mode],
            _stream_handle(stream))
    return _prepared("mr_allreduce_sum_noalloc", lib().mr_allreduce_sum_noalloc, args, (ptrs, list(bufs), out))


def allreduce_sum_noalloc(bufs: Sequence, out, mode: str = "oneshot", stream=None):
    """allreduce_sum without any device allocation (rank buffers up to NOALLOC_MAX_BYTES)."""
    prepare_allreduce_noalloc(bufs, out, mode, stream)()
    return out


def reduce_scatter_chunk(n: int, W: int, dtype: str, rank: int) -> tuple[int, int]:
    """(offset, count) of rank ``rank``'s chunk of an n-element reduce-scatter."""
    off, cnt = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().mr_reduce_scatter_chunk(n, W, DTYPE_CODE[dtype], rank, ctypes.byref(off), ctypes.byref(cnt)),
           "mr_reduce_scatter_chunk")
    return int(off.value), int(cnt.value)


def prepare_reduce_scatter(bufs: Sequence, rank: int, out, stream=None):
    """Pre-marshalled mr_reduce_scatter_sum: out = rank ``rank``'s chunk of the sum of ``bufs``."""
    _dev_tensor(out, "out")
    n = bufs[0].numel() if len(bufs) else 0
    _same(bufs, out, "rank buffer", n)
    _, cnt = reduce_scatter_chunk(n, len(bufs), dtype_name(out), rank)
    if out.numel() != cnt:
        raise ValueError(f"out must hold the chunk's {cnt} elements")
    ptrs = (ctypes.c_void_p * max(len(bufs), 1))(*[b.data_ptr() for b in bufs])
    args = (ptrs, len(bufs), n, DTYPE_CODE[dtype_name(out)], rank, out.data_ptr(), _stream_handle(stream))
    return _prepared("mr_reduce_scatter_sum", lib().mr_reduce_scatter_sum, args, (ptrs, list(bufs), out))


def reduce_scatter_sum(bufs: Sequence, rank: int, out, stream=None):
    """out = rank ``rank``'s chunk of the elementwise sum of the W same-shape tensors ``bufs``."""
    prepare_reduce_scatter(bufs, rank, out, stream)()
    return out


def prepare_allgather_param_contig(src, W: int, G: int, splits: Sequence[int], out, stream=None):
    """Pre-marshalled mr_allgather_param_contig (src rank-major [W][T], T = sum(splits))."""
    _dev_tensor(src, "src")
    sp, T = _splits_array(splits)
    if W < 1 or src.numel() != W * T:
        raise ValueError(f"src must hold W*sum(splits) = {max(W, 0) * T} elements")
    _same([out], src, "out", src.numel())
    args = (src.data_ptr(), W, G, sp, len(sp), DTYPE_CODE[dtype_name(src)], out.data_ptr(), _stream_handle(stream))
    return _prepared("mr_allgather_param_contig", lib().mr_allgather_param_contig, args, (sp, src, out))


def allgather_param_contig(src, W: int, G: int, splits: Sequence[int], out, stream=None):
    """Scatter the rank-major ``src`` ([W][T], T = sum(splits)) into [param][rank] order in ``out``."""
    prepare_allgather_param_contig(src, W, G, splits, out, stream)()
    return out


def prepare_allgather_param_contig_sdma(src, W: int, G: int, splits: Sequence[int], out, stream=None):
    """Pre-marshalled mr_allgather_param_contig_sdma: the same placement on the SDMA copy engines (a
    synchronous call: it waits for ``stream``, copies, and returns when the copies are complete)."""
    _dev_tensor(src, "src")
    sp, T = _splits_array(splits)
    if W < 1 or src.numel() != W * T:
        raise ValueError(f"src must hold W*sum(splits) = {max(W, 0) * T} elements")
    _same([out], src, "out", src.numel())
    args = (src.data_ptr(), W, G, sp, len(sp), DTYPE_CODE[dtype_name(src)], out.data_ptr(), _stream_handle(stream))
    return _prepared("mr_allgather_param_contig_sdma", lib().mr_allgather_param_contig_sdma, args, (sp, src, out))


def allgather_param_contig_sdma(src, W: int, G: int, splits: Sequence[int], out, stream=None):
    """mr_allgather_param_contig's placement copied by the SDMA engines (synchronous)."""
    prepare_allgather_param_contig_sdma(src, W, G, splits, out, stream)()
    return out


def sdma_engines() -> int:
    """SDMA engines the current device offers for copies within its own memory."""
    return int(lib().mr_sdma_engines())


def _shard_ptrs(shards):
    if not len(shards):
        raise ValueError("at least one shard")
    _same(shards, shards[0], "shard", shards[0].numel())
    return (ctypes.c_void_p * len(shards))(*[t.data_ptr() for t in shards])


def prepare_allgather_shards(shards: Sequence, out, G: int | None = None, splits: Sequence[int] | None = None,
                             stream=None):
    """Pre-marshalled gather from W shards: rank-major into ``out`` (``splits`` None, mr_allgather_into_tensor)
    or param-contiguous (mr_allgather_param_contig_shards, each shard sum(splits) elements)."""
    ptrs = _shard_ptrs(shards)
    W, T = len(shards), shards[0].numel()
    _same([out], shards[0], "out", W * T)
    dt = DTYPE_CODE[dtype_name(out)]
    if splits is None:
        name, args = "mr_allgather_into_tensor", (ptrs, W, T, dt, out.data_ptr(), _stream_handle(stream))
    else:
        sp, ST = _splits_array(splits)
        if ST != T:
            raise ValueError(f"each shard must hold sum(splits) = {ST} elements")
        name = "mr_allgather_param_contig_shards"
        args = (ptrs, W, W if G is None else G, sp, len(sp), dt, out.data_ptr(), _stream_handle(stream))
    return _prepared(name, getattr(lib(), name), args, (args, list(shards), out))


def allgather_into_tensor(shards: Sequence, out, stream=None):
    """out[r*T:(r+1)*T] = shards[r] (rank-major all-gather of W shards of T elements)."""
    prepare_allgather_shards(shards, out, stream=stream)()
    return out


def allgather_param_contig_shards(shards: Sequence, G: int, splits: Sequence[int], out, stream=None):
    """[param][rank] all-gather written straight from W shards (each sum(splits) elements)."""
    prepare_allgather_shards(shards, out, G, splits, stream)()
    return out


def allgather_list(shards: Sequence, outs: Sequence, stream=None):
    """outs[r] = shards[r] for every rank (list-output all-gather), one launch."""
    ptrs = _shard_ptrs(shards)
    if len(outs) != len(shards):
        raise ValueError("one output per shard")
    _same(outs, shards[0], "output", shards[0].numel())
    optrs = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    _check(lib().mr_allgather_list(ptrs, len(shards), shards[0].numel(), DTYPE_CODE[dtype_name(shards[0])], optrs,
                                   _stream_handle(stream)), "mr_allgather_list")
    return outs


def workspace_bytes(W: int, n: int, dtype: str) -> int:
    return int(lib().mr_workspace_bytes(W, n, DTYPE_CODE[dtype]))


def set_workspace(buf=None, stream=None) -> None:
    """Bind a caller-owned uint8 device tensor as the two-shot workspace of ``stream`` (None unbinds)."""
    ptr, nbytes = (None, 0) if buf is None else (buf.data_ptr(), buf.numel() * buf.element_size())
    _check(lib().mr_set_workspace(_stream_handle(stream), ptr, nbytes), "mr_set_workspace")


def workspace_check(stream=None) -> int:
    """Synchronise ``stream`` and return (and clear) its two-shot barrier error word."""
    flags = ctypes.c_uint32(0)
    _check(lib().mr_workspace_check(_stream_handle(stream), ctypes.byref(flags)), "mr_workspace_check")
    return int(flags.value)


def set_option(name: str, value) -> None:
    """Set a process-wide option: ``twoshot_sync`` ("auto", "tile", "chunk", "grid", "last"), ``spin_limit`` (int),
    ``tile_shape`` ("auto", "wide", "medium", "narrow", "wide_pair") or ``sdma_cu_below`` (bytes)."""
    if name == "twoshot_sync" and isinstance(value, str):
        value = TWOSHOT_SYNC[value]
    if name == "tile_shape" and isinstance(value, str):
        value = TILE_SHAPE[value]
    _check(lib().mr_set_option(OPTION_CODE[name], int(value)), "mr_set_option")


def get_option(name: str):
    v = ctypes.c_int64(0)
    _check(lib().mr_get_option(OPTION_CODE[name], ctypes.byref(v)), "mr_get_option")
    if name == "twoshot_sync":
        return {c: k for k, c in TWOSHOT_SYNC.items()}[v.value]
    if name == "tile_shape":
        return {c: k for k, c in TILE_SHAPE.items()}[v.value]
    return int(v.value)
