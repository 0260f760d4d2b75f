"""Param-contiguous all-gather placement oracle.  Test infrastructure only.

Page "ccl: hierarchical cross-node AllGather (intra-node SDMA + inter-node RDMA) #441", the commit that
adds ``enqueue_param_contiguous``: the gathered result goes straight into FSDP's [param][rank] output.
The W ranks form W/G node-blocks of G ranks.  For node-block m and parameter split s the destination
block starts at ``O_s*W + m*G*E_s`` and consecutive slots g are ``E_s`` apart, so rank r = m*G + g
lands at ``O_s*W + r*E_s``.  ``O_s`` is the exclusive prefix sum of the split element counts in split
order (the splits are counted in elements of the dtype) and ``T = sum(E_s)`` is one rank's shard
length.  The commit that fuses the per-(node-block, split) launches loops over node-blocks, then splits,
then slots; the loop order below is that one.  The copy is done on integer views, so every bit pattern
(NaN payloads included) is kept.
"""
from __future__ import annotations

import numpy as np


def param_offsets(splits) -> tuple[np.ndarray, int]:
    """Exclusive prefix sums O_s (uint64) and the shard length T."""
    e = np.asarray(splits, dtype=np.uint64)
    o = np.zeros(len(e), dtype=np.uint64)
    if len(e) > 1:
        o[1:] = np.cumsum(e[:-1], dtype=np.uint64)
    return o, int(e.sum(dtype=np.uint64))


def allgather_param_contig_ref(src: np.ndarray, W: int, G: int, splits) -> np.ndarray:
    """``src`` is the rank-major gathered buffer [W][T] (flat, any integer bit view).

    Returns the [param][rank] buffer of the same length.
    """
    if W < 1 or G < 1 or W % G != 0:
        raise ValueError("need W >= 1, G >= 1 and G dividing W")
    e = [int(v) for v in np.asarray(splits, dtype=np.uint64)]
    o, T = param_offsets(e)
    if src.shape != (W * T,):
        raise ValueError(f"src must hold W*T = {W * T} elements, has {src.shape}")
    out = np.empty_like(src)
    for m in range(W // G):                     # node-blocks
        for s, E in enumerate(e):               # parameter splits
            O = int(o[s])
            dst_block = O * W + m * G * E       # start of node-block m inside param s
            for g in range(G):                  # slots of the node-block, stride E
                r = m * G + g
                dst = dst_block + g * E
                out[dst:dst + E] = src[r * T + O:r * T + O + E]
    return out


def allgather_into_tensor_ref(shards: list[np.ndarray]) -> np.ndarray:
    """Rank-major all-gather of W equal shards (torch.distributed.all_gather_into_tensor's layout):
    out[r*T + j] = shards[r][j]."""
    T = shards[0].shape[0]
    out = np.empty(len(shards) * T, dtype=shards[0].dtype)
    for r, x in enumerate(shards):
        if x.shape != (T,):
            raise ValueError("shards must have the same length")
        out[r * T:(r + 1) * T] = x
    return out


def allgather_list_ref(shards: list[np.ndarray]) -> list[np.ndarray]:
    """List-output all-gather (torch.distributed.all_gather's layout): output r is a copy of shard r."""
    return [x.copy() for x in shards]


def allgather_param_contig_shards_ref(shards: list[np.ndarray], G: int, splits) -> np.ndarray:
    """Param-contiguous all-gather straight from W separate rank shards (the zero-copy push of the
    page's enqueue_param_contiguous): the same placement as allgather_param_contig_ref applied to the
    rank-major concatenation of the shards."""
    return allgather_param_contig_ref(allgather_into_tensor_ref(shards), len(shards), G, splits)
