"""CPU oracle for the W-way sum-reduce and the param-contiguous gather.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this package: only
the tests, the smoke check and the bench's CPU-baseline leg use it.  It shares no code with the HIP
library and never reads anything the HIP library produced.

It is deliberately plain and slow: numpy on unsigned bit views, vectorised over elements only, with no
blocking, fusion or reordering beyond what the definitions below state.  Two operations:

* ``allreduce_sum_ref`` -- the elementwise sum over W rank buffers that one-shot and two-shot custom
  all-reduce compute (page "Question and suggestions about custom allreduce", sglang discussion 2918:
  the quoted trt_reduce_internal.cu comment on the per-block one-shot schedule, where each block pulls
  its chunk from every peer and sums it; page "triton_multimem_all_reduce.py", multimem_all_reduce_kernel,
  where each 128-bit pack is sum-reduced across all ranks).  The pages fix neither the accumulation
  precision nor the order; this oracle takes fp32 accumulation in rank order 0..W-1, starting from rank
  0's widened value, and round-to-nearest-even narrowing to the output type.
* ``allgather_param_contig_ref`` -- the rank-major to [param][rank] placement of the hierarchical
  all-gather (page "ccl: hierarchical cross-node AllGather (intra-node SDMA + inter-node RDMA) #441",
  the commit that adds ``enqueue_param_contiguous`` and the commit that fuses the node-block x split
  loop into one launch): for node-block m, split s and slot g, rank r = m*G + g lands at
  ``O_s*W + m*G*E_s + g*E_s``.

Also: ``reduce_scatter_sum_ref`` (one owner's 1/W share of the same sum, the phase-1 half of two-shot),
``allgather_into_tensor_ref`` / ``allgather_list_ref`` (rank-major and list-output all-gather of W shards)
and ``allgather_param_contig_shards_ref`` (the param-contiguous placement straight from W shards).

Pins (tests/test_oracle.py) tie every function to something other than itself: exact-rational IEEE
arithmetic written from the standard, closed forms, invariants and library routines.
"""
from __future__ import annotations

from .numerics import narrow, widen  # noqa: F401
from .reduce import (allreduce_sum_ref, allreduce_sum_ref_threaded, reduce_scatter_chunk,  # noqa: F401
                     reduce_scatter_sum_ref)
from .gather import (allgather_into_tensor_ref, allgather_list_ref, allgather_param_contig_ref,  # noqa: F401
                     allgather_param_contig_shards_ref, param_offsets)
