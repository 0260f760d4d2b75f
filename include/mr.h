/*
 * mr.h -- C ABI of libmr: the W-way elementwise sum-reduce and the param-contiguous gather on one
 * MI355X (gfx950).
 *
 * Plain C. Only <stddef.h> and <stdint.h> are needed.  Every pointer argument marked "device" is GPU
 * memory (hipMalloc'd or torch-allocated) on the current HIP device; "host" pointers are CPU memory
 * read during the call only.  Streams are hipStream_t values (NULL = the default stream); the type
 * below is layout-compatible with hipStream_t, so HIP callers pass their stream directly.
 *
 * Semantics shared by every entry point:
 *  - Work is enqueued asynchronously on `stream`; no call synchronises the host except
 *    mr_workspace_check, mr_set_workspace when it frees library-owned buffers, and the copy-engine
 *    gather mr_allgather_param_contig_sdma (see there).  Kernel faults surface at the caller's next
 *    synchronisation (HIP convention).
 *  - Arguments are validated before any HIP call; an invalid call enqueues nothing.
 *  - The caller owns every buffer it passes and keeps it alive until the stream work completes (with
 *    a caching allocator and side streams, record the buffer on the stream).  The library never frees
 *    caller memory.
 *  - Return value: MR_OK (0) or a negative mr_status code; mr_status_string() names it and
 *    mr_last_hip_error() gives the hipError_t behind the calling thread's last MR_ERR_HIP.
 */
#ifndef MR_H_
#define MR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* mr_stream; /* == hipStream_t */

typedef int mr_status;
#define MR_OK 0
#define MR_ERR_INVALID_ARG (-1) /* null pointer, W/G/P out of range, size overflow */
#define MR_ERR_DTYPE (-2)       /* dtype not supported by this operation */
#define MR_ERR_ALIAS (-3)       /* output partially overlaps an input */
#define MR_ERR_WORKSPACE (-4)   /* two-shot workspace missing or too small (barrier errors: mr_workspace_check) */
#define MR_ERR_HIP (-5)         /* a HIP runtime call failed; see mr_last_hip_error() */
#define MR_ERR_ENGINE (-6)      /* SDMA copy engines unavailable or a copy failed; see mr_last_hip_error() */

typedef enum mr_dtype { MR_BF16 = 0, MR_FP16 = 1, MR_FP32 = 2, MR_INT32 = 3 } mr_dtype;
typedef enum mr_mode { MR_ONESHOT = 0, MR_TWOSHOT = 1 } mr_mode;

#define MR_MAX_W 16
#define MR_MAX_PARAMS_PER_LAUNCH 128
#define MR_MAX_TABLE_W 64 /* ranks in the shard-list gathers (pointer tables ride in the launch arguments) */

/* Human-readable name of a status code (static string, never NULL). */
const char* mr_status_string(mr_status status);

/* hipError_t value behind the calling thread's most recent MR_ERR_HIP, or for MR_ERR_ENGINE the HSA
 * runtime's hsa_status_t (or -1: an engine reported a failed copy); 0 if none. */
int mr_last_hip_error(void);

/*
 * mr_allreduce_sum -- one rank's result of a sum all-reduce over W rank buffers.
 *
 * Computes, for every element i < n,
 *     out[i] = narrow( (((widen(bufs[0][i]) + widen(bufs[1][i])) + ...) + widen(bufs[W-1][i])) )
 * with each term widened exactly to fp32, every add an fp32 round-to-nearest-even add in rank order
 * 0..W-1 (no reassociation, subnormals kept), and the sum rounded to nearest even into `dtype`.
 * That is the elementwise sum each block of a one-shot custom all-reduce forms after pulling its
 * chunk from every peer (page "Question and suggestions about custom allreduce", the quoted one-shot
 * block schedule), and the per-slice sum of two-shot (same page, reduce-scatter then gather; page
 * "triton_multimem_all_reduce.py", the per-rank slice of 128-bit packs).  The result is bit-identical
 * in both modes.
 *
 *  bufs   host array of W device pointers, each to n contiguous elements of `dtype` (read only).
 *         Pointers may repeat.  Any alignment is accepted.  When every pointer and out have the same
 *         address modulo 16 the kernels use aligned 16-byte loads and stores; when they are all
 *         multiples of the element size but their 16-byte phases differ, each input pack is realigned
 *         in registers from the two aligned packs it straddles (slightly slower: about 26.4 us
 *         instead of 24.5 us one-shot, 35 us instead of 31.5 us two-shot, for W=8 bf16 at 16 MiB); when some
 *         pointer is not a multiple of the element size, the call runs element by element with
 *         single-byte loads and stores only (much slower), never an unaligned multi-byte access.
 *  W      1 .. MR_MAX_W.
 *  n      elements per buffer; n == 0 is a successful no-op.
 *  dtype  MR_BF16, MR_FP16 or MR_FP32 (output has the same dtype); MR_INT32 -> MR_ERR_DTYPE.
 *  out    device pointer to n elements.  out == bufs[k] (exactly) is allowed (in place); any other
 *         overlap with an input -> MR_ERR_ALIAS.
 *  mode   MR_ONESHOT: one pass, W reads and one write per element.
 *         MR_TWOSHOT: phase 1 reduces the message into a stage buffer, share by share, an intra-GPU
 *         flag hand-off orders the phases, phase 2 copies the stage into out; the result is the
 *         same.  The shares are whole 16-byte packs of the aligned body (on out's 16-byte grid):
 *         W chunks of ceil(packs/W) packs each (the last ones may be short or empty), or, on the
 *         16-byte path with W <= 8 (the last arriver at any size, per-tile flags from 16 to
 *         64 MiB), one run of units per XCD (1, 4 or 16 KiB of output each, by size); the few
 *         elements before out's first 16-byte boundary and after its last whole pack are reduced
 *         with the first share.  (mr_reduce_scatter_sum's chunks, which are defined on element
 *         indices, coincide with the W chunks when n is a multiple of 16 bytes and out is 16-byte
 *         aligned.)  Needs a workspace (see below).
 *  stream hipStream_t to enqueue on.
 */
mr_status mr_allreduce_sum(const void* const* bufs, int W, size_t n, mr_dtype dtype, void* out,
                           mr_mode mode, mr_stream stream);

/*
 * mr_allgather_param_contig -- scatter a rank-major gathered buffer into [param][rank] order.
 *
 * src holds W rank shards of T = sum(splits) elements each, back to back ([W][T]).  Shard r is laid
 * out as P parameter pieces of splits[s] elements at offset O_s = splits[0] + ... + splits[s-1].
 * out receives, for every parameter s, the W pieces of s one after another:
 *     out[O_s*W + r*splits[s] + j] = src[r*T + O_s + j]
 * Ranks form W/G node-blocks of G ranks; the launch walks node-block m, then parameter s, then slot g
 * (rank r = m*G + g), placing node-block m of parameter s at O_s*W + m*G*splits[s] with slot stride
 * splits[s] (page "ccl: hierarchical cross-node AllGather (intra-node SDMA + inter-node RDMA) #441",
 * the commit adding enqueue_param_contiguous and the commit fusing the node-block x split loop into
 * one launch).  The output does not depend on G.  It is a pure bit copy: every dtype bit pattern,
 * NaN payloads included, is preserved; dtype only sets the element size.
 *
 *  src     device pointer, W*T elements (read only).
 *  W       1 .. 65535;  G >= 1 with W % G == 0 (G == W: one node-block).
 *  splits  host array of P element counts (splits[s] == 0 allowed).  Read during the call only.
 *  P       >= 1.  Up to MR_MAX_PARAMS_PER_LAUNCH parameters go in one kernel launch; more are split
 *          into independent launches of up to that many parameters each (all validated before the
 *          first is enqueued).
 *  dtype   any mr_dtype (element size 2 or 4 bytes).
 *  out     device pointer, W*T elements.  Any overlap with src -> MR_ERR_ALIAS.
 *  Any alignment of src and out is accepted: pieces whose source and destination share a 16-byte
 *  phase are copied as aligned 16-byte packs, others as destination-aligned packs realigned in
 *  registers, and pointers that are not multiples of the element size make the launch work in bytes
 *  (byte-granular edges).  All offsets are 64-bit; buffers beyond 2^31 bytes are supported.
 */
mr_status mr_allgather_param_contig(const void* src_rank_major, int W, int G, const uint64_t* splits,
                                    int P, mr_dtype dtype, void* out, mr_stream stream);

/*
 * mr_allgather_param_contig_sdma -- mr_allgather_param_contig's placement, copied by the GPU's SDMA
 * engines instead of its compute units.
 *
 * The mori page's hierarchical all-gather moves intra-node data on copy engines so that a concurrent
 * GEMM keeps the compute units (page "ccl: hierarchical cross-node AllGather (intra-node SDMA +
 * inter-node RDMA) #441", PR summary: copy engines against CU contention).  Here every (parameter,
 * rank) piece -- src[r*T + O_s .. + splits[s]) to out[O_s*W + r*splits[s] ..) -- is one 1-D engine copy
 * (pieces above 8 MiB are cut), spread over every SDMA engine the device reports.  An engine spends
 * about 15 microseconds on every copy beyond its bytes, so parameters whose pieces are smaller than
 * MR_OPT_SDMA_CU_BELOW bytes are copied instead by one launch of the param-contiguous kernel on
 * `stream`, which runs beside the engine copies (the same page later moves a copy step from the
 * engines to a compute-unit kernel).  Output bits are those of mr_allgather_param_contig.
 *
 * Arguments, limits and errors as mr_allgather_param_contig, plus MR_ERR_ENGINE.  Unlike every other
 * entry point this call is synchronous: it waits until `stream` has finished its earlier work (the
 * engines are not ordered by the stream), then copies (the kernel part, if any, enqueued on `stream`),
 * and returns once every copy is complete, the kernel part's included; work
 * enqueued on any stream afterwards sees the result.  Not capturable in a HIP graph.  The first call
 * on a device initialises the HSA runtime and creates one HSA signal that the library keeps for that
 * device until the process ends.
 *
 * mr_sdma_engines: number of SDMA engines the current device offers for its own memory; 0 if none or
 * the HSA runtime is unavailable, and then mr_last_hip_error() gives the HSA runtime's hsa_status_t.
 */
mr_status mr_allgather_param_contig_sdma(const void* src_rank_major, int W, int G, const uint64_t* splits, int P,
                                         mr_dtype dtype, void* out, mr_stream stream);
int mr_sdma_engines(void);

/*
 * mr_reduce_scatter_chunk / mr_reduce_scatter_sum -- one rank's share of a sum reduce-scatter.
 *
 * Two-shot's first phase hands chunk c of the message to owner c (page "Question and suggestions
 * about custom allreduce", the two-shot reduce-scatter; page "triton_multimem_all_reduce.py", each
 * rank's slice of cdiv(numel/8, W) 128-bit packs); it is also the gradient half of FSDP sharding.
 * Chunk c is elements [c*C, min((c+1)*C, n)) with C = ceil(n/W) rounded up to a whole 16 bytes
 * (8 bf16/fp16 or 4 fp32 elements), so trailing chunks may be short or empty.
 *
 * mr_reduce_scatter_chunk: host-only; writes chunk `rank`'s first element and length.
 * mr_reduce_scatter_sum:   out[j] = the mr_allreduce_sum formula at element offset+j, for j < count,
 *                          reading only that chunk of each rank buffer.  bufs/W/n/dtype as for
 *                          mr_allreduce_sum; 0 <= rank < W; out is a device buffer of `count`
 *                          elements; out may equal bufs[k] + offset exactly (in place), any other
 *                          overlap with a read chunk -> MR_ERR_ALIAS.  count == 0 is a no-op.
 */
mr_status mr_reduce_scatter_chunk(size_t n, int W, mr_dtype dtype, int rank, size_t* offset, size_t* count);
mr_status mr_reduce_scatter_sum(const void* const* bufs, int W, size_t n, mr_dtype dtype, int rank, void* out,
                                mr_stream stream);

/*
 * mr_allreduce_sum_noalloc -- mr_allreduce_sum that never allocates device memory, for callers that
 * cannot allocate: code under HIP graph capture, serving loops that must not allocate, harnesses that
 * forbid it.
 *
 * Same arguments, result bits and errors as mr_allreduce_sum, with these differences:
 *  - the two-shot workspace is a device array inside the library (MR_NOALLOC_MAX_BYTES of stage plus
 *    the barrier words, about 34 MiB per GPU), held by each GPU the library runs on until the process
 *    ends; the first call on a device looks its address up and clears it on `stream`;
 *  - a rank buffer larger than MR_NOALLOC_MAX_BYTES (n * element size) -> MR_ERR_WORKSPACE, nothing
 *    enqueued;
 *  - the two-shot hand-off is always the last arriver (on XCD-local units on the 16-byte path with
 *    W <= 8, else on chunk tiles), ignoring MR_OPT_TWOSHOT_SYNC and
 *    MR_OPT_TILE_SHAPE: no workgroup of it ever waits, so it never leaves a barrier word set after a
 *    launch and never produces an invalid output; there is no error word to check;
 *  - every call on one GPU shares that GPU's array: two-shot calls that overlap in time on one GPU (on
 *    two streams, or from two host threads) race and give undefined output.  One-shot calls use no
 *    workspace and never race.
 */
#define MR_NOALLOC_MAX_BYTES ((size_t)32 << 20)
mr_status mr_allreduce_sum_noalloc(const void* const* bufs, int W, size_t n, mr_dtype dtype, void* out,
                                   mr_mode mode, mr_stream stream);

/*
 * All-gathers from W separate rank shards (each a device buffer of T elements), one launch each.
 * Bit copies of any dtype; 1 <= W <= MR_MAX_TABLE_W; shards may not overlap any output (MR_ERR_ALIAS).
 * Shard and output pointers may have any alignment (as for mr_allgather_param_contig).
 *
 * mr_allgather_into_tensor:  rank-major gather (torch.distributed.all_gather_into_tensor's layout):
 *                            out[r*T + j] = shards[r][j]; out holds W*T elements.
 * mr_allgather_list:         list-output gather (torch.distributed.all_gather's layout, page "ccl:
 *                            hierarchical cross-node AllGather ...", the commit adding the list-output
 *                            all_gather): outs[r][j] = shards[r][j]; outs is a host array of W device
 *                            buffers of T elements that may not overlap one another.
 * mr_allgather_param_contig_shards: the param-contiguous placement of mr_allgather_param_contig
 *                            written straight from the W shards, with no rank-major intermediate (the
 *                            zero-copy push of enqueue_param_contiguous on the same page):
 *                            out[O_s*W + r*splits[s] + j] = shards[r][O_s + j].
 */
mr_status mr_allgather_into_tensor(const void* const* shards, int W, size_t T, mr_dtype dtype, void* out,
                                   mr_stream stream);
mr_status mr_allgather_list(const void* const* shards, int W, size_t T, mr_dtype dtype, void* const* outs,
                            mr_stream stream);
mr_status mr_allgather_param_contig_shards(const void* const* shards, int W, int G, const uint64_t* splits, int P,
                                           mr_dtype dtype, void* out, mr_stream stream);

/*
 * Two-shot workspace.
 *
 * By default the library allocates, on first two-shot use of a (device, stream) pair, a grow-only
 * workspace of at least mr_workspace_bytes() bytes holding the stage buffer and the barrier words.
 * Growth at least doubles the size and keeps the replaced buffer alive, so launches in flight and HIP
 * graphs that captured a two-shot call on the stream stay valid; replaced buffers are freed only by
 * mr_set_workspace on that stream.  One workspace per (device, stream): eager two-shot calls on
 * different streams never share barrier words.
 *
 * A two-shot call made while its stream is being captured into a HIP graph uses a library-owned
 * workspace of that capture (device, stream, capture id), allocated during the capture with this
 * thread's capture mode relaxed for the allocation and cleared by a kernel recorded into the graph.  So
 * graphs captured one after another on one stream -- torch.cuda.graph captures every graph on one
 * shared stream -- never share barrier words, and may be replayed at the same time on different
 * streams.  Two replays of the same graph that overlap in time do share its workspace and race.  These
 * workspaces live until mr_set_workspace is called on the capture stream (destroy the graphs first).
 * Caller-owned memory bound with mr_set_workspace is used for captured calls too.
 *
 * Every launch returns its barrier words and flags to zero before it ends, also when a bounded wait
 * gave up (the call that timed out has invalid output; later calls are unaffected).
 *
 * mr_workspace_bytes: bytes a caller-owned workspace needs for a two-shot call of this shape.
 * mr_set_workspace:   bind caller-owned device memory (256-byte aligned) as the workspace of `stream`
 *                     on the current device, replacing any library-owned one; the barrier words and
 *                     flags are cleared on `stream` here.  Memory too small to hold them plus some
 *                     stage -> MR_ERR_INVALID_ARG; a bound workspace too small for a later call makes
 *                     that call return MR_ERR_WORKSPACE.  dev_ptr == NULL unbinds (the library
 *                     allocates again on next use).  Either way it synchronises `stream` and frees
 *                     every library-owned workspace buffer of the stream (its captures' included), so
 *                     a graph that captured a two-shot call on it must not be replayed afterwards.
 *                     If a free fails, the call returns MR_ERR_HIP and leaves the stream with no
 *                     workspace bound.  Not thread-safe against concurrent calls on that stream.
 * mr_workspace_check: synchronises `stream`, then reads and clears the barrier error words of its
 *                     workspaces (its own and those of graphs captured on it).  *flags receives their
 *                     OR: 0 = no error; bit 0 = a phase-2 workgroup gave up waiting for phase 1, so
 *                     that call's output is not valid; bits 1 and 2 = the XCD-local two-shot
 *                     recomputed units from the rank buffers (after a wait gave up / because a
 *                     unit's producer ran on another XCD than the workgroup that copies it), output
 *                     valid.  Returns MR_ERR_WORKSPACE if
 *                     there is no workspace for the stream.
 */
size_t mr_workspace_bytes(int W, size_t n, mr_dtype dtype);
mr_status mr_set_workspace(mr_stream stream, void* dev_ptr, size_t bytes);
mr_status mr_workspace_check(mr_stream stream, uint32_t* flags);

/*
 * Process-wide options (thread-safe; they apply to calls made after the change).
 *
 * MR_OPT_TWOSHOT_SYNC  how a two-shot phase-2 tile waits for phase 1 (all give identical results):
 *   MR_TWOSHOT_SYNC_AUTO  (default) LAST up to 32 MiB per rank buffer, TILE above;
 *   MR_TWOSHOT_SYNC_TILE  per-tile producer flags: a phase-2 tile waits only for the
 *                         phase-1 tiles it copies (the per-block flag hand-off of the custom
 *                         allreduce page's block_barrier, applied to the two phases);
 *   MR_TWOSHOT_SYNC_CHUNK per-chunk barrier: waits for every phase-1 tile of its 1/W chunk;
 *   MR_TWOSHOT_SYNC_GRID  grid barrier: waits for every phase-1 tile of every chunk;
 *   MR_TWOSHOT_SYNC_LAST  no waiting: each group of phase-1 tiles counts its releases, and the
 *                         workgroup whose release completes the group copies it.
 *   Under TILE (16 to 64 MiB per rank buffer) and LAST (any size) the 16-byte path with W <= 8 runs
 *   on XCD-local units (16 KiB of output each from 8 MiB per rank buffer, 4 or 1 KiB below; one run
 *   per XCD) unless MR_OPT_TILE_SHAPE forces a tile shape; otherwise on W chunks.
 * MR_OPT_SPIN_LIMIT    polls a waiting workgroup makes before it gives up and sets the workspace error
 *                      word (see mr_workspace_check); default 2^22.  A value of 0 makes every wait
 *                      that is not already satisfied give up at once (for testing error handling).
 * MR_OPT_TILE_SHAPE    tile shape of the sum-reduce kernels (results are identical for every shape):
 *   MR_TILE_AUTO   (default) chosen from the message size and dtype: narrow below 64 Ki packs
 *                  of 16 B, medium below 256 Ki (fp32) or 512 Ki (16-bit types) packs,
 *                  MR_TILE_WIDE_PAIR from 1 Mi to 4 Mi packs (16 to 64 MiB per rank buffer) when
 *                  W <= 8, wide otherwise; two-shot: 64-pack tiles below 8 Ki packs, 256 below 128 Ki, 1024 above;
 *   MR_TILE_WIDE   one-shot 256 lanes x 4 packs of 16 B (256 x 1 for W > 8), two-shot phase-1
 *                  tiles of 1024 packs;
 *   MR_TILE_MEDIUM one-shot 256 x 1, two-shot 256-pack tiles;
 *   MR_TILE_NARROW one-shot 64 x 1, two-shot 64-pack tiles;
 *   MR_TILE_WIDE_PAIR  one-shot: wide tiles pipelined on a persistent grid of resident workgroups,
 *                  each storing one tile's sums while the next tile's loads are in flight (W <= 8;
 *                  wide for W > 8); two-shot under TILE or LAST: XCD-local units at any size
 *                  (W <= 8, 16-byte path), otherwise as MR_TILE_WIDE.
 * MR_OPT_SDMA_CU_BELOW mr_allgather_param_contig_sdma: a parameter whose per-rank piece is smaller than
 *                      this many bytes is copied by the compute-unit kernel, the others by the engines;
 *                      0 puts every piece on the engines.  0 .. 2^32-1, default 1048576 (1 MiB).  The
 *                      kernel part needs free compute units: beside a kernel that holds them all, the
 *                      call returns only after that kernel has made room, so a caller that must not
 *                      wait on other work sets 0.
 * Unknown options or out-of-range values -> MR_ERR_INVALID_ARG.  Environment variables
 * MR_TWOSHOT_SYNC, MR_SPIN_LIMIT, MR_TILE_SHAPE and MR_SDMA_CU_BELOW set the initial values when the
 * library loads; a value that is not a whole number in the option's range is ignored.  MR_TRACE=1 makes
 * every launch print its plan (path, shape, grid) to stderr.
 */
typedef enum mr_option {
  MR_OPT_TWOSHOT_SYNC = 0,
  MR_OPT_SPIN_LIMIT = 1,
  MR_OPT_TILE_SHAPE = 2,
  MR_OPT_SDMA_CU_BELOW = 3
} mr_option;
#define MR_TWOSHOT_SYNC_TILE 0
#define MR_TWOSHOT_SYNC_CHUNK 1
#define MR_TWOSHOT_SYNC_GRID 2
#define MR_TWOSHOT_SYNC_LAST 3
#define MR_TWOSHOT_SYNC_AUTO 4
#define MR_TILE_AUTO 0
#define MR_TILE_WIDE 1
#define MR_TILE_MEDIUM 2
#define MR_TILE_NARROW 3
#define MR_TILE_WIDE_PAIR 4
mr_status mr_set_option(mr_option opt, int64_t value);
mr_status mr_get_option(mr_option opt, int64_t* value);

/* Library ABI version (major*100 + minor).  1.01 added MR_OPT_TILE_SHAPE, MR_TWOSHOT_SYNC_LAST and
 * MR_TWOSHOT_SYNC_AUTO (the new default hand-off); 1.02 added MR_TILE_WIDE_PAIR; 1.03 added
 * mr_allgather_param_contig_sdma, mr_sdma_engines and MR_ERR_ENGINE; 1.04 added
 * mr_allreduce_sum_noalloc and the last-arriver hand-off on XCD-local units (the default up to 32 MiB
 * per rank buffer); 1.05 added MR_OPT_SDMA_CU_BELOW (small parameters of the SDMA gather on the
 * compute units). */
int mr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MR_H_ */
