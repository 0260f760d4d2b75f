/*
 * mr_probe.h -- entry points of libmr that are not part of its C ABI (include/mr.h).
 *
 * A measurement kernel, which bounds what the reduce can reach on the machine it runs on (so that a
 * benchmark can report the reduce's rate beside the rate of the plain access pattern it is made of,
 * measured in the same process on the same buffers), and planning hooks through which host-side tests
 * check the library's own launch plans against brute force.  None of them launches work except
 * mrx_stream_mix.
 */
#ifndef MR_PROBE_H_
#define MR_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mrx_stream_mix -- K read streams and optionally one write stream, with the one-shot reduce's
 * access pattern and none of its arithmetic.
 *
 * reads   host array of K device pointers (1 <= K <= 8), each to `bytes` bytes, 16-byte aligned.
 * out     device pointer to `bytes` bytes, 16-byte aligned.  With write 1 or 2 every 16-byte word of
 *         out receives the XOR of the K words at the same offset; with write == 0 the kernel loads
 *         the K streams and stores a word only where the XOR equals one fixed 64-bit pattern (so the
 *         loads cannot be dropped), which leaves out unspecified but within its bytes.
 * bytes   a multiple of 16; 0 is a no-op.
 * write   0: reads only; 1: reads and the write, one tile per workgroup; 2: reads and the write on
 *         the pipelined one-shot's schedule (a persistent grid of resident workgroups, each issuing a
 *         tile's loads before storing the previous tile's XOR).  Other values -> -1.
 * Lane layout: 256-lane workgroups, each lane four 16-byte words per stream (1024 words per tile,
 * wave-contiguous), every load of a lane in flight before the XOR, non-temporal loads and stores --
 * the wide one-shot tile.  Returns 0 (hipSuccess), the hipError_t of a failed launch, or -1 for
 * invalid arguments (nothing is enqueued then).
 */
int mrx_stream_mix(const void* const* reads, int K, void* out, size_t bytes, int write, void* stream);

/*
 * mrx_twoshot_plan -- the plan mr_allreduce_sum would launch for a two-shot call: W rank buffers of n
 * elements of `dtype`, out at address out_addr, all pointers at out's 16-byte phase if same_phase,
 * options sync_opt / shape_opt (MR_TWOSHOT_SYNC_*, MR_TILE_*), wait_free as mr_allreduce_sum_noalloc.
 * f[0..15] receive: xcd, units, run, run_padded, chunks, chunk_units, t1, t2, ratio, unit1 (packs per
 * phase-1 tile, or per XCD-local unit when xcd is 1), sync, vec, head, npacks, grid (workgroups), flag
 * words used.  Returns 0, or -1 for invalid arguments.
 */
int mrx_twoshot_plan(int W, size_t n, int dtype, uintptr_t out_addr, int same_phase, int sync_opt, int shape_opt,
                     int wait_free, uint64_t* f, int nf);

/*
 * mrx_reduce_shape -- how mr_allreduce_sum would lay out a call on these pointers: f[0] vec (16-byte
 * path), f[1] realign (some input in another 16-byte phase than out), f[2] bytes (a pointer off the
 * element grid: byte accesses only), f[3] head elements before out's 16-byte boundary, f[4] packs,
 * f[5 + r] rank r's phase past out's, (bufs[r] - out) mod 16.  Needs nf >= 5 + MR_MAX_W (21).
 */
int mrx_reduce_shape(const void* const* bufs, int W, size_t n, int dtype, const void* out, uint64_t* f, int nf);

/*
 * mrx_gather_phase_masks -- the 16-bit phase masks the gather planner keeps for a split table: bit
 * (dst_off - src_off) mod 16 of every (parameter, rank) piece, for a rank-major source (*rm_mask) and
 * for per-rank shard sources (rank_masks[r], r < n_rank_masks, W <= 64).  Returns 0 or an mr_status.
 * mrx_needs_realign -- whether a mask requires the realigning kernel build for a given source - out
 * base-address difference.
 */
int mrx_gather_phase_masks(int W, int G, const uint64_t* splits, int P, int dtype, uint16_t* rm_mask,
                           uint16_t* rank_masks, int n_rank_masks);
int mrx_needs_realign(uint16_t mask, uint64_t base_difference);

/*
 * mrx_gather_tiles -- the tile table the gather planner builds for a split table of at most 128
 * parameters when only parameters whose per-rank piece is smaller than cu_below bytes are copied by the
 * kernel (the SDMA gather's compute-unit part; UINT64_MAX: every parameter): prefix[s] = tiles of the
 * parameters before s, s = 0..P (n_prefix >= P + 1), and *rm_mask the rank-major phase mask over those
 * parameters' pieces.  Returns 0 or an mr_status (-1 for a table too small or P > 128).
 */
int mrx_gather_tiles(int W, int G, const uint64_t* splits, int P, int dtype, uint64_t cu_below, uint32_t* prefix,
                     int n_prefix, uint16_t* rm_mask);

#ifdef __cplusplus
}
#endif

#endif /* MR_PROBE_H_ */
