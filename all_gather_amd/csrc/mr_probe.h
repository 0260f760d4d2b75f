/*
 * mr_probe.h -- measurement kernels of libmr that are not part of its C ABI (include/mr.h).
 *
 * They bound what the reduce can reach on the machine it runs on, so that a benchmark can report
 * the reduce's rate beside the rate of the plain access pattern it is made of, measured in the same
 * process on the same buffers.
 */
#ifndef MR_PROBE_H_
#define MR_PROBE_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mrx_stream_mix -- K read streams and optionally one write stream, with the one-shot reduce's
 * access pattern and none of its arithmetic.
 *
 * reads   host array of K device pointers (1 <= K <= 8), each to `bytes` bytes, 16-byte aligned.
 * out     device pointer to `bytes` bytes, 16-byte aligned.  With write != 0 every 16-byte word of
 *         out receives the XOR of the K words at the same offset; with write == 0 the kernel loads
 *         the K streams and stores a word only where the XOR equals one fixed 64-bit pattern (so the
 *         loads cannot be dropped), which leaves out unspecified but within its bytes.
 * bytes   a multiple of 16; 0 is a no-op.
 * Lane layout: 256-lane workgroups, each lane four 16-byte words per stream (1024 words per
 * workgroup, wave-contiguous), every load of a lane in flight before the XOR, non-temporal loads and
 * stores -- the wide one-shot tile.  Returns 0 (hipSuccess), the hipError_t of a failed launch, or -1
 * for invalid arguments (nothing is enqueued then).
 */
int mrx_stream_mix(const void* const* reads, int K, void* out, size_t bytes, int write, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MR_PROBE_H_ */
