// mr_allreduce_sum_noalloc: the sum all-reduce with its two-shot workspace in a file-scope device
// array, for callers that cannot allocate device memory (code under HIP graph capture, serving loops
// that must not allocate, harnesses that forbid it).
//
// The array (`scratch`) holds what the library's per-stream workspace holds: the barrier words, the
// producer flags and the stage.  Each GPU the library runs on has its own copy for as long as the
// process lives.  In host code the array's name is only a host-side stand-in, so the device address of
// each GPU's copy is looked up once per device with hipGetSymbolAddress (with that device current) and
// only that address is used afterwards.  The two-shot kernels return every barrier word and flag to
// zero by the end of each launch under the hand-offs this entry point allows (the last arriver, which
// never waits, and the XCD-local units, which recompute a unit instead of failing a wait), so the
// array only needs clearing once, at set-up; the stage keeps the last call's sums, which no call reads
// before writing.  All calls on one GPU share its array: two two-shot calls that overlap in time on one
// GPU (two streams, or two host threads) race on it.

#include <mutex>

#include "mr_internal.h"

namespace {

// Two-shot of up to MR_NOALLOC_MAX_BYTES per rank buffer: the workspace layout of that size fits
// (barrier words 16 KiB, one flag word per 256 bytes, stage, 256 bytes of alignment slack).
constexpr size_t kScratchBytes = size_t(34) << 20;
static_assert(MR_NOALLOC_MAX_BYTES == (size_t(32) << 20), "limit documented in mr.h");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once set up

// The device address of this device's array, cleared on `st` the first time (0 on success, else the
// hipError_t of the lookup or the clear).
hipError_t scratch_for(int dev, hipStream_t st, char** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    e = mr::clear_workspace_words(static_cast<char*>(p), kScratchBytes, st);
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" mr_status mr_allreduce_sum_noalloc(const void* const* bufs, int W, size_t n, mr_dtype dtype, void* out,
                                              mr_mode mode, mr_stream stream) {
  const mr_status s = mr::check_allreduce_args(bufs, W, n, dtype, out, mode);
  if (s != MR_OK || n == 0) return s;
  if (n * static_cast<size_t>(mr::elem_size(dtype)) > MR_NOALLOC_MAX_BYTES) return MR_ERR_WORKSPACE;
  if (mr::workspace_bytes_for(n, mr::elem_size(dtype)) > kScratchBytes) return MR_ERR_WORKSPACE;  // not reached
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) return MR_ERR_INVALID_ARG;
  char* base = nullptr;
  if (e == hipSuccess) e = scratch_for(dev, st, &base);
  if (e != hipSuccess) {
    mr::set_last_hip_error(static_cast<int>(e));
    return MR_ERR_HIP;
  }
  return mr::allreduce_in_workspace(bufs, W, n, dtype, out, mode, st, base, kScratchBytes);
}
