// Measurement kernels (declared in mr_probe.h, outside the C ABI of include/mr.h): the one-shot
// reduce's HBM access pattern with the arithmetic replaced by an XOR, so that the reduce's rate can be
// set beside the rate of K read streams plus one write stream on the same buffers in the same run.

#include "mr_internal.h"
#include "mr_probe.h"

namespace mr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Streams {
  const u32x4* p[8];
};

constexpr int kProbeBlock = 256;
constexpr int kProbeU = 4;  // 16-byte words per lane per stream

template <int K, bool WR>
__global__ __launch_bounds__(kProbeBlock) void stream_mix(Streams in, u32x4* out, size_t nwords) {
  const size_t first = static_cast<size_t>(blockIdx.x) * (kProbeBlock * kProbeU) +
                       static_cast<size_t>(threadIdx.x >> 6) * (64 * kProbeU) + (threadIdx.x & 63);
  u32x4 v[kProbeU][K];
#pragma unroll
  for (int r = 0; r < K; ++r)
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      const size_t i = first + static_cast<size_t>(u) * 64;
      if (i < nwords) v[u][r] = __builtin_nontemporal_load(in.p[r] + i);
    }
#pragma unroll
  for (int u = 0; u < kProbeU; ++u) {
    const size_t i = first + static_cast<size_t>(u) * 64;
    if (i < nwords) {
      u32x4 x = v[u][0];
#pragma unroll
      for (int r = 1; r < K; ++r) x ^= v[u][r];
      if (WR || (x[0] == 0x9e3779b9u && x[1] == 0x7f4a7c15u)) __builtin_nontemporal_store(x, out + i);
    }
  }
}

// The same streams on the pipelined one-shot's schedule: a persistent grid of resident workgroups, each
// walking tiles b, b + grid, ... and issuing a tile's loads before it stores the previous tile's XOR.
template <int K>
__global__ __launch_bounds__(kProbeBlock) void stream_mix_pipe(Streams in, u32x4* out, size_t nwords, size_t ntiles) {
  constexpr size_t kTile = kProbeBlock * kProbeU;
  const size_t lane = static_cast<size_t>(threadIdx.x >> 6) * (64 * kProbeU) + (threadIdx.x & 63);
  const size_t nfull = nwords / kTile;  // full tiles: no per-lane bounds checks, as in the one-shot
  u32x4 held[kProbeU];
  size_t prev = ~size_t(0);
  size_t t = blockIdx.x;
  for (; t < nfull; t += gridDim.x) {
    const size_t first = t * kTile + lane;
    u32x4 v[kProbeU][K];
#pragma unroll
    for (int r = 0; r < K; ++r)
#pragma unroll
      for (int u = 0; u < kProbeU; ++u) v[u][r] = __builtin_nontemporal_load(in.p[r] + first + static_cast<size_t>(u) * 64);
    __asm__ volatile("" ::: "memory");
    if (prev != ~size_t(0)) {
#pragma unroll
      for (int u = 0; u < kProbeU; ++u) __builtin_nontemporal_store(held[u], out + prev + static_cast<size_t>(u) * 64);
    }
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      u32x4 x = v[u][0];
#pragma unroll
      for (int r = 1; r < K; ++r) x ^= v[u][r];
      held[u] = x;
    }
    prev = first;
  }
  if (prev != ~size_t(0)) {
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) __builtin_nontemporal_store(held[u], out + prev + static_cast<size_t>(u) * 64);
  }
  if (t < ntiles) {  // the partial last tile, checked
    const size_t first = t * kTile + lane;
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      const size_t i = first + static_cast<size_t>(u) * 64;
      if (i < nwords) {
        u32x4 x = in.p[0][i];
#pragma unroll
        for (int r = 1; r < K; ++r) x ^= in.p[r][i];
        __builtin_nontemporal_store(x, out + i);
      }
    }
  }
}

template <int K>
hipError_t launch_k(const Streams& s, u32x4* out, size_t nwords, int write, hipStream_t st) {
  const size_t tiles = (nwords + kProbeBlock * kProbeU - 1) / (kProbeBlock * kProbeU);
  const dim3 block(kProbeBlock);
  if (write == 2) {
    const size_t resident = resident_workgroups(stream_mix_pipe<K>, kProbeBlock);
    const size_t grid = resident && resident < tiles ? resident : tiles;
    hipLaunchKernelGGL((stream_mix_pipe<K>), dim3(static_cast<unsigned>(grid)), block, 0, st, s, out, nwords, tiles);
  } else if (write) {
    hipLaunchKernelGGL((stream_mix<K, true>), dim3(static_cast<unsigned>(tiles)), block, 0, st, s, out, nwords);
  } else {
    hipLaunchKernelGGL((stream_mix<K, false>), dim3(static_cast<unsigned>(tiles)), block, 0, st, s, out, nwords);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace mr

extern "C" int mrx_stream_mix(const void* const* reads, int K, void* out, size_t bytes, int write, void* stream) {
  if (K < 1 || K > 8 || !reads || !out || bytes % 16 != 0 || write < 0 || write > 2) return -1;
  if (bytes == 0) return 0;
  const size_t nwords = bytes / 16;
  if ((nwords + 1023) / 1024 >= (size_t(1) << 31)) return -1;
  mr::Streams s{};
  for (int r = 0; r < K; ++r) {
    if (!reads[r] || reinterpret_cast<uintptr_t>(reads[r]) % 16 != 0) return -1;
    s.p[r] = static_cast<const mr::u32x4*>(reads[r]);
  }
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return -1;
  mr::u32x4* o = static_cast<mr::u32x4*>(out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (K) {
    case 1: e = mr::launch_k<1>(s, o, nwords, write, st); break;
    case 2: e = mr::launch_k<2>(s, o, nwords, write, st); break;
    case 3: e = mr::launch_k<3>(s, o, nwords, write, st); break;
    case 4: e = mr::launch_k<4>(s, o, nwords, write, st); break;
    case 5: e = mr::launch_k<5>(s, o, nwords, write, st); break;
    case 6: e = mr::launch_k<6>(s, o, nwords, write, st); break;
    case 7: e = mr::launch_k<7>(s, o, nwords, write, st); break;
    default: e = mr::launch_k<8>(s, o, nwords, write, st); break;
  }
  return static_cast<int>(e);
}
