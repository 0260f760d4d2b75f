// Fused param-contiguous scatter for gfx950: rank-major [W][T] -> [param][rank], one launch.
//
// Page "ccl: hierarchical cross-node AllGather (intra-node SDMA + inter-node RDMA) #441": the commit
// adding enqueue_param_contiguous places node-block m of parameter s at O_s*W + m*G*E_s with slot
// stride E_s (rank r = m*G + g lands at O_s*W + r*E_s); the commit after it replaces the
// N_nodes x N_params launches with one kernel that loops over node-blocks and splits.  Here one launch
// covers every (node-block, parameter, slot) segment: the host cuts each segment into 16 KiB tiles and
// puts a per-parameter tile prefix in the kernel arguments; a workgroup maps its tile index back to
// (m, s, g, k) with a scalar binary search and copies the tile.  The copy is a bit copy with 64-bit
// offsets; 16-byte loads and stores when source and destination share the same 16-byte phase.

#include "mr_internal.h"

namespace mr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyU = kGatherTileBytes / (16 * kBlock);  // 16-byte words per lane per tile (4)
static_assert(kCopyU * 16 * kBlock == kGatherTileBytes, "tile must be a whole number of block sweeps");

// Copy `len` bytes, src and dst at the same offset modulo 16 (or any offsets on the narrow path).
__device__ __forceinline__ void copy_span(const char* src, char* dst, uint32_t len, uint32_t elem) {
  const uintptr_t ps = reinterpret_cast<uintptr_t>(src), pd = reinterpret_cast<uintptr_t>(dst);
  if (((ps ^ pd) & 15u) == 0) {
    // same phase: element-wise head up to 16-byte alignment, 16-byte body, element-wise tail
    uint32_t head = static_cast<uint32_t>((16u - (ps & 15u)) & 15u);
    if (head > len) head = len;
    const uint32_t body = (len - head) & ~15u;
    const uint32_t nw = body >> 4;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + head);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst + head);
    u32x4 v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t i = u * kBlock + threadIdx.x;
      if (i < nw) v[u] = __builtin_nontemporal_load(s4 + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t i = u * kBlock + threadIdx.x;
      if (i < nw) __builtin_nontemporal_store(v[u], d4 + i);
    }
    // head bytes [0, head) and tail bytes [head + body, len), in whole elements
    const uint32_t tail0 = head + body;
    const uint32_t edge = head + (len - tail0);
    for (uint32_t b = threadIdx.x * elem; b < edge; b += kBlock * elem) {
      const uint32_t o = b < head ? b : tail0 + (b - head);
      if (elem == 2)
        *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
      else
        *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
    }
  } else {
    // different phases: element copies (rare: odd split sizes with 2-byte elements)
    for (uint32_t b = threadIdx.x * elem; b < len; b += kBlock * elem) {
      if (elem == 2)
        *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
      else
        *reinterpret_cast<uint32_t*>(dst + b) = *reinterpret_cast<const uint32_t*>(src + b);
    }
  }
}

__global__ __launch_bounds__(kBlock) void param_contig(GatherArgs a) {
  for (uint32_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
    // tile -> node-block m, parameter s, slot g, tile k of that (m, s, g) segment (uniform per block)
    const uint32_t m = t / a.tiles_per_block;
    const uint32_t in_block = t - m * a.tiles_per_block;
    uint32_t lo = 0, hi = a.P;  // find s with tile_prefix[s] <= in_block < tile_prefix[s+1]
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (a.tile_prefix[mid] <= in_block) lo = mid; else hi = mid;
    }
    const uint32_t s = lo;
    const uint32_t per_slot = (a.tile_prefix[s + 1] - a.tile_prefix[s]) / a.G;
    const uint32_t local = in_block - a.tile_prefix[s];
    const uint32_t g = local / per_slot;
    const uint32_t k = local - g * per_slot;

    const uint64_t Os = a.O[s];
    const uint64_t Es = a.O[s + 1] - Os;
    const uint64_t r = static_cast<uint64_t>(m) * a.G + g;
    const uint64_t dst_block = Os * a.W + static_cast<uint64_t>(m) * a.G * Es;  // node-block m of param s
    const uint64_t dst_elem = dst_block + static_cast<uint64_t>(g) * Es;         // slot g, stride E_s
    const uint64_t src_elem = r * a.T + Os;

    const uint64_t seg_bytes = Es * a.elem;
    const uint64_t b0 = static_cast<uint64_t>(k) * kGatherTileBytes;
    const uint64_t rem = seg_bytes - b0;
    const uint32_t len = rem < kGatherTileBytes ? static_cast<uint32_t>(rem) : kGatherTileBytes;
    copy_span(a.src + src_elem * a.elem + b0, a.out + dst_elem * a.elem + b0, len, a.elem);
  }
}

}  // namespace

hipError_t launch_param_contig(const GatherArgs& a, hipStream_t st) {
  if (a.total_tiles == 0) return hipSuccess;
  const uint32_t kMaxGrid = 1u << 22;
  const uint32_t grid = a.total_tiles < kMaxGrid ? a.total_tiles : kMaxGrid;
  hipLaunchKernelGGL(param_contig, dim3(grid), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace mr
