// Fused param-contiguous scatter for gfx950: rank-major [W][T] -> [param][rank], one launch.
// (Per-parameter tiles for param-major destinations: see param_block_tile.)
//
// Page "ccl: hierarchical cross-node AllGather (intra-node SDMA + inter-node RDMA) #441": the commit
// adding enqueue_param_contiguous places node-block m of parameter s at O_s*W + m*G*E_s with slot
// stride E_s (rank r = m*G + g lands at O_s*W + r*E_s); the commit after it replaces the
// N_nodes x N_params launches with one kernel that loops over node-blocks and splits.  Here one launch
// covers every (node-block, parameter, slot) segment: the host gives each segment of parameter s the
// same number of 16 KiB tiles and puts a per-parameter tile prefix in the kernel arguments; a
// workgroup maps its tile index back to (m, s, g, k) with a scalar binary search and copies the tile.
// Tile boundaries fall on 256-byte lines of the destination, so two workgroups never write parts of
// one line (a partial line costs a full one: aligning them cut the scatter's time by about 4%).
// 512-lane workgroups moving 16 KiB (two 16-byte words per lane) measured best among 256..1024 lanes
// and 8..128 KiB tiles.  The copy is a bit copy with 64-bit offsets; 16-byte non-temporal loads and
// stores when source and destination share the same 16-byte phase, else 4-byte (or 2-byte) words with
// the whole tile's loads in flight before its stores.

#include "mr_internal.h"

namespace mr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGB = kGatherBlock;
constexpr int kCopyU = kGatherTileBytes / (16 * kGB);  // 16-byte words per lane per full tile
static_assert(kCopyU * 16 * kGB == kGatherTileBytes, "a tile is a whole number of workgroup sweeps");

template <int S>
__device__ __forceinline__ void copy_elem(const char* src, char* dst, uint32_t o) {
  if (S == 2) *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
  else *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
}

// Copy `n` words of type Wd (src and dst both Wd-aligned), a whole tile's loads in flight before its
// stores: the path for spans whose source and destination have different 16-byte phases.
template <typename Wd>
__device__ __forceinline__ void copy_words(const char* src, char* dst, uint32_t n) {
  constexpr int U = kGatherTileBytes / (static_cast<int>(sizeof(Wd)) * kGB);  // words per lane per tile
  const Wd* s = reinterpret_cast<const Wd*>(src);
  Wd* d = reinterpret_cast<Wd*>(dst);
  for (uint32_t w0 = 0; w0 < n; w0 += U * kGB) {
    Wd v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = w0 + u * kGB + threadIdx.x;
      if (i < n) v[u] = __builtin_nontemporal_load(s + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = w0 + u * kGB + threadIdx.x;
      if (i < n) __builtin_nontemporal_store(v[u], d + i);
    }
  }
}

// Copy `len` (<= one tile) bytes of whole elements.
template <int S>
__device__ __forceinline__ void copy_span(const char* src, char* dst, uint32_t len) {
  const uintptr_t ps = reinterpret_cast<uintptr_t>(src), pd = reinterpret_cast<uintptr_t>(dst);
  if (((ps ^ pd) & 15u) == 0) {
    // same 16-byte phase: element-wise head up to 16-byte alignment, 16-byte body, element-wise tail
    uint32_t head = static_cast<uint32_t>((16u - (ps & 15u)) & 15u);
    if (head > len) head = len;
    const uint32_t body = (len - head) & ~15u;
    const uint32_t nw = body >> 4;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + head);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst + head);
    for (uint32_t w0 = 0; w0 < nw; w0 += kCopyU * kGB) {
      u32x4 v[kCopyU];
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) {
        const uint32_t i = w0 + u * kGB + threadIdx.x;
        if (i < nw) v[u] = __builtin_nontemporal_load(s4 + i);
      }
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) {
        const uint32_t i = w0 + u * kGB + threadIdx.x;
        if (i < nw) __builtin_nontemporal_store(v[u], d4 + i);
      }
    }
    const uint32_t tail0 = head + body;
    const uint32_t edge = head + (len - tail0);
    for (uint32_t b = threadIdx.x * S; b < edge; b += kGB * S) copy_elem<S>(src, dst, b < head ? b : tail0 + (b - head));
  } else if (((ps ^ pd) & 3u) == 0) {
    // different 16-byte phases, same 4-byte phase (split sizes that are not a multiple of the pack):
    // a 2-byte element up to 4-byte alignment, 4-byte words, a 2-byte element at the end
    const uint32_t head = (S == 2 && (ps & 2u) && len >= 2) ? 2u : 0u;
    if (head && threadIdx.x == 0) copy_elem<2>(src, dst, 0);
    const uint32_t nw = (len - head) >> 2;
    copy_words<uint32_t>(src + head, dst + head, nw);
    const uint32_t tail0 = head + (nw << 2);
    if (tail0 < len && threadIdx.x == 0) copy_elem<2>(src, dst, tail0);
  } else {
    // 2-byte elements whose 4-byte phases differ: 2-byte words
    copy_words<uint16_t>(src, dst, len >> 1);
  }
}

// Param-major destination: the W slots of parameter s are contiguous in out (W*E_s elements from
// O_s*W), so tiles are cut per parameter over that whole block and a tile crossing a rank boundary
// switches source row mid-tile.  Same-GPU A/B against tiles cut per (node-block, parameter, slot)
// segment, three interleaved repeats: config 4 (W=8, G=4, P=64 log-uniform) bf16 158 -> 154 us, fp32
// 304 -> 298 us, from separate shards bf16 153 -> 150 us; equal fp32 splits at the same size, P=32
// 300 -> 293 us, P=128 315 -> 303 us (W*P partial tiles become P).
template <int S>
__device__ __forceinline__ void param_block_tile(const GatherArgs& a, uint32_t t) {
  uint32_t lo = 0, hi = a.P;  // parameter s with tile_prefix[s] <= t < tile_prefix[s+1]
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (a.tile_prefix[mid] <= t) lo = mid; else hi = mid;
  }
  const uint32_t s = lo;
  const uint32_t k = t - a.tile_prefix[s];
  const uint64_t Os = a.O[s];
  const uint64_t ES = (a.O[s + 1] - Os) * S;  // bytes of one rank's piece of parameter s
  char* pd = a.out + Os * a.W * S;            // the parameter's block: slot r at r*ES
  const uint64_t seg = ES * a.W;
  // tiles end on 256-byte lines of the destination (the block's lead offset shifts them)
  const uint64_t lead = reinterpret_cast<uintptr_t>(pd) & (kGatherLine - 1);
  const uint64_t b0r = static_cast<uint64_t>(k) * kGatherTileBytes;
  const uint64_t b0 = b0r > lead ? b0r - lead : 0;
  const uint64_t b1r = b0r + kGatherTileBytes - lead;
  const uint64_t b1 = b1r < seg ? b1r : seg;
  for (uint64_t x = b0; x < b1;) {  // one piece per rank the tile touches (rank r = m*G + g)
    const uint64_t r = x / ES;
    const uint64_t xe = (r + 1) * ES < b1 ? (r + 1) * ES : b1;
    const char* sp = a.src_table ? a.src_tab[r] + Os * S : a.src + (r * a.T + Os) * S;
    copy_span<S>(sp + (x - r * ES), pd + x, static_cast<uint32_t>(xe - x));
    x = xe;
  }
}

template <int S>
__global__ __launch_bounds__(kGB) void param_contig(GatherArgs a) {
  if (a.span) {
    for (uint32_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) param_block_tile<S>(a, t);
    return;
  }
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
    // source: rank r's shard, inside the rank-major buffer or from the shard table
    const char* sp = a.src_table ? a.src_tab[r] + Os * S : a.src + (r * a.T + Os) * S;
    // destination: the [param][rank] slot, or rank r's own output (list-output all-gather)
    char* dp = a.dst_table ? a.dst_tab[r] + Os * S : a.out + dst_elem * S;
    // tiles of the segment end on 256-byte lines of the destination: tile k spans [k*TILE - lead,
    // (k+1)*TILE - lead) with lead = the destination's offset into its line, clipped to the segment
    const uint64_t seg = Es * S;
    const uint64_t lead = reinterpret_cast<uintptr_t>(dp) & (kGatherLine - 1);
    const uint64_t b0r = static_cast<uint64_t>(k) * kGatherTileBytes;
    const uint64_t b0 = b0r > lead ? b0r - lead : 0;
    const uint64_t b1r = b0r + kGatherTileBytes - lead;
    const uint64_t b1 = b1r < seg ? b1r : seg;
    if (b0 < b1) copy_span<S>(sp + b0, dp + b0, static_cast<uint32_t>(b1 - b0));
  }
}

}  // namespace

hipError_t launch_param_contig(const GatherArgs& a, hipStream_t st) {
  if (a.total_tiles == 0) return hipSuccess;
  const uint32_t kMaxGrid = 1u << 20;
  const uint32_t grid = a.total_tiles < kMaxGrid ? a.total_tiles : kMaxGrid;
  if (a.elem == 2)
    hipLaunchKernelGGL(param_contig<2>, dim3(grid), dim3(kGB), 0, st, a);
  else
    hipLaunchKernelGGL(param_contig<4>, dim3(grid), dim3(kGB), 0, st, a);
  return hipGetLastError();
}

// Tiles per (node-block, parameter, slot) segment of E elements: enough for a shift of up to one line
// that puts tile boundaries on destination lines (the last tile of a segment may then be empty).
uint64_t gather_tiles_per_segment(uint64_t E, uint32_t elem) {
  if (E == 0) return 0;
  return (E * elem + (kGatherLine - 1) + kGatherTileBytes - 1) / kGatherTileBytes;
}

}  // namespace mr
