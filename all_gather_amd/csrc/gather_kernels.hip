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
// stores when source and destination share the same 16-byte phase, else the same packs realigned in
// registers from the two source packs each destination pack straddles.

#include "mr_internal.h"

namespace mr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGB = kGatherBlock;
constexpr int kCopyU = kGatherTileBytes / (16 * kGB);  // 16-byte words per lane per full tile
static_assert(kCopyU * 16 * kGB == kGatherTileBytes, "a tile is a whole number of workgroup sweeps");

// One element (S = 1: one byte, for pointers off their dtype's element grid; the host then plans the
// whole gather in bytes, so no access wider than a byte touches an address off its own alignment).
template <int S>
__device__ __forceinline__ void copy_elem(const char* src, char* dst, uint32_t o) {
  if (S == 1) dst[o] = src[o];
  else if (S == 2) *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
  else *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
}

// Output dword i of a destination-aligned pack whose source starts M bytes into the aligned pair
// (A, B): bytes M+4i .. M+4i+3 of A:B.
template <int M>
__device__ __forceinline__ u32x4 realign(const u32x4& A, const u32x4& B) {
  const uint32_t w[8] = {A[0], A[1], A[2], A[3], B[0], B[1], B[2], B[3]};
  constexpr int Q = M / 4, R = M % 4;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = R == 0 ? w[Q + i] : __builtin_amdgcn_alignbyte(w[Q + i + 1], w[Q + i], R);
  return o;
}

// wave_shl:1 (a DPP move across the 64-lane wave): lane l receives v of lane l + 1; lane 63 keeps `old`.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), 0x130, 0xf, 0xf, false));
}

// 16-byte stores to a 16-byte-aligned destination from a source M (1..15; a multiple of the element
// size, so even unless the gather is planned in bytes) bytes past a 16-byte
// boundary: each lane loads the two aligned source packs its output straddles and realigns them in
// registers.  Every loaded pack holds at least one byte of the span, so no access leaves the pages the
// source occupies.
template <int M>
__device__ __forceinline__ void copy_realigned(const u32x4* sa, u32x4* d4, uint32_t nw) {
  if (nw == kCopyU * kGB) {
    // a whole tile: no per-lane checks (same-GPU A/B, three interleaved repeats, W=8 G=4 P=64
    // log-uniform splits of any size: bf16 156.0-158.8 -> 146.7-148.0 us, fp32 294.4-294.7 -> 281.9-282.5 us).
    // Pack i + 1 is the next lane's pack i, so only lane 63 of each wave loads it (it lies in the next
    // wave's first lane); the others take it over with a DPP move: fp32 278.4-278.8 -> 276.9-277.3 us,
    // 8 shards one element off 140.7-142.3 -> 139.8-140.6 us, bf16 144.8-146.0 -> 144.9-145.3 us.
    const bool l63 = (threadIdx.x & 63) == 63;
    u32x4 a[kCopyU], nx[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t i = u * kGB + threadIdx.x;
      a[u] = __builtin_nontemporal_load(sa + i);
      nx[u] = u32x4{0u, 0u, 0u, 0u};
      if (l63) nx[u] = sa[i + 1];
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      u32x4 b;
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = from_next_lane(nx[u][k], a[u][k]);
      __builtin_nontemporal_store(realign<M>(a[u], b), d4 + u * kGB + threadIdx.x);
    }
    return;
  }
  for (uint32_t w0 = 0; w0 < nw; w0 += kCopyU * kGB) {
    u32x4 a[kCopyU], b[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t i = w0 + u * kGB + threadIdx.x;
      if (i < nw) {
        a[u] = __builtin_nontemporal_load(sa + i);
        b[u] = sa[i + 1];  // the next lane's pack: usually still in cache
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t i = w0 + u * kGB + threadIdx.x;
      if (i < nw) __builtin_nontemporal_store(realign<M>(a[u], b[u]), d4 + i);
    }
  }
}

// RA: the launch may hold spans whose source and destination 16-byte phases differ.  The kernel is
// built twice because the realigning path, compiled in, slows the aligned one it never runs (same-GPU
// A/B, W=8 G=4 P=64 log-uniform splits, bf16: 143 -> 146-149 us); the host picks the lean build whenever every span is in phase.
template <int S, bool RA>
__device__ __forceinline__ void copy_span(const char* src, char* dst, uint32_t len) {
  const uintptr_t ps = reinterpret_cast<uintptr_t>(src), pd = reinterpret_cast<uintptr_t>(dst);
  if (((ps ^ pd) & 15u) == 0) {
    // same 16-byte phase: element-wise head up to 16-byte alignment, 16-byte body, element-wise tail.
    // Loads and stores are non-temporal: plain loads cost 6% and plain stores 5% (same-GPU A/B, W=8 G=4
    // P=64 bf16 splits: 138.7 us against 147.0-147.4 and 145.0-145.3 us)
    uint32_t head = static_cast<uint32_t>((16u - (ps & 15u)) & 15u);
    if (head > len) head = len;
    const uint32_t body = (len - head) & ~15u;
    const uint32_t nw = body >> 4;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + head);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst + head);
    if (nw == kCopyU * kGB && head == 0 && len == nw * 16u) {
      // a whole aligned tile: straight-line loads and stores with no per-lane checks, so each store
      // waits only for its own load (same-GPU A/B, three interleaved repeats, W=8 G=4 P=64
      // log-uniform splits: bf16 142.2-143.2 -> 137.9-138.6 us, fp32 279.7-280.1 -> 276.7-277.1 us;
      // 8 shards into one tensor 134.2-134.5 -> 131.9-132.2 us)
      u32x4 v[kCopyU];
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) v[u] = __builtin_nontemporal_load(s4 + u * kGB + threadIdx.x);
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) __builtin_nontemporal_store(v[u], d4 + u * kGB + threadIdx.x);
      return;
    }
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
  } else if (!RA) {
    // not reached: the host launches this build only when every span is in phase
    for (uint32_t b = threadIdx.x * S; b < len; b += kGB * S) copy_elem<S>(src, dst, b);
  } else {
    // different 16-byte phases (split sizes that are not a multiple of 16 bytes): elements up to the
    // destination's 16-byte boundary, realigned 16-byte packs, elements at the end
    uint32_t head = static_cast<uint32_t>((16u - (pd & 15u)) & 15u);
    if (head > len) head = len;
    const uint32_t nw = (len - head) >> 4;
    const uint32_t m = static_cast<uint32_t>((ps + head) & 15u);  // source offset past its boundary
    const u32x4* sa = reinterpret_cast<const u32x4*>(src + head - m);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst + head);
    // m is a nonzero multiple of the element size S (S = 1 when the host planned in bytes)
    switch (m) {  // uniform per tile: one compile-time realignment per source offset
      case 4: copy_realigned<4>(sa, d4, nw); break;
      case 8: copy_realigned<8>(sa, d4, nw); break;
      case 12: copy_realigned<12>(sa, d4, nw); break;
      default:
        if constexpr (S <= 2) {
          switch (m) {
            case 2: copy_realigned<2>(sa, d4, nw); break;
            case 6: copy_realigned<6>(sa, d4, nw); break;
            case 10: copy_realigned<10>(sa, d4, nw); break;
            case 14: copy_realigned<14>(sa, d4, nw); break;
            default:
              if constexpr (S == 1) {
                switch (m) {
                  case 1: copy_realigned<1>(sa, d4, nw); break;
                  case 3: copy_realigned<3>(sa, d4, nw); break;
                  case 5: copy_realigned<5>(sa, d4, nw); break;
                  case 7: copy_realigned<7>(sa, d4, nw); break;
                  case 9: copy_realigned<9>(sa, d4, nw); break;
                  case 11: copy_realigned<11>(sa, d4, nw); break;
                  case 13: copy_realigned<13>(sa, d4, nw); break;
                  default: copy_realigned<15>(sa, d4, nw); break;
                }
              }
              break;
          }
        }
        break;
    }
    const uint32_t tail0 = head + (nw << 4);
    const uint32_t edge = head + (len - tail0);
    for (uint32_t b = threadIdx.x * S; b < edge; b += kGB * S) copy_elem<S>(src, dst, b < head ? b : tail0 + (b - head));
  }
}

// Param-major destination: the W slots of parameter s are contiguous in out (W*E_s elements from
// O_s*W), so tiles are cut per parameter over that whole block and a tile crossing a rank boundary
// switches source row mid-tile (W*P partial tiles become P).  Same-GPU A/B of lean builds against
// tiles cut per (node-block, parameter, slot) segment, three interleaved repeats, FSDP-style splits
// (W=8, G=4, P=64 log-uniform): bf16 143.1-144.2 -> 142.1-142.7 us, fp32 282.7-283.6 -> 279.5-281.0 us, from
// separate shards bf16 141.9-142.2 -> 140.1-140.4 us; but one parameter (a rank-major copy) fp32
// 271-272.5 -> 277.6-278.8 us, so the host uses these tiles only when P > 1.
template <int S, bool RA>
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
  if constexpr (!RA) {
    // A whole tile that crosses exactly one rank boundary, on a 16-byte pack boundary: each lane takes
    // its pack from rank r0 or r0 + 1 with a select, in straight-line code, instead of two checked
    // spans.  343 of the 26,303 tiles of the W=8 G=4 P=64 bf16 splits; same-GPU A/B, three interleaved
    // repeats: 138.8-139.6 -> 137.3-137.4 us (fp32 277.4-278.8 -> 277.3-277.8 us).
    if (b1 - b0 == kGatherTileBytes) {
      const uint64_t r0 = b0 / ES;
      const uint64_t xb = (r0 + 1) * ES;  // the first rank boundary after b0
      if (xb < b1 && b1 - xb <= ES && ((xb - b0) & 15u) == 0) {
        const char* s0 = (a.src_table ? a.src_tab[r0] + Os * S : a.src + (r0 * a.T + Os) * S) + (b0 - r0 * ES);
        const char* s1 = a.src_table ? a.src_tab[r0 + 1] + Os * S : a.src + ((r0 + 1) * a.T + Os) * S;
        char* d = pd + b0;
        if (((reinterpret_cast<uintptr_t>(s0) | reinterpret_cast<uintptr_t>(s1) | reinterpret_cast<uintptr_t>(d)) & 15u) == 0) {
          const uint32_t split = static_cast<uint32_t>((xb - b0) >> 4);  // packs taken from rank r0
          const u32x4* q0 = reinterpret_cast<const u32x4*>(s0);
          const u32x4* q1 = reinterpret_cast<const u32x4*>(s1);
          u32x4* d4 = reinterpret_cast<u32x4*>(d);
          u32x4 v[kCopyU];
#pragma unroll
          for (int u = 0; u < kCopyU; ++u) {
            const uint32_t i = u * kGB + threadIdx.x;
            v[u] = __builtin_nontemporal_load(i < split ? q0 + i : q1 + (i - split));
          }
#pragma unroll
          for (int u = 0; u < kCopyU; ++u) __builtin_nontemporal_store(v[u], d4 + u * kGB + threadIdx.x);
          return;
        }
      }
    }
  }
  for (uint64_t x = b0; x < b1;) {  // one piece per rank the tile touches (rank r = m*G + g)
    const uint64_t r = x / ES;
    const uint64_t xe = (r + 1) * ES < b1 ? (r + 1) * ES : b1;
    const char* sp = a.src_table ? a.src_tab[r] + Os * S : a.src + (r * a.T + Os) * S;
    copy_span<S, RA>(sp + (x - r * ES), pd + x, static_cast<uint32_t>(xe - x));
    x = xe;
  }
}

template <int S, bool RA>
__global__ __launch_bounds__(kGB) void param_contig(GatherArgs a) {
  if (a.span) {
    for (uint32_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) param_block_tile<S, RA>(a, t);
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
    if (b0 < b1) copy_span<S, RA>(sp + b0, dp + b0, static_cast<uint32_t>(b1 - b0));
  }
}

}  // namespace

hipError_t launch_param_contig(const GatherArgs& a, bool realign, hipStream_t st) {
  if (a.total_tiles == 0) return hipSuccess;
  const uint32_t kMaxGrid = 1u << 20;
  const uint32_t grid = a.total_tiles < kMaxGrid ? a.total_tiles : kMaxGrid;
  if (a.elem == 1)  // planned in bytes: pointers off the element grid
    hipLaunchKernelGGL((param_contig<1, true>), dim3(grid), dim3(kGB), 0, st, a);
  else if (a.elem == 2 && realign)
    hipLaunchKernelGGL((param_contig<2, true>), dim3(grid), dim3(kGB), 0, st, a);
  else if (a.elem == 2)
    hipLaunchKernelGGL((param_contig<2, false>), dim3(grid), dim3(kGB), 0, st, a);
  else if (realign)
    hipLaunchKernelGGL((param_contig<4, true>), dim3(grid), dim3(kGB), 0, st, a);
  else
    hipLaunchKernelGGL((param_contig<4, false>), dim3(grid), dim3(kGB), 0, st, a);
  return hipGetLastError();
}

// Tiles per (node-block, parameter, slot) segment of E elements: enough for a shift of up to one line
// that puts tile boundaries on destination lines (the last tile of a segment may then be empty).
uint64_t gather_tiles_per_segment(uint64_t E, uint32_t elem) {
  if (E == 0) return 0;
  return (E * elem + (kGatherLine - 1) + kGatherTileBytes - 1) / kGatherTileBytes;
}

}  // namespace mr
