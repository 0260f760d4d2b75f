// Internal launch interface shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mr.h"

namespace mr {

constexpr int kBlock = 256;    // element-wise and gather workgroups (4 wave64s)

inline int elem_size(mr_dtype d) { return (d == MR_BF16 || d == MR_FP16) ? 2 : 4; }

// ------------------------------------------------------------------------------- two-shot workspace
//
//   [0, 16 KiB)                 Ctrl: ticket counters and barrier words, one 256-byte line each
//   [16 KiB, stage_off)         producer flags, one u32 per phase-1 tile (capacity bytes/256 tiles,
//                               enough for the element-wise path's one tile per 256 elements)
//   [stage_off, bytes)          stage buffer (n elements + kStageSlack bytes of alignment slack: the
//                               stage's 16-byte body starts at stage_off + 256)
// Every word before stage_off is zero between calls; the calls restore that themselves.
constexpr size_t kCtrlBytes = 16384;
constexpr size_t kStageSlack = 256;

struct Ctrl {
  uint32_t claim[MR_MAX_W][64];  // per-chunk ticket counters (grid barrier: phase-1 tile pools)
  uint32_t done1[MR_MAX_W][64];  // per-chunk phase-1 completions (chunk and grid barriers)
  uint32_t done2[MR_MAX_W][64];  // per-chunk phase-2 completions (grid barrier: phase-2 group pools)
  uint32_t gdone[64];            // workgroups finished (grid barrier)
  uint32_t err[64];              // bit 0: a wait gave up after the spin limit (that call's output is not
                                 // valid); bits 1 and 2: the XCD-local two-shot recomputed units after a
                                 // wait gave up / whose producer ran on another XCD (output valid)
};
static_assert(sizeof(Ctrl) <= kCtrlBytes, "ctrl layout");

inline size_t ws_flag_words(size_t bytes) { return bytes >> 8; }
inline size_t ws_stage_offset(size_t bytes) {
  return kCtrlBytes + ((ws_flag_words(bytes) * 4 + 255) & ~size_t(255));
}

// How phase 2 waits for phase 1.
enum TwoShotSync : uint32_t {
  kSyncTile = 0,   // per-tile producer flags: a phase-2 tile waits for the phase-1 tiles it copies
  kSyncChunk = 1,  // per-chunk barrier: waits for every phase-1 tile of its chunk
  kSyncGrid = 2,   // grid barrier: waits for every phase-1 tile of every chunk
  kSyncLast = 3,   // no waits: the workgroup that completes a group of phase-1 tiles copies that group
  kSyncAuto = 4,   // chosen from the message size (twoshot_sync_for)
};

// Tile shape of the reduce kernels (MR_OPT_TILE_SHAPE).  Wide tiles suit large messages; small ones
// need narrower tiles so that the grid still holds enough workgroups to keep every CU busy.
enum TileShape : uint32_t { kShapeAuto = 0, kShapeWide = 1, kShapeMedium = 2, kShapeNarrow = 3, kShapeWidePair = 4 };

// Auto choices, from graph-replayed sweeps at W=8 over 64 KiB .. 64 MiB per rank (bf16 and fp32):
// the narrow one-shot tile halves the time of messages below 1 MiB against the wide one (3.0 vs
// 5.4 us at 64 KiB), the medium one leads from 1 to 2-4 MiB, and the wide one from 4 MiB (fp32) or
// 8 MiB (bf16) up.  For two-shot, 256-pack tiles lead below 2 MiB and 1024-pack tiles above.  From 16
// to 64 MiB per rank (kShapeWidePair) the one-shot runs its wide tiles pipelined on a persistent grid
// of resident workgroups, each storing one tile's results while the next tile's loads are in flight
// (it first held pairs of tiles per workgroup, hence the name); one wide tile per workgroup leads again
// from 128 MiB.
constexpr size_t kPipeMaxPacks = size_t(1) << 22;  // largest one-shot on the pipelined wide tiles (64 MiB of bf16)
inline uint32_t oneshot_shape(size_t npacks, int elem_size, uint32_t forced) {
  if (forced != kShapeAuto) return forced;
  const size_t wide_from = elem_size == 4 ? (size_t(1) << 18) : (size_t(1) << 19);
  if (npacks >= (size_t(1) << 20) && npacks <= kPipeMaxPacks) return kShapeWidePair;
  if (npacks >= wide_from) return kShapeWide;          // 256 lanes x 4 packs
  if (npacks >= (size_t(1) << 16)) return kShapeMedium;  // 256 lanes x 1 pack
  return kShapeNarrow;                                   // 64 lanes x 1 pack
}
// Lanes (= packs) of the two-shot's wide phase-1 tile; the kernel's workgroup size and the planner's
// tile size both come from it.
#ifndef MR_TS_BLOCK
#define MR_TS_BLOCK 1024
#endif
constexpr uint32_t kTwoShotWideTile = MR_TS_BLOCK;
static_assert(kTwoShotWideTile == 256 || kTwoShotWideTile == 512 || kTwoShotWideTile == 1024, "workgroup size");
// Two-shot phase-1 tile (lanes = packs per tile) for a message of `npacks` packs.  The grid barrier
// orders every workgroup through one ticket counter (about 11.6 ns per same-address atomic), so it
// keeps the tile count low: 256-pack tiles only below 64 Ki packs, never 64-pack ones.
inline uint32_t twoshot_tile_packs(size_t npacks, uint32_t sync, uint32_t forced) {
  const bool grid = sync == kSyncGrid;
  const uint32_t shape = forced != kShapeAuto                              ? forced
                         : npacks >= (size_t(1) << (grid ? 16 : 17))      ? kShapeWide
                         : grid || npacks >= (size_t(1) << 13)            ? kShapeMedium
                                                                          : kShapeNarrow;
  return shape == kShapeNarrow ? 64u : shape == kShapeMedium ? 256u : kTwoShotWideTile;
}
// XCD-local units (twoshot_xcd, 16-byte path, W <= 8).  Under the last-arriver hand-off they lead at
// every size (narrow or medium units below 8 MiB per rank buffer, twoshot_xcd_unit_packs); under per-tile
// flags (copier workgroups) from 1 Mi packs to 4 Mi packs (16 to 64 MiB), beyond which the ticketed chunk
// tiles lead.  MR_TILE_WIDE_PAIR forces them, on wide units, for either hand-off at any size.
// Same-GPU A/B, W=8 bf16, rotating sets, best of three (us; eager launches):
//   per rank              4 MiB   8 MiB   16 MiB   32 MiB   64 MiB   256 MiB
//   XCD, last arriver     12.72   17.46   31.85    62.38    122.2    463.2     (wide units)
//   XCD, copiers          13.24   21.13   35.97    63.64    118.3    472.7
//   ticketed, last        11.54   19.06   37.33    71.75    143.4    573.5
//   ticketed, tile flags  15.51   19.87   35.63    66.37    124.1    454.6
//   two launches          13.01   19.75   33.11    62.93    122.1    490.0
constexpr uint32_t kXcds = 8;      // XCDs of an MI355X: one run of units each
constexpr uint32_t kXcdGroup = 4;  // units per phase-2 copy
#ifndef MR_XCD_LAST_GROUP
#define MR_XCD_LAST_GROUP 4
#endif
constexpr uint32_t kXcdLastGroup = MR_XCD_LAST_GROUP;  // units per copy under the last-arriver hand-off
inline bool twoshot_xcd_units(int vec, int W, size_t npacks, uint32_t sync, uint32_t forced) {
  if (!vec || W > 8 || (sync != kSyncTile && sync != kSyncLast)) return false;
  if (forced == kShapeWidePair) return true;
  if (forced != kShapeAuto) return false;
  if (sync == kSyncLast) return true;
  return npacks >= (size_t(1) << 20) && npacks <= (size_t(1) << 22);
}
// Packs per XCD-local unit: wide (256 lanes x 4 packs) for the copier workgroups, under MR_TILE_WIDE_PAIR,
// and from 512 Ki packs (8 MiB per rank buffer); below that the last arriver takes narrow units (64 x 1)
// under 64 Ki packs and medium ones (256 x 1) above.  Graph-replayed, W=8 bf16, us (narrow / medium /
// wide units; ticketed last arriver): 256 KiB 4.11 / 4.29 / 7.56; 5.34.  1 MiB 6.13 / 5.55 / 9.03; 6.85.
// 2 MiB 7.83 / 7.67 / 10.17; 8.92.  4 MiB 11.6 / 11.9 / 12.4; 12.1.
inline size_t twoshot_xcd_unit_packs(size_t npacks, uint32_t sync, uint32_t forced) {
  if (sync != kSyncLast || forced == kShapeWidePair || npacks >= (size_t(1) << 19)) return 1024;
  return npacks < (size_t(1) << 16) ? 64 : 256;
}
// Two-shot hand-off under MR_TWOSHOT_SYNC_AUTO: the last arriver on XCD-local units up to 32 MiB per rank
// buffer, per-tile flags above (tables above).
inline uint32_t twoshot_sync_for(size_t bytes, uint32_t sync) {
  if (sync != kSyncAuto) return sync;
  return bytes <= (size_t(32) << 20) ? kSyncLast : kSyncTile;
}

struct RankPtrs {
  const char* p[MR_MAX_W];
  // realigned 16-byte path: byte offset of rank r's 16-byte phase past out's, (p[r] - out) mod 16
  uint8_t shift[MR_MAX_W];
};

// Element layout of one reduce call after the host has split off the unaligned head and tail.
//   [0, head)                        element-wise
//   [head, head + npacks*V)          16-byte packs (V = 16 / elem_size), aligned on out
//   [head + npacks*V, n)             element-wise tail
// Pointers that are all multiples of the element size take the 16-byte path; when some input's 16-byte
// phase differs from out's, `realign` is set and that input's packs are loaded as the two aligned packs
// they straddle and realigned in registers (RankPtrs::shift).  A pointer that is not a multiple of the
// element size makes the whole call element-wise with byte accesses only (vec == 0, bytes == 1).
struct ReduceShape {
  size_t n;
  size_t head;
  size_t npacks;   // packs of the vector body
  int vec;
  int realign;     // vec path with some input out of out's 16-byte phase
  int bytes;       // element-wise path with byte loads and stores (some pointer not element-aligned)
};

struct TwoShotPlan {
  uint32_t chunks;       // W chunks
  size_t chunk_units;    // packs (or elements on the element-wise path) per chunk
  uint32_t t1;           // phase-1 tiles per chunk
  uint32_t t2;           // phase-2 tiles per chunk
  uint32_t ratio;        // phase-1 tiles per phase-2 tile
  uint32_t unit1;        // units per phase-1 tile; XCD-local units: 16-byte packs per unit (64, 256 or 1024)
  uint32_t unit2;        // units per phase-2 tile
  uint32_t sync;         // TwoShotSync
  uint32_t spin_limit;   // bounded wait (polls)
  // XCD-local units (xcd == 1; the chunk fields above are then unused by the kernel)
  uint32_t xcd;
  uint32_t run;          // units per XCD run
  uint32_t run_padded;   // run rounded up to whole copy groups
  size_t units;          // units of the message (16 KiB of output each)
};

// Workgroups of a two-shot launch, and the flag words it uses (one per phase-1 tile; XCD-local units:
// one per unit, or with the last-arriver hand-off one 64-bit arrival word per copy group of each run).
inline uint64_t twoshot_grid(const TwoShotPlan& pl) {
  if (pl.xcd) return uint64_t{kXcds} * (pl.sync == kSyncLast ? pl.run : pl.run_padded + pl.run_padded / kXcdGroup);
  return uint64_t{pl.chunks} * (pl.sync == kSyncLast ? pl.t1 : pl.t1 + pl.t2);
}
inline size_t twoshot_flag_words(const TwoShotPlan& pl) {
  if (pl.xcd) return pl.sync == kSyncLast ? 2 * size_t{kXcds} * ((pl.run + kXcdLastGroup - 1) / kXcdLastGroup) : pl.units;
  return size_t{pl.chunks} * pl.t1;
}

hipError_t launch_oneshot(const RankPtrs& in, int W, mr_dtype dt, char* out, const ReduceShape& sh,
                          uint32_t shape, hipStream_t st);  // shape: TileShape, already resolved
hipError_t launch_twoshot(const RankPtrs& in, int W, mr_dtype dt, char* out, char* stage, Ctrl* ctrl,
                          uint32_t* flags, const ReduceShape& sh, const TwoShotPlan& pl, hipStream_t st);
TwoShotPlan plan_twoshot(int W, const ReduceShape& sh, uint32_t sync, uint32_t spin_limit, uint32_t shape);
hipError_t launch_zero_words(void* p, size_t words, hipStream_t st);

// Host-side helpers of api.hip shared with the no-allocation entry point (noalloc.hip).
void set_last_hip_error(int e);
size_t workspace_bytes_for(size_t n, int esize);  // a workspace that holds a two-shot call of n elements
hipError_t clear_workspace_words(char* base, size_t bytes, hipStream_t st);  // barrier words and flags
mr_status check_allreduce_args(const void* const* bufs, int W, size_t n, mr_dtype dtype, const void* out, mr_mode mode);
// mr_allreduce_sum with the two-shot workspace given (never allocated) and only the hand-offs that leave
// it clean after every launch
mr_status allreduce_in_workspace(const void* const* bufs, int W, size_t n, mr_dtype dtype, void* out, mr_mode mode,
                                 hipStream_t st, char* ws_base, size_t ws_bytes);

// ---------------------------------------------------------------------------------- param-contiguous
constexpr int kMaxParams = MR_MAX_PARAMS_PER_LAUNCH;
#ifndef MR_GATHER_TILE
#define MR_GATHER_TILE 16384
#endif
#ifndef MR_GATHER_BLOCK
#define MR_GATHER_BLOCK 512
#endif
#ifndef MR_GATHER_LINE
#define MR_GATHER_LINE 256
#endif
constexpr uint32_t kGatherTileBytes = MR_GATHER_TILE;  // bytes per tile (one workgroup)
constexpr int kGatherBlock = MR_GATHER_BLOCK;          // lanes per gather workgroup
constexpr uint32_t kGatherLine = MR_GATHER_LINE;       // tile boundaries fall on destination lines of this size (1: off)

constexpr int kMaxTable = MR_MAX_TABLE_W;  // rank pointer tables in the kernel arguments

struct GatherArgs {
  const char* src;                       // rank-major source (src_tab unused)
  char* out;                             // param-major destination (dst_tab unused)
  const char* src_tab[kMaxTable];        // with src_table: rank r's shard (T elements)
  char* dst_tab[kMaxTable];              // with dst_table: rank r's own output (T elements)
  uint32_t src_table, dst_table;
  uint32_t span;                         // 1: tiles cut per parameter across its W ranks (param-major
                                         // destination); 0: per (node-block, parameter, slot) segment
  uint64_t T;                            // elements per rank shard
  uint64_t O[kMaxParams + 1];            // O[s]: element offset of parameter s inside a shard; O[P] = its end
  uint32_t tile_prefix[kMaxParams + 1];  // span: tiles of params < s; else node-block-local: G * tiles
                                         // per segment of params < s
  uint32_t P;
  uint32_t W, G;
  uint32_t elem;                         // bytes per element
  uint32_t tiles_per_block;              // tiles of one node-block (= tile_prefix[P]; span: all tiles)
  uint32_t total_tiles;                  // span: tile_prefix[P]; else W/G node-blocks * tiles_per_block
};

// SDMA copy engines (sdma.hip).  sdma_copy copies every piece on the current device's engines and
// waits for all of them: 0 on success, an hsa_status_t (> 0) if the engines are unavailable or a copy
// could not be issued, -1 if an engine reported a failed copy.
struct CopyPiece {
  const char* src;
  char* dst;
  uint64_t bytes;
};
int sdma_copy(const CopyPiece* pieces, size_t count);
int sdma_engine_count(int* status);  // status: the hsa_status_t of finding the engines

// realign: some span's source and destination differ in 16-byte phase (selects the kernel build)
hipError_t launch_param_contig(const GatherArgs& a, bool realign, hipStream_t st);
uint64_t gather_tiles_per_segment(uint64_t E, uint32_t elem);

// Workgroups of `kernel` (B lanes, no dynamic LDS) resident on the current device at once: its
// occupancy per CU times the CUs, looked up once per device; 0 if the runtime cannot say.
template <typename K>
size_t resident_workgroups(K kernel, int B) {
  constexpr int kDevices = 64;
  static std::atomic<long long> cache[kDevices];  // 0: not looked up yet, -1: unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kDevices) {
    const long long c = cache[dev].load(std::memory_order_relaxed);
    if (c) return c > 0 ? static_cast<size_t>(c) : 0;
  }
  int per_cu = 0, cus = 0;
  long long n = -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, B, 0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && per_cu > 0 && cus > 0)
    n = static_cast<long long>(per_cu) * cus;
  if (dev < kDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n > 0 ? static_cast<size_t>(n) : 0;
}

}  // namespace mr
