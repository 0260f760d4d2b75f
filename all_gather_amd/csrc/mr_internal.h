// Internal launch interface shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mr.h"

namespace mr {

constexpr int kBlock = 256;             // threads per workgroup (4 wave64s)
constexpr size_t kCtrlBytes = 1024;     // barrier words at the head of a two-shot workspace
constexpr size_t kStageAlign = 256;

inline int elem_size(mr_dtype d) { return (d == MR_BF16 || d == MR_FP16) ? 2 : 4; }

// Barrier words of a two-shot workspace; each counter sits on its own 256-byte line.
struct Ctrl {
  uint32_t claim;     // ticket counter: the order in which workgroups start
  uint32_t pad0[63];
  uint32_t done1;     // phase-1 tiles released
  uint32_t pad1[63];
  uint32_t done2;     // phase-2 tiles finished (the last one resets the words)
  uint32_t pad2[63];
  uint32_t err;       // bit 0: a phase-2 wait gave up
  uint32_t pad3[63];
};
static_assert(sizeof(Ctrl) == kCtrlBytes, "ctrl layout");

struct RankPtrs {
  const char* p[MR_MAX_W];
};

// Element layout of one reduce call after the host has split off the unaligned head and tail.
//   [0, head)                        element-wise
//   [head, head + npacks*V)          16-byte packs (V = 16 / elem_size)
//   [head + npacks*V, n)             element-wise tail
// When the pointers do not share one alignment, vec == 0 and everything is element-wise (V = 1).
struct ReduceShape {
  size_t n;
  size_t head;
  size_t npacks;   // packs of the vector body (or elements when vec == 0)
  int vec;
};

struct TwoShotPlan {
  uint32_t chunks;           // W chunks
  size_t chunk_packs;        // packs per chunk (the last chunk may be shorter or empty)
  uint32_t tiles1_per_chunk; // phase-1 tiles per chunk
  uint32_t tiles2_per_chunk; // phase-2 tiles per chunk
  uint32_t n1, n2;           // phase-1 / phase-2 tile counts
  uint32_t spin_limit;       // bounded wait of a phase-2 workgroup (polls)
};

hipError_t launch_oneshot(const RankPtrs& in, int W, mr_dtype dt, char* out, const ReduceShape& sh,
                          hipStream_t st);
hipError_t launch_twoshot(const RankPtrs& in, int W, mr_dtype dt, char* out, char* stage, Ctrl* ctrl,
                          const ReduceShape& sh, const TwoShotPlan& pl, hipStream_t st);
TwoShotPlan plan_twoshot(int W, const ReduceShape& sh, uint32_t spin_limit);
hipError_t launch_zero_ctrl(Ctrl* ctrl, hipStream_t st);

// ---------------------------------------------------------------------------------- param-contiguous
constexpr int kMaxParams = MR_MAX_PARAMS_PER_LAUNCH;
constexpr uint32_t kGatherTileBytes = 16384;

struct GatherArgs {
  const char* src;
  char* out;
  uint64_t T;                       // elements per rank shard
  uint64_t O[kMaxParams + 1];       // O[s]: element offset of parameter s inside a shard; O[P] = its end
  uint32_t tile_prefix[kMaxParams + 1];  // node-block-local tile prefix: G * sum of tiles of params < s
  uint32_t P;
  uint32_t W, G;
  uint32_t elem;                    // bytes per element
  uint32_t tiles_per_block;         // tiles of one node-block (= tile_prefix[P])
  uint32_t total_tiles;             // W/G node-blocks * tiles_per_block
};

hipError_t launch_param_contig(const GatherArgs& a, hipStream_t st);

}  // namespace mr
