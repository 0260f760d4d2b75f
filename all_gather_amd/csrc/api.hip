// C ABI of libmr: argument validation, launch planning and the two-shot workspace registry.
// The public contract (argument meaning, layout, ownership, errors) is documented in include/mr.h.

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstddef>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "mr_internal.h"
#include "mr_probe.h"

namespace {

thread_local int g_last_hip_error = 0;

// An option's initial value from the environment: a whole number in [lo, hi], else the default (the
// same ranges mr_set_option accepts).
uint32_t env_u32(const char* name, uint32_t dflt, unsigned long lo, unsigned long hi) {
  const char* v = std::getenv(name);
  if (!v || !*v || *v == '-') return dflt;
  char* end = nullptr;
  const unsigned long x = std::strtoul(v, &end, 0);
  return (end && *end == 0 && x >= lo && x <= hi) ? static_cast<uint32_t>(x) : dflt;
}

// Piece size (bytes per rank of one parameter) below which mr_allgather_param_contig_sdma copies a
// parameter with the param-contiguous kernel instead of the engines (MR_OPT_SDMA_CU_BELOW).  An engine
// spends about 15 us on every copy beyond its bytes (2 KiB to 256 KiB pieces all took 15-17 us per copy
// per engine) and moves about 51 GB/s, so a 1 MiB piece costs it 15 + 20 us.  Same-GPU A/B, W=8 G=4
// P=64 FSDP-style splits bf16, per call alone / beside bf16 8192^3 GEMMs: every piece on the engines
// 1076-1093 / 1101-1107 us, below 256 KiB on the kernel 796-804 / 871-875, below 1 MiB 689-696 / 873-876,
// below 4 MiB 300-310 / 881-883; the GEMM's rate was the same in every case.  Beside the GEMM the
// kernel part waits for compute units that the GEMM's workgroups hold, which sets the call's time.
#ifndef MR_SDMA_CU_BELOW_DEFAULT
#define MR_SDMA_CU_BELOW_DEFAULT (1u << 20)
#endif

// Process-wide options (mr_set_option); defaults may be overridden by the environment at load.
std::atomic<uint32_t> g_spin_limit{env_u32("MR_SPIN_LIMIT", 1u << 22, 0, 0xffffffffUL)};
std::atomic<uint32_t> g_twoshot_sync{env_u32("MR_TWOSHOT_SYNC", mr::kSyncAuto, MR_TWOSHOT_SYNC_TILE, MR_TWOSHOT_SYNC_AUTO)};
std::atomic<uint32_t> g_tile_shape{env_u32("MR_TILE_SHAPE", mr::kShapeAuto, MR_TILE_AUTO, MR_TILE_WIDE_PAIR)};
std::atomic<uint32_t> g_sdma_cu_below{env_u32("MR_SDMA_CU_BELOW", MR_SDMA_CU_BELOW_DEFAULT, 0, 0xffffffffUL)};
const bool g_trace = env_u32("MR_TRACE", 0, 0, 1) != 0;

mr_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return MR_ERR_HIP;
}

bool is_float(mr_dtype d) { return d == MR_BF16 || d == MR_FP16 || d == MR_FP32; }
bool valid_dtype(int d) { return d >= MR_BF16 && d <= MR_INT32; }

bool overlap(uintptr_t a, size_t na, uintptr_t b, size_t nb) {
  return na && nb && a < b + nb && b < a + na;
}

// Is the pointer a multiple of the element size?  (Pointers that are not take the byte paths.)
bool elem_aligned(const void* p, uint64_t es) { return reinterpret_cast<uintptr_t>(p) % es == 0; }

// ------------------------------------------------------------------------------ workspace registry
struct Workspace {
  char* base = nullptr;
  size_t bytes = 0;
  bool owned = false;
};

// Workspaces by (device, stream, capture id).  Capture id 0 is the stream's own workspace (eager calls,
// and caller-owned memory bound with mr_set_workspace); a call made while the stream is being captured
// into a HIP graph gets a library-owned workspace of that capture, so graphs captured one after
// another on one stream (torch.cuda.graph captures every graph on one shared stream) never share
// barrier words and may be replayed at the same time on different streams.
using WsKey = std::tuple<int, hipStream_t, unsigned long long>;
std::mutex g_ws_mu;
std::map<WsKey, Workspace> g_ws;
// Library-owned buffers that a larger workspace replaced, by (device, stream).  Launches still in
// flight, and HIP graphs that captured a two-shot call, may point at them, so they are freed only when
// the caller unbinds the stream's workspace (mr_set_workspace).  Growth at least doubles, so they total
// less than the live one.
std::map<std::pair<int, hipStream_t>, std::vector<char*>> g_retired;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Smallest workspace whose layout (barrier words, flags, stage) holds a stage of n elements plus 256
// bytes of alignment slack.  Its flag capacity (bytes/256 words) covers the largest plan for n: one
// flag per 256-element tile on the element-wise path, plus one per chunk for ragged chunks.
size_t ws_bytes_for(size_t n, int esize) {
  const size_t base = mr::kCtrlBytes + n * static_cast<size_t>(esize) + mr::kStageSlack + 16;
  return round_up(base + base / 63 + 4096, 4096);
}

bool ws_fits(size_t bytes, size_t n, int esize, size_t flags_needed) {
  return mr::ws_stage_offset(bytes) + n * static_cast<size_t>(esize) + mr::kStageSlack <= bytes &&
         flags_needed <= mr::ws_flag_words(bytes);
}

hipError_t ws_clear(char* base, size_t bytes, hipStream_t st) {
  return mr::launch_zero_words(base, mr::ws_stage_offset(bytes) / 4, st);
}

// Returns the workspace of (current device, stream) able to hold a two-shot call of n elements
// needing `flags` producer flags, allocating or growing a library-owned one.
mr_status get_workspace(hipStream_t st, size_t n, int esize, size_t flags, Workspace* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long capture = 0;
  e = hipStreamGetCaptureInfo(st, &cs, &capture);
  if (e != hipSuccess) return hip_fail(e);
  if (cs != hipStreamCaptureStatusActive) capture = 0;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if (capture) {  // caller-owned memory bound to the stream is used for captured calls too
    auto own = g_ws.find(WsKey{dev, st, 0});
    if (own != g_ws.end() && own->second.base && !own->second.owned) {
      if (!ws_fits(own->second.bytes, n, esize, flags)) return MR_ERR_WORKSPACE;
      *out = own->second;
      return MR_OK;
    }
  }
  Workspace& w = g_ws[WsKey{dev, st, capture}];
  if (w.base && ws_fits(w.bytes, n, esize, flags)) {
    *out = w;
    return MR_OK;
  }
  if (w.base && !w.owned) return MR_ERR_WORKSPACE;  // caller-owned and too small
  // Any size at or above the rule's also fits: the stage start moves by 1/64 of the extra bytes.
  size_t bytes = round_up(ws_bytes_for(n, esize), size_t(1) << 20);
  if (w.base && bytes < 2 * w.bytes) bytes = 2 * w.bytes;
  if (!ws_fits(bytes, n, esize, flags)) return MR_ERR_WORKSPACE;  // the sizing rule covers every plan
  void* p = nullptr;
  if (capture) {
    // an allocation is not a stream operation: allowed inside a capture once this thread's capture mode
    // is relaxed for the call (the clear below is a kernel, recorded into the graph before the reduce)
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    e = hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess) return hip_fail(e);
    e = hipMalloc(&p, bytes);
    (void)hipThreadExchangeStreamCaptureMode(&mode);
  } else {
    e = hipMalloc(&p, bytes);
  }
  if (e != hipSuccess) return hip_fail(e);
  e = ws_clear(static_cast<char*>(p), bytes, st);
  if (e != hipSuccess) {
    (void)hipFree(p);  // the launch error is the one reported
    return hip_fail(e);
  }
  if (w.base) g_retired[{dev, st}].push_back(w.base);  // grown: keep the old buffer alive (see g_retired)
  w.base = static_cast<char*>(p);
  w.bytes = bytes;
  w.owned = true;
  *out = w;
  return MR_OK;
}


// ------------------------------------------------------------------------------------ reduce launch
// 16-byte layout of a reduce call: element-wise head up to out's 16-byte boundary, packs, element-wise
// tail; everything element-wise when the pointers do not share one 16-byte phase.
mr::ReduceShape reduce_shape(size_t n, int es, uintptr_t po, bool same_phase, bool on_grid = true) {
  mr::ReduceShape sh{};
  sh.n = n;
  sh.vec = on_grid ? 1 : 0;
  sh.realign = on_grid && !same_phase ? 1 : 0;
  sh.bytes = on_grid ? 0 : 1;
  if (sh.vec) {
    const size_t V = 16 / static_cast<size_t>(es);
    size_t head = ((16u - (po & 15u)) & 15u) / static_cast<size_t>(es);
    if (head > n) head = n;
    sh.head = head;
    sh.npacks = (n - head) / V;
  }
  return sh;
}

// The two-shot plan of a call under the given options (wait_free: see reduce_launch).
mr::TwoShotPlan twoshot_plan_for(int W, const mr::ReduceShape& sh, int es, uint32_t sync_opt, uint32_t shape_opt,
                                 bool wait_free) {
  uint32_t sync = mr::twoshot_sync_for(sh.n * static_cast<size_t>(es), sync_opt);
  uint32_t shape = shape_opt;
  if (wait_free) {  // the last arriver, on ticketed tiles or XCD-local units by size: nothing ever waits
    shape = mr::kShapeAuto;
    sync = mr::kSyncLast;
  }
  return mr::plan_twoshot(W, sh, sync, g_spin_limit.load(), shape);
}

// Alias check, 16-byte layout of the call, and the one-shot or two-shot launch.  `ins` are already
// validated non-null.
// `fixed`: a workspace the call must use instead of the stream's (the no-allocation entry point);
// `wait_free`: take only the last-arriver hand-off (ticketed tiles or XCD-local units by size), in which
// no workgroup ever waits: every word is back at zero when a launch ends and no output is ever invalid.
mr_status reduce_launch(const char* const* ins, int W, size_t n, mr_dtype dtype, char* out, mr_mode mode,
                        hipStream_t st, const Workspace* fixed = nullptr, bool wait_free = false) {
  const int es = mr::elem_size(dtype);
  const size_t nbytes = n * static_cast<size_t>(es);
  const uintptr_t po = reinterpret_cast<uintptr_t>(out);
  mr::RankPtrs in{};
  bool same_phase = true;
  bool aligned = po % static_cast<uintptr_t>(es) == 0;
  for (int r = 0; r < W; ++r) {
    const uintptr_t pr = reinterpret_cast<uintptr_t>(ins[r]);
    if (pr != po && overlap(pr, nbytes, po, nbytes)) return MR_ERR_ALIAS;
    if ((pr & 15u) != (po & 15u)) same_phase = false;
    if (pr % static_cast<uintptr_t>(es) != 0) aligned = false;
    in.p[r] = ins[r];
    in.shift[r] = static_cast<uint8_t>((pr - po) & 15u);
  }
  const mr::ReduceShape sh = reduce_shape(n, es, po, same_phase, aligned);
  hipError_t e;
  if (mode == MR_ONESHOT) {
    const uint32_t shape = mr::oneshot_shape(sh.npacks, es, g_tile_shape.load());
    if (g_trace)
      std::fprintf(stderr, "[mr] allreduce oneshot W=%d n=%zu dtype=%d vec=%d head=%zu packs=%zu shape=%u\n", W, n,
                   static_cast<int>(dtype), sh.vec, sh.head, sh.npacks, shape);
    e = mr::launch_oneshot(in, W, dtype, out, sh, shape, st);
  } else {
    const mr::TwoShotPlan pl = twoshot_plan_for(W, sh, es, g_twoshot_sync.load(), g_tile_shape.load(), wait_free);
    if (mr::twoshot_grid(pl) >= (1ull << 24)) return MR_ERR_INVALID_ARG;
    const size_t flags_needed = mr::twoshot_flag_words(pl);
    Workspace ws;
    if (fixed) {
      if (!ws_fits(fixed->bytes, n, es, flags_needed)) return MR_ERR_WORKSPACE;
      ws = *fixed;
    } else {
      mr_status s = get_workspace(st, n, es, flags_needed, &ws);
      if (s != MR_OK) return s;
    }
    // The stage shares out's 16-byte phase, so its body is 16-byte aligned too, and the body starts on a
    // 256-byte boundary, so units of 16 KiB never share a cache line: each stage line is then loaded
    // by one workgroup, once per launch.
    const size_t hb = sh.vec ? sh.head * static_cast<size_t>(es) : 0;
    char* stage = ws.base + mr::ws_stage_offset(ws.bytes) + (hb ? mr::kStageSlack - hb : 0);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws.base + mr::kCtrlBytes);
    if (g_trace)
      std::fprintf(stderr, "[mr] allreduce twoshot W=%d n=%zu dtype=%d vec=%d sync=%u chunk=%zu tile=%u t1=%u t2=%u "
                   "xcd=%u units=%zu run=%u\n", W, n, static_cast<int>(dtype), sh.vec, pl.sync, pl.chunk_units, pl.unit1,
                   pl.t1, pl.t2, pl.xcd, pl.units, pl.run);
    e = mr::launch_twoshot(in, W, dtype, out, stage, reinterpret_cast<mr::Ctrl*>(ws.base), flags, sh, pl, st);
  }
  return e == hipSuccess ? MR_OK : hip_fail(e);
}

// ------------------------------------------------------------------------------------ gather launches
// Splits are validated and cut into launch groups of up to kMaxParams parameters before anything is
// enqueued; the entry points then fill in the pointers of every group and launch them in order.
struct GatherPlan {
  uint64_t T = 0;
  uint64_t es = 0;
  // Phase of every piece (parameter s, rank r) of a param-major output, as bit (dst_off - src_off) mod 16,
  // where dst_off = (O_s*W + r*E_s)*es.  A launch may take the lean kernel build only if, for the call's
  // base pointers, every piece's source and destination share a 16-byte phase.
  uint16_t rm_mask = 0;              // source rank-major: src_off = (r*T + O_s)*es (period 16 in r)
  std::vector<uint16_t> rank_mask;   // source from per-rank pointers: src_off = O_s*es, one mask per rank
  std::vector<mr::GatherArgs> groups;
};

// Does a bit other than bit d (the call's base-pointer difference mod 16) appear in the mask?
bool needs_realign(uint16_t mask, uintptr_t d) { return (mask & ~(1u << (d & 15u))) != 0; }

// span: tiles cut per parameter over its W*E_s contiguous destination elements (every param-major
// output); otherwise per (node-block, parameter, slot) segment (the list output's separate buffers).
// bytes: plan the same placement on bytes (element size 1, every count times the dtype's size), for
// pointers that are not multiples of the element size.
// cu_below: only parameters whose per-rank piece is smaller than this many bytes get tiles (the others
// keep their offsets but no tile maps to them, so a launch copies the small parameters alone).
mr_status gather_plan(int W, int G, const uint64_t* splits, int P, mr_dtype dtype, bool span, GatherPlan* gp,
                      bool bytes = false, uint64_t cu_below = UINT64_MAX) {
  if (G < 1 || W % G != 0) return MR_ERR_INVALID_ARG;
  if (P < 1 || !splits) return MR_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return MR_ERR_INVALID_ARG;
  const uint64_t scale = bytes ? static_cast<uint64_t>(mr::elem_size(dtype)) : 1;
  const uint64_t es = bytes ? 1 : static_cast<uint64_t>(mr::elem_size(dtype));
  uint64_t T = 0;
  for (int s = 0; s < P; ++s) {
    if (splits[s] > (1ull << 56) || T > (1ull << 56)) return MR_ERR_INVALID_ARG;
    T += splits[s] * scale;
  }
  if (T > (1ull << 56) / (static_cast<uint64_t>(W) * es)) return MR_ERR_INVALID_ARG;
  // gp may be a reused cache slot: reset every field (vectors keep their capacity)
  gp->T = T;
  gp->es = es;
  gp->rm_mask = 0;
  gp->groups.clear();
  gp->rank_mask.assign(W <= MR_MAX_TABLE_W ? static_cast<size_t>(W) : 0, 0);
  if (T == 0) return MR_OK;
  {
    uint64_t O = 0;
    for (int s = 0; s < P; ++s) {
      const uint64_t E = splits[s] * scale;
      for (int r = 0; E && E * es < cu_below && r < W; ++r) {
        const uint64_t dst_off = (O * W + static_cast<uint64_t>(r) * E) * es;
        if (r < 16) gp->rm_mask |= static_cast<uint16_t>(1u << ((dst_off - (static_cast<uint64_t>(r) * T + O) * es) & 15u));
        if (r < static_cast<int>(gp->rank_mask.size()))
          gp->rank_mask[r] |= static_cast<uint16_t>(1u << ((dst_off - O * es) & 15u));
      }
      O += E;
    }
  }
  uint64_t base = 0;  // shard offset of the first parameter of a group
  for (int s0 = 0; s0 < P; s0 += mr::kMaxParams) {
    const int np = (P - s0) < mr::kMaxParams ? (P - s0) : mr::kMaxParams;
    mr::GatherArgs a;
    std::memset(&a, 0, sizeof(a));
    a.T = T;
    a.P = static_cast<uint32_t>(np);
    a.W = static_cast<uint32_t>(W);
    a.G = static_cast<uint32_t>(G);
    a.elem = static_cast<uint32_t>(es);
    a.span = span ? 1u : 0u;
    uint64_t tiles = 0;
    for (int i = 0; i < np; ++i) {
      a.O[i] = base;
      a.tile_prefix[i] = static_cast<uint32_t>(tiles);
      const uint64_t E = splits[s0 + i] * scale;
      if (E * es < cu_below)
        tiles += span ? mr::gather_tiles_per_segment(E * static_cast<uint64_t>(W), static_cast<uint32_t>(es))
                      : static_cast<uint64_t>(G) * mr::gather_tiles_per_segment(E, static_cast<uint32_t>(es));
      base += E;
      if (tiles >= (1ull << 31)) return MR_ERR_INVALID_ARG;
    }
    a.O[np] = base;
    a.tile_prefix[np] = static_cast<uint32_t>(tiles);
    a.tiles_per_block = static_cast<uint32_t>(tiles);
    const uint64_t total = span ? tiles : tiles * static_cast<uint64_t>(W / G);
    if (total >= (1ull << 32)) return MR_ERR_INVALID_ARG;
    a.total_tiles = static_cast<uint32_t>(total);
    gp->groups.push_back(a);
  }
  return MR_OK;
}

// Plans depend only on (W, G, P, dtype, splits).  FSDP issues the same few gathers every step, so each
// thread keeps its last kPlanSlots plans: a repeated call neither recomputes the prefix sums and tile
// tables nor allocates.  Failed plans are not kept.
struct CachedPlan {
  bool used = false;
  bool span = false;
  bool bytes = false;
  uint64_t cu_below = UINT64_MAX;
  int W = 0, G = 0, P = 0;
  mr_dtype dtype = MR_BF16;
  std::vector<uint64_t> splits;
  GatherPlan plan;
};
constexpr int kPlanSlots = 8;
thread_local CachedPlan t_plans[kPlanSlots];
thread_local int t_plan_next = 0;

mr_status cached_gather_plan(int W, int G, const uint64_t* splits, int P, mr_dtype dtype, bool span,
                             const GatherPlan** out, bool bytes = false, uint64_t cu_below = UINT64_MAX) {
  if (P < 1 || !splits) return MR_ERR_INVALID_ARG;
  const size_t key_bytes = static_cast<size_t>(P) * sizeof(uint64_t);
  for (const CachedPlan& c : t_plans)
    if (c.used && c.span == span && c.bytes == bytes && c.cu_below == cu_below && c.W == W && c.G == G && c.P == P &&
        c.dtype == dtype &&
        std::memcmp(c.splits.data(), splits, key_bytes) == 0) {
      *out = &c.plan;
      return MR_OK;
    }
  CachedPlan& c = t_plans[t_plan_next];
  t_plan_next = (t_plan_next + 1) % kPlanSlots;
  c.used = false;
  const mr_status s = gather_plan(W, G, splits, P, dtype, span, &c.plan, bytes, cu_below);
  if (s != MR_OK) return s;
  c.span = span;
  c.bytes = bytes;
  c.cu_below = cu_below;
  c.W = W;
  c.G = G;
  c.P = P;
  c.dtype = dtype;
  c.splits.assign(splits, splits + P);
  c.used = true;
  *out = &c.plan;
  return MR_OK;
}

// Launch every group of a plan; `bind` fills in this call's pointers on a copy of the group's arguments;
// `realign` selects the kernel build that handles out-of-phase pieces.
template <typename Bind>
mr_status gather_launch(const GatherPlan& gp, Bind bind, bool realign, hipStream_t st) {
  for (const mr::GatherArgs& g : gp.groups) {
    mr::GatherArgs a = g;
    bind(a);
    if (g_trace)
      std::fprintf(stderr, "[mr] gather W=%u G=%u params=%u T=%llu tiles=%u span=%u realign=%d src_table=%u dst_table=%u\n",
                   a.W, a.G, a.P, static_cast<unsigned long long>(a.T), a.total_tiles, a.span, realign ? 1 : 0,
                   a.src_table, a.dst_table);
    const hipError_t e = mr::launch_param_contig(a, realign, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return MR_OK;
}

}  // namespace

namespace mr {

void set_last_hip_error(int e) { g_last_hip_error = e; }

size_t workspace_bytes_for(size_t n, int esize) { return ws_bytes_for(n, esize); }

hipError_t clear_workspace_words(char* base, size_t bytes, hipStream_t st) { return ws_clear(base, bytes, st); }

mr_status check_allreduce_args(const void* const* bufs, int W, size_t n, mr_dtype dtype, const void* out, mr_mode mode) {
  if (W < 1 || W > MR_MAX_W) return MR_ERR_INVALID_ARG;
  if (mode != MR_ONESHOT && mode != MR_TWOSHOT) return MR_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return MR_ERR_INVALID_ARG;
  if (!is_float(dtype)) return MR_ERR_DTYPE;
  if (n == 0) return MR_OK;
  if (!bufs || !out) return MR_ERR_INVALID_ARG;
  const int es = elem_size(dtype);
  if (n > (SIZE_MAX / 2 - kCtrlBytes) / static_cast<size_t>(es)) return MR_ERR_INVALID_ARG;
  for (int r = 0; r < W; ++r)
    if (!bufs[r]) return MR_ERR_INVALID_ARG;
  return MR_OK;  // any alignment: pointers off the element grid take the byte-access path
}

mr_status allreduce_in_workspace(const void* const* bufs, int W, size_t n, mr_dtype dtype, void* out, mr_mode mode,
                                 hipStream_t st, char* ws_base, size_t ws_bytes) {
  const mr_status s = check_allreduce_args(bufs, W, n, dtype, out, mode);
  if (s != MR_OK || n == 0) return s;
  const char* ins[MR_MAX_W];
  for (int r = 0; r < W; ++r) ins[r] = static_cast<const char*>(bufs[r]);
  Workspace ws;
  ws.base = ws_base;
  ws.bytes = ws_bytes;
  return reduce_launch(ins, W, n, dtype, static_cast<char*>(out), mode, st, &ws, true);
}

}  // namespace mr

extern "C" {

const char* mr_status_string(mr_status s) {
  switch (s) {
    case MR_OK: return "MR_OK";
    case MR_ERR_INVALID_ARG: return "MR_ERR_INVALID_ARG: invalid argument";
    case MR_ERR_DTYPE: return "MR_ERR_DTYPE: dtype not supported by this operation";
    case MR_ERR_ALIAS: return "MR_ERR_ALIAS: output partially overlaps an input";
    case MR_ERR_WORKSPACE: return "MR_ERR_WORKSPACE: two-shot workspace missing, too small or in error";
    case MR_ERR_HIP: return "MR_ERR_HIP: HIP runtime call failed";
    case MR_ERR_ENGINE: return "MR_ERR_ENGINE: copy engines unavailable or a copy failed";
    default: return "unknown mr_status";
  }
}

int mr_last_hip_error(void) { return g_last_hip_error; }

int mr_version(void) { return 105; }

size_t mr_workspace_bytes(int W, size_t n, mr_dtype dtype) {
  if (W < 1 || W > MR_MAX_W || !is_float(dtype)) return 0;
  const int es = mr::elem_size(dtype);
  if (n > (SIZE_MAX / 4) / static_cast<size_t>(es)) return 0;
  return ws_bytes_for(n, es);
}

mr_status mr_set_option(mr_option opt, int64_t value) {
  switch (opt) {
    case MR_OPT_TWOSHOT_SYNC:
      if (value < MR_TWOSHOT_SYNC_TILE || value > MR_TWOSHOT_SYNC_AUTO) return MR_ERR_INVALID_ARG;
      g_twoshot_sync.store(static_cast<uint32_t>(value));
      return MR_OK;
    case MR_OPT_SPIN_LIMIT:
      if (value < 0 || value > 0xffffffffll) return MR_ERR_INVALID_ARG;
      g_spin_limit.store(static_cast<uint32_t>(value));
      return MR_OK;
    case MR_OPT_TILE_SHAPE:
      if (value < MR_TILE_AUTO || value > MR_TILE_WIDE_PAIR) return MR_ERR_INVALID_ARG;
      g_tile_shape.store(static_cast<uint32_t>(value));
      return MR_OK;
    case MR_OPT_SDMA_CU_BELOW:
      if (value < 0 || value > 0xffffffffll) return MR_ERR_INVALID_ARG;
      g_sdma_cu_below.store(static_cast<uint32_t>(value));
      return MR_OK;
    default:
      return MR_ERR_INVALID_ARG;
  }
}

mr_status mr_get_option(mr_option opt, int64_t* value) {
  if (!value) return MR_ERR_INVALID_ARG;
  switch (opt) {
    case MR_OPT_TWOSHOT_SYNC: *value = g_twoshot_sync.load(); return MR_OK;
    case MR_OPT_SPIN_LIMIT: *value = g_spin_limit.load(); return MR_OK;
    case MR_OPT_TILE_SHAPE: *value = g_tile_shape.load(); return MR_OK;
    case MR_OPT_SDMA_CU_BELOW: *value = g_sdma_cu_below.load(); return MR_OK;
    default: return MR_ERR_INVALID_ARG;
  }
}

mr_status mr_allreduce_sum(const void* const* bufs, int W, size_t n, mr_dtype dtype, void* out, mr_mode mode,
                           mr_stream stream) {
  const mr_status s = mr::check_allreduce_args(bufs, W, n, dtype, out, mode);
  if (s != MR_OK || n == 0) return s;
  const char* ins[MR_MAX_W];
  for (int r = 0; r < W; ++r) ins[r] = static_cast<const char*>(bufs[r]);
  return reduce_launch(ins, W, n, dtype, static_cast<char*>(out), mode, reinterpret_cast<hipStream_t>(stream));
}

mr_status mr_reduce_scatter_chunk(size_t n, int W, mr_dtype dtype, int rank, size_t* offset, size_t* count) {
  if (W < 1 || W > MR_MAX_W || rank < 0 || rank >= W || !offset || !count) return MR_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return MR_ERR_INVALID_ARG;
  if (!is_float(dtype)) return MR_ERR_DTYPE;
  const size_t V = 16 / static_cast<size_t>(mr::elem_size(dtype));
  if (n > SIZE_MAX / 2) return MR_ERR_INVALID_ARG;
  const size_t per = (n + W - 1) / W;
  const size_t C = (per + V - 1) / V * V;
  const size_t start = static_cast<size_t>(rank) * C < n ? static_cast<size_t>(rank) * C : n;
  *offset = start;
  *count = (start + C < n ? start + C : n) - start;
  return MR_OK;
}

mr_status mr_reduce_scatter_sum(const void* const* bufs, int W, size_t n, mr_dtype dtype, int rank, void* out,
                                mr_stream stream) {
  size_t off = 0, cnt = 0;
  mr_status s = mr_reduce_scatter_chunk(n, W, dtype, rank, &off, &cnt);
  if (s != MR_OK) return s;
  if (cnt == 0) return MR_OK;
  if (!bufs || !out) return MR_ERR_INVALID_ARG;
  const size_t es = static_cast<size_t>(mr::elem_size(dtype));
  const char* ins[MR_MAX_W];
  for (int r = 0; r < W; ++r) {
    if (!bufs[r]) return MR_ERR_INVALID_ARG;
    ins[r] = static_cast<const char*>(bufs[r]) + off * es;  // this rank's chunk of every rank buffer
  }
  return reduce_launch(ins, W, cnt, dtype, static_cast<char*>(out), MR_ONESHOT, reinterpret_cast<hipStream_t>(stream));
}

// Element size of a gather's pointers: the dtype's, or 1 when some pointer is off the element grid (then
// the plan and the copy work on bytes).
bool gather_on_grid(mr_dtype dtype, std::initializer_list<const void*> ptrs) {
  if (!valid_dtype(dtype)) return true;
  const uint64_t es = static_cast<uint64_t>(mr::elem_size(dtype));
  for (const void* p : ptrs)
    if (!elem_aligned(p, es)) return false;
  return true;
}

mr_status mr_allgather_param_contig(const void* src, int W, int G, const uint64_t* splits, int P, mr_dtype dtype,
                                    void* out, mr_stream stream) {
  if (W < 1 || W > 65535) return MR_ERR_INVALID_ARG;
  const GatherPlan* gp = nullptr;
  // tiles span a parameter's W slots when there are several parameters; one parameter (a plain
  // rank-major copy) measured faster with per-slot tiles
  mr_status s = cached_gather_plan(W, G, splits, P, dtype, P > 1, &gp, !gather_on_grid(dtype, {src, out}));
  if (s != MR_OK || gp->T == 0) return s;
  if (!src || !out) return MR_ERR_INVALID_ARG;
  const uint64_t total_bytes = static_cast<uint64_t>(W) * gp->T * gp->es;
  if (overlap(reinterpret_cast<uintptr_t>(src), total_bytes, reinterpret_cast<uintptr_t>(out), total_bytes))
    return MR_ERR_ALIAS;
  const bool realign =
      needs_realign(gp->rm_mask, reinterpret_cast<uintptr_t>(src) - reinterpret_cast<uintptr_t>(out));
  return gather_launch(*gp, [&](mr::GatherArgs& a) {
    a.src = static_cast<const char*>(src);
    a.out = static_cast<char*>(out);
  }, realign, reinterpret_cast<hipStream_t>(stream));
}

mr_status mr_allgather_param_contig_sdma(const void* src, int W, int G, const uint64_t* splits, int P, mr_dtype dtype,
                                         void* out, mr_stream stream) {
  if (W < 1 || W > 65535) return MR_ERR_INVALID_ARG;
  const uint64_t cu_below = g_sdma_cu_below.load();
  const GatherPlan* gp = nullptr;
  // the plan gives the kernel the tiles of the parameters below cu_below and the engines their offsets
  mr_status s = cached_gather_plan(W, G, splits, P, dtype, P > 1, &gp, !gather_on_grid(dtype, {src, out}), cu_below);
  if (s != MR_OK || gp->T == 0) return s;
  if (!src || !out) return MR_ERR_INVALID_ARG;
  const uint64_t total_bytes = static_cast<uint64_t>(W) * gp->T * gp->es;
  if (overlap(reinterpret_cast<uintptr_t>(src), total_bytes, reinterpret_cast<uintptr_t>(out), total_bytes))
    return MR_ERR_ALIAS;
  // one piece per (parameter, rank) of the other parameters, in the order of the page's node-block ->
  // split -> slot loop; pieces that continue the previous one on both sides are merged (one parameter:
  // a single copy)
  std::vector<mr::CopyPiece> pieces;
  const char* sb = static_cast<const char*>(src);
  char* ob = static_cast<char*>(out);
  const uint64_t es = gp->es, T = gp->T;
  bool cu_part = false;
  for (const mr::GatherArgs& g : gp->groups) cu_part = cu_part || g.total_tiles != 0;
  for (int m = 0; m < W / G; ++m)
    for (const mr::GatherArgs& g : gp->groups)
      for (uint32_t i = 0; i < g.P; ++i) {
        const uint64_t O = g.O[i], E = g.O[i + 1] - O;
        if (E * es < cu_below) continue;  // copied by the kernel
        for (int gg = 0; E && gg < G; ++gg) {
          const uint64_t r = static_cast<uint64_t>(m) * G + gg;
          const mr::CopyPiece c{sb + (r * T + O) * es, ob + (O * W + r * E) * es, E * es};
          if (!pieces.empty() && pieces.back().src + pieces.back().bytes == c.src &&
              pieces.back().dst + pieces.back().bytes == c.dst)
            pieces.back().bytes += c.bytes;
          else
            pieces.push_back(c);
        }
      }
  int hsa = 0;
  if (mr::sdma_engine_count(&hsa) == 0) {  // before anything is enqueued
    g_last_hip_error = hsa;
    return MR_ERR_ENGINE;
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);  // src is ready
  if (e != hipSuccess) return hip_fail(e);
  if (cu_part) {  // the small parameters' kernel runs on the stream beside the engine copies
    s = gather_launch(*gp, [&](mr::GatherArgs& a) {
      a.src = sb;
      a.out = ob;
    }, needs_realign(gp->rm_mask, reinterpret_cast<uintptr_t>(src) - reinterpret_cast<uintptr_t>(out)), st);
    if (s != MR_OK) return s;
  }
  const int rc = mr::sdma_copy(pieces.data(), pieces.size());
  e = cu_part ? hipStreamSynchronize(st) : hipSuccess;
  if (rc != 0) {
    g_last_hip_error = rc;
    return MR_ERR_ENGINE;
  }
  return e == hipSuccess ? MR_OK : hip_fail(e);
}

// ------------------------------------------------------------------------ planning hooks (mr_probe.h)

int mrx_twoshot_plan(int W, size_t n, int dtype, uintptr_t out_addr, int same_phase, int sync_opt, int shape_opt,
                     int wait_free, uint64_t* f, int nf) {
  if (W < 1 || W > MR_MAX_W || !is_float(static_cast<mr_dtype>(dtype)) || !f || nf < 16) return -1;
  const int es = mr::elem_size(static_cast<mr_dtype>(dtype));
  const mr::ReduceShape sh = reduce_shape(n, es, out_addr, same_phase != 0);
  const mr::TwoShotPlan pl = twoshot_plan_for(W, sh, es, static_cast<uint32_t>(sync_opt), static_cast<uint32_t>(shape_opt),
                                              wait_free != 0);
  const uint64_t v[16] = {pl.xcd, pl.units, pl.run, pl.run_padded, pl.chunks, pl.chunk_units, pl.t1, pl.t2, pl.ratio,
                          pl.unit1, pl.sync, static_cast<uint64_t>(sh.vec), sh.head, sh.npacks, mr::twoshot_grid(pl),
                          mr::twoshot_flag_words(pl)};
  for (int i = 0; i < 16; ++i) f[i] = v[i];
  return 0;
}

int mrx_reduce_shape(const void* const* bufs, int W, size_t n, int dtype, const void* out, uint64_t* f, int nf) {
  if (W < 1 || W > MR_MAX_W || !bufs || !out || !is_float(static_cast<mr_dtype>(dtype)) || !f || nf < 5 + MR_MAX_W)
    return -1;
  const int es = mr::elem_size(static_cast<mr_dtype>(dtype));
  const uintptr_t po = reinterpret_cast<uintptr_t>(out);
  bool same_phase = true, aligned = po % static_cast<uintptr_t>(es) == 0;
  for (int r = 0; r < W; ++r) {
    const uintptr_t pr = reinterpret_cast<uintptr_t>(bufs[r]);
    if ((pr & 15u) != (po & 15u)) same_phase = false;
    if (pr % static_cast<uintptr_t>(es) != 0) aligned = false;
    f[5 + r] = (pr - po) & 15u;
  }
  const mr::ReduceShape sh = reduce_shape(n, es, po, same_phase, aligned);
  f[0] = static_cast<uint64_t>(sh.vec);
  f[1] = static_cast<uint64_t>(sh.realign);
  f[2] = static_cast<uint64_t>(sh.bytes);
  f[3] = sh.head;
  f[4] = sh.npacks;
  return 0;
}

int mrx_gather_phase_masks(int W, int G, const uint64_t* splits, int P, int dtype, uint16_t* rm_mask,
                           uint16_t* rank_masks, int n_rank_masks) {
  if (W < 1 || W > 65535 || !rm_mask || (n_rank_masks && !rank_masks)) return -1;
  GatherPlan gp;
  const mr_status s = gather_plan(W, G, splits, P, static_cast<mr_dtype>(dtype), P > 1, &gp);
  if (s != MR_OK) return s;
  *rm_mask = gp.rm_mask;
  for (int r = 0; r < n_rank_masks; ++r) rank_masks[r] = r < static_cast<int>(gp.rank_mask.size()) ? gp.rank_mask[r] : 0;
  return 0;
}

int mrx_needs_realign(uint16_t mask, uint64_t base_difference) {
  return needs_realign(mask, static_cast<uintptr_t>(base_difference)) ? 1 : 0;
}

int mrx_gather_tiles(int W, int G, const uint64_t* splits, int P, int dtype, uint64_t cu_below, uint32_t* prefix,
                     int n_prefix, uint16_t* rm_mask) {
  if (W < 1 || W > 65535 || P > static_cast<int>(mr::kMaxParams) || !prefix || n_prefix < P + 1 || !rm_mask) return -1;
  GatherPlan gp;
  const mr_status s = gather_plan(W, G, splits, P, static_cast<mr_dtype>(dtype), P > 1, &gp, false, cu_below);
  if (s != MR_OK) return s;
  *rm_mask = gp.rm_mask;
  for (int i = 0; i <= P; ++i) prefix[i] = gp.groups.empty() ? 0 : gp.groups[0].tile_prefix[i];
  return 0;
}

int mr_sdma_engines(void) {
  int status = 0;
  const int count = mr::sdma_engine_count(&status);
  if (count == 0) g_last_hip_error = status;
  return count;
}

mr_status mr_allgather_param_contig_shards(const void* const* shards, int W, int G, const uint64_t* splits, int P,
                                           mr_dtype dtype, void* out, mr_stream stream) {
  if (W < 1 || W > MR_MAX_TABLE_W) return MR_ERR_INVALID_ARG;
  bool on_grid = gather_on_grid(dtype, {out});
  for (int r = 0; shards && r < W; ++r) on_grid = on_grid && gather_on_grid(dtype, {shards[r]});
  const GatherPlan* gp = nullptr;
  mr_status s = cached_gather_plan(W, G, splits, P, dtype, P > 1, &gp, !on_grid);
  if (s != MR_OK || gp->T == 0) return s;
  if (!shards || !out) return MR_ERR_INVALID_ARG;
  const uint64_t shard_bytes = gp->T * gp->es, out_bytes = static_cast<uint64_t>(W) * shard_bytes;
  bool realign = false;
  for (int r = 0; r < W; ++r) {
    if (!shards[r]) return MR_ERR_INVALID_ARG;
    if (overlap(reinterpret_cast<uintptr_t>(shards[r]), shard_bytes, reinterpret_cast<uintptr_t>(out), out_bytes))
      return MR_ERR_ALIAS;
    realign = realign || needs_realign(gp->rank_mask[r], reinterpret_cast<uintptr_t>(shards[r]) -
                                                             reinterpret_cast<uintptr_t>(out));
  }
  return gather_launch(*gp, [&](mr::GatherArgs& a) {
    a.src_table = 1;
    for (int r = 0; r < W; ++r) a.src_tab[r] = static_cast<const char*>(shards[r]);
    a.out = static_cast<char*>(out);
  }, realign, reinterpret_cast<hipStream_t>(stream));
}

mr_status mr_allgather_into_tensor(const void* const* shards, int W, size_t T, mr_dtype dtype, void* out,
                                   mr_stream stream) {
  if (W < 1) return MR_ERR_INVALID_ARG;
  const uint64_t split = T;
  return mr_allgather_param_contig_shards(shards, W, W, &split, 1, dtype, out, stream);
}

mr_status mr_allgather_list(const void* const* shards, int W, size_t T, mr_dtype dtype, void* const* outs,
                            mr_stream stream) {
  if (W < 1 || W > MR_MAX_TABLE_W) return MR_ERR_INVALID_ARG;
  const uint64_t split = T;
  bool on_grid = true;
  for (int i = 0; shards && outs && i < W; ++i) on_grid = on_grid && gather_on_grid(dtype, {shards[i], outs[i]});
  const GatherPlan* gp = nullptr;
  mr_status s = cached_gather_plan(W, W, &split, 1, dtype, false, &gp, !on_grid);
  if (s != MR_OK || gp->T == 0) return s;
  if (!shards || !outs) return MR_ERR_INVALID_ARG;
  const uint64_t bytes = gp->T * gp->es;
  bool realign = false;
  for (int i = 0; i < W; ++i) {
    if (!shards[i] || !outs[i]) return MR_ERR_INVALID_ARG;
    realign = realign || ((reinterpret_cast<uintptr_t>(shards[i]) - reinterpret_cast<uintptr_t>(outs[i])) & 15u) != 0;
    for (int j = 0; j < W; ++j) {
      const uintptr_t oi = reinterpret_cast<uintptr_t>(outs[i]);
      if (overlap(oi, bytes, reinterpret_cast<uintptr_t>(shards[j]), bytes)) return MR_ERR_ALIAS;
      if (j != i && overlap(oi, bytes, reinterpret_cast<uintptr_t>(outs[j]), bytes)) return MR_ERR_ALIAS;
    }
  }
  return gather_launch(*gp, [&](mr::GatherArgs& a) {
    a.src_table = 1;
    a.dst_table = 1;
    for (int r = 0; r < W; ++r) {
      a.src_tab[r] = static_cast<const char*>(shards[r]);
      a.dst_tab[r] = static_cast<char*>(outs[r]);
    }
  }, realign, reinterpret_cast<hipStream_t>(stream));
}

mr_status mr_set_workspace(mr_stream stream, void* dev_ptr, size_t bytes) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dev_ptr && (bytes < mr::ws_stage_offset(bytes) + 256 || (reinterpret_cast<uintptr_t>(dev_ptr) % 256) != 0))
    return MR_ERR_INVALID_ARG;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_ws_mu);
  // every library-owned buffer of this stream: its own workspace, those of captures made on it, and
  // the ones growth replaced
  std::vector<char*> owned = std::move(g_retired[{dev, st}]);
  g_retired.erase({dev, st});
  for (auto it = g_ws.begin(); it != g_ws.end();) {
    if (std::get<0>(it->first) == dev && std::get<1>(it->first) == st) {
      if (it->second.base && it->second.owned) owned.push_back(it->second.base);
      it = g_ws.erase(it);
    } else {
      ++it;
    }
  }
  if (!owned.empty()) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      g_retired[{dev, st}] = std::move(owned);  // nothing freed; the stream is left unbound
      return hip_fail(e);
    }
    // every buffer is released even if one free fails; the first failure is reported and the stream is
    // left unbound (the buffers are dropped either way, never freed twice)
    hipError_t fe = hipSuccess;
    for (char* b : owned) {
      const hipError_t f = hipFree(b);
      if (fe == hipSuccess) fe = f;
    }
    if (fe != hipSuccess) return hip_fail(fe);
  }
  Workspace& w = g_ws[WsKey{dev, st, 0}];
  if (!dev_ptr) return MR_OK;
  e = ws_clear(static_cast<char*>(dev_ptr), bytes, st);
  if (e != hipSuccess) return hip_fail(e);
  w.base = static_cast<char*>(dev_ptr);
  w.bytes = bytes;
  w.owned = false;
  return MR_OK;
}

mr_status mr_workspace_check(mr_stream stream, uint32_t* flags) {
  if (!flags) return MR_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::vector<Workspace> ws;  // the stream's own workspace and those of captures made on it
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    for (const auto& kv : g_ws)
      if (std::get<0>(kv.first) == dev && std::get<1>(kv.first) == st && kv.second.base) ws.push_back(kv.second);
  }
  if (ws.empty()) return MR_ERR_WORKSPACE;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  uint32_t all = 0;
  for (const Workspace& w : ws) {
    uint32_t err = 0;
    e = hipMemcpy(&err, w.base + offsetof(mr::Ctrl, err), sizeof(err), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
    all |= err;
    // clear the error word and every barrier word and flag (each launch re-arms them itself; this
    // also resets a workspace that a caller's own kernels may have written)
    e = ws_clear(w.base, w.bytes, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  *flags = all;
  return MR_OK;
}

}  // extern "C"
