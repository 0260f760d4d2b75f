// W-way elementwise sum-reduce kernels for gfx950: one-shot and two-shot.
//
// The sum is the one a custom all-reduce forms per element (page "Question and suggestions about
// custom allreduce": the quoted one-shot schedule pulls a chunk from every peer and sums it; the same
// page's two-shot question: reduce-scatter, then gather).  Each term is widened exactly to fp32 and
// added in rank order 0..W-1 with fp32 round-to-nearest-even adds; the sum is rounded to nearest even
// into the buffer dtype.  The work is HBM streaming (W+1 bytes moved per element byte, at most W-1
// adds per element), so the kernels are shaped for memory-level parallelism: one 16-byte load per
// lane per rank buffer, all W loads of U packs issued before any arithmetic, wave64 workgroups of 256
// lanes, non-temporal hints because no byte is touched twice.  No LDS, no MFMA.

#include "mr_internal.h"

namespace mr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------- dtype traits

// bf16 = upper half of an fp32.  Narrowing adds 0x7fff plus the lowest kept bit and drops 16 bits:
// the carry rounds up exactly when the dropped half exceeds one half, or equals it with an odd kept
// part (round to nearest, ties to even); a carry out of the fraction steps the exponent, which turns
// values past the largest bf16 into infinity.  NaN keeps its sign and top payload and becomes quiet.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}

struct Bf16 {
  static constexpr int kSize = 2;
  static constexpr int V = 8;
  __device__ static float load1(const char* p) {
    return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
  }
  __device__ static void store1(char* p, float f) {
    *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(bf16_rne(f));
  }
  __device__ static void widen(const u32x4& w, float (&f)[V]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static u32x4 narrow(const float (&f)[V]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_rne(f[2 * i]) | (bf16_rne(f[2 * i + 1]) << 16);
    return w;
  }
};

// fp16 <-> fp32 through the hardware converts: exact widening, round-to-nearest-even narrowing
// (the default rounding mode) with fp16 subnormals kept (the default fp16 denormal mode).
struct Fp16 {
  static constexpr int kSize = 2;
  static constexpr int V = 8;
  __device__ static float h2f(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  __device__ static uint32_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
  __device__ static float load1(const char* p) { return h2f(*reinterpret_cast<const uint16_t*>(p)); }
  __device__ static void store1(char* p, float f) { *reinterpret_cast<uint16_t*>(p) = f2h(f); }
  __device__ static void widen(const u32x4& w, float (&f)[V]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = h2f(w[i] & 0xffffu);
      f[2 * i + 1] = h2f(w[i] >> 16);
    }
  }
  __device__ static u32x4 narrow(const float (&f)[V]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f2h(f[2 * i]) | (f2h(f[2 * i + 1]) << 16);
    return w;
  }
};

struct Fp32 {
  static constexpr int kSize = 4;
  static constexpr int V = 4;
  __device__ static float load1(const char* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static void store1(char* p, float f) { *reinterpret_cast<float*>(p) = f; }
  __device__ static void widen(const u32x4& w, float (&f)[V]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  __device__ static u32x4 narrow(const float (&f)[V]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
    return w;
  }
};

// ---------------------------------------------------------------------------------- shared bodies

// One element, any alignment: fp32 accumulation in rank order.
template <typename D, int W>
__device__ __forceinline__ void reduce_elem(const RankPtrs& in, char* dst, size_t e) {
  const size_t off = e * D::kSize;
  float acc = D::load1(in.p[0] + off);
#pragma unroll
  for (int r = 1; r < W; ++r) acc = acc + D::load1(in.p[r] + off);
  D::store1(dst + off, acc);
}

// U packs per lane, lane-interleaved: pack index i = first + u*kBlock + lane, for i < end.
// All W*U loads are issued before the first add so they are in flight together.
template <typename D, int W, int U>
__device__ __forceinline__ void reduce_packs(const RankPtrs& in, size_t head, char* dst, size_t first,
                                             size_t end) {
  const size_t hb = head * D::kSize;
  u32x4 v[U][W];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (i < end) {
#pragma unroll
      for (int r = 0; r < W; ++r)
        v[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in.p[r] + hb) + i);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (i < end) {
      float acc[D::V];
      D::widen(v[u][0], acc);
#pragma unroll
      for (int r = 1; r < W; ++r) {
        float t[D::V];
        D::widen(v[u][r], t);
#pragma unroll
        for (int k = 0; k < D::V; ++k) acc[k] = acc[k] + t[k];
      }
      __builtin_nontemporal_store(D::narrow(acc), reinterpret_cast<u32x4*>(dst + hb) + i);
    }
  }
}

template <int U>
__device__ __forceinline__ void copy_packs(const char* src, char* dst, size_t hb, size_t first, size_t end) {
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (i < end) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + hb) + i);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (i < end) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst + hb) + i);
  }
}

// Elements outside the 16-byte body: [0, head) and [head + npacks*V, n).  At most 2V-2 of them.
template <typename D, int W>
__device__ __forceinline__ void reduce_edges(const RankPtrs& in, char* dst, const ReduceShape& sh) {
  const size_t tail0 = sh.head + sh.npacks * D::V;
  const size_t count = sh.head + (sh.n - tail0);
  for (size_t k = threadIdx.x; k < count; k += kBlock) reduce_elem<D, W>(in, dst, k < sh.head ? k : tail0 + (k - sh.head));
}

template <typename D>
__device__ __forceinline__ void copy_edges(const char* src, char* dst, const ReduceShape& sh) {
  const size_t tail0 = sh.head + sh.npacks * D::V;
  const size_t count = sh.head + (sh.n - tail0);
  for (size_t k = threadIdx.x; k < count; k += kBlock) {
    const size_t off = (k < sh.head ? k : tail0 + (k - sh.head)) * D::kSize;
    if (D::kSize == 2)
      *reinterpret_cast<uint16_t*>(dst + off) = *reinterpret_cast<const uint16_t*>(src + off);
    else
      *reinterpret_cast<uint32_t*>(dst + off) = *reinterpret_cast<const uint32_t*>(src + off);
  }
}

// ---------------------------------------------------------------------------------------- one-shot

constexpr int kOneShotU = 2;  // packs per lane per tile

template <typename D, int W>
__global__ __launch_bounds__(kBlock) void oneshot_vec(RankPtrs in, char* out, ReduceShape sh, size_t ntiles) {
  constexpr size_t kTile = static_cast<size_t>(kBlock) * kOneShotU;
  for (size_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const size_t first = t * kTile;
    reduce_packs<D, W, kOneShotU>(in, sh.head, out, first, sh.npacks);
  }
  if (blockIdx.x == 0) reduce_edges<D, W>(in, out, sh);
}

template <typename D, int W>
__global__ __launch_bounds__(kBlock) void oneshot_elem(RankPtrs in, char* out, size_t n) {
  for (size_t e = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * kBlock)
    reduce_elem<D, W>(in, out, e);
}

// ---------------------------------------------------------------------------------------- two-shot
//
// Phase 1 (reduce-scatter): chunk c of the message, c = 0..W-1, is reduced tile by tile into the
// stage buffer.  Phase 2 (gather-copy): the stage is copied into out, chunks taken in the reverse
// order, so a phase-2 workgroup copies bytes other workgroups reduced.
//
// Ordering the phases.  Workgroups take a ticket from an atomic counter when they start; tickets
// below n1 do phase-1 tiles, the rest phase-2 tiles.  A phase-1 workgroup releases its stores with an
// agent-scope release increment of done1 (after a workgroup barrier, so every lane's stores are in
// its XCD's L2 before the release writes them back).  A phase-2 workgroup acquire-waits until done1
// reaches n1.  Because tickets follow start order, every phase-1 tile belongs to a workgroup that
// already runs and never waits, so the wait ends whether or not the whole grid is co-resident (no
// reliance on workgroup 0 starting first, nor on two such kernels never sharing the GPU).  The wait
// is bounded all the same: past spin_limit polls it sets an error bit and goes on.  Words reset
// themselves: the holder of the last ticket clears `claim`, the last phase-2 workgroup clears done1
// and done2, so consecutive launches on one stream need no host-side reset.

constexpr int kTwoShotU1 = 2;  // packs per lane per phase-1 tile
constexpr int kTwoShotU2 = 8;  // packs per lane per phase-2 tile

__device__ __forceinline__ uint32_t take_ticket(Ctrl* ctrl, uint32_t total) {
  __shared__ uint32_t s_ticket;
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(&ctrl->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == total - 1) __hip_atomic_store(&ctrl->claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ticket = t;
  }
  __syncthreads();
  return s_ticket;
}

__device__ __forceinline__ void release_phase1(Ctrl* ctrl) {
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&ctrl->done1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_phase1(Ctrl* ctrl, uint32_t n1, uint32_t spin_limit) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (__hip_atomic_load(&ctrl->done1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n1) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > spin_limit) {
        __hip_atomic_fetch_or(&ctrl->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

__device__ __forceinline__ void finish_phase2(Ctrl* ctrl, uint32_t n2) {
  if (threadIdx.x == 0) {
    const uint32_t d = __hip_atomic_fetch_add(&ctrl->done2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == n2 - 1) {
      __hip_atomic_store(&ctrl->done1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->done2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename D, int W>
__global__ __launch_bounds__(kBlock) void twoshot_vec(RankPtrs in, char* out, char* stage, Ctrl* ctrl,
                                                      ReduceShape sh, TwoShotPlan pl) {
  const uint32_t t = take_ticket(ctrl, pl.n1 + pl.n2);
  const size_t hb = sh.head * D::kSize;
  if (t < pl.n1) {
    const uint32_t c = t / pl.tiles1_per_chunk, k = t % pl.tiles1_per_chunk;
    const size_t c0 = static_cast<size_t>(c) * pl.chunk_packs;
    const size_t c1 = c0 + pl.chunk_packs < sh.npacks ? c0 + pl.chunk_packs : sh.npacks;
    reduce_packs<D, W, kTwoShotU1>(in, sh.head, stage, c0 + static_cast<size_t>(k) * kBlock * kTwoShotU1, c1);
    if (t == 0) reduce_edges<D, W>(in, stage, sh);
    release_phase1(ctrl);
  } else {
    const uint32_t q = t - pl.n1;
    acquire_phase1(ctrl, pl.n1, pl.spin_limit);
    const uint32_t c = (pl.chunks - 1) - q / pl.tiles2_per_chunk, k = q % pl.tiles2_per_chunk;
    const size_t c0 = static_cast<size_t>(c) * pl.chunk_packs;
    const size_t c1 = c0 + pl.chunk_packs < sh.npacks ? c0 + pl.chunk_packs : sh.npacks;
    copy_packs<kTwoShotU2>(stage, out, hb, c0 + static_cast<size_t>(k) * kBlock * kTwoShotU2, c1);
    if (q == 0) copy_edges<D>(stage, out, sh);
    finish_phase2(ctrl, pl.n2);
  }
}

// Element-wise two-shot for pointers that do not share one 16-byte alignment (V = 1).
template <typename D, int W>
__global__ __launch_bounds__(kBlock) void twoshot_elem(RankPtrs in, char* out, char* stage, Ctrl* ctrl,
                                                       ReduceShape sh, TwoShotPlan pl) {
  const uint32_t t = take_ticket(ctrl, pl.n1 + pl.n2);
  if (t < pl.n1) {
    const uint32_t c = t / pl.tiles1_per_chunk, k = t % pl.tiles1_per_chunk;
    const size_t c0 = static_cast<size_t>(c) * pl.chunk_packs;
    const size_t c1 = c0 + pl.chunk_packs < sh.n ? c0 + pl.chunk_packs : sh.n;
    const size_t first = c0 + static_cast<size_t>(k) * kBlock * kTwoShotU1;
#pragma unroll
    for (int u = 0; u < kTwoShotU1; ++u) {
      const size_t e = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
      if (e < c1) reduce_elem<D, W>(in, stage, e);
    }
    release_phase1(ctrl);
  } else {
    const uint32_t q = t - pl.n1;
    acquire_phase1(ctrl, pl.n1, pl.spin_limit);
    const uint32_t c = (pl.chunks - 1) - q / pl.tiles2_per_chunk, k = q % pl.tiles2_per_chunk;
    const size_t c0 = static_cast<size_t>(c) * pl.chunk_packs;
    const size_t c1 = c0 + pl.chunk_packs < sh.n ? c0 + pl.chunk_packs : sh.n;
    const size_t first = c0 + static_cast<size_t>(k) * kBlock * kTwoShotU2;
#pragma unroll
    for (int u = 0; u < kTwoShotU2; ++u) {
      const size_t e = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
      if (e < c1) {
        const size_t off = e * D::kSize;
        if (D::kSize == 2)
          *reinterpret_cast<uint16_t*>(out + off) = *reinterpret_cast<const uint16_t*>(stage + off);
        else
          *reinterpret_cast<uint32_t*>(out + off) = *reinterpret_cast<const uint32_t*>(stage + off);
      }
    }
    finish_phase2(ctrl, pl.n2);
  }
}

__global__ void zero_ctrl(Ctrl* ctrl) {
  reinterpret_cast<uint32_t*>(ctrl)[threadIdx.x] = 0u;
}

// ------------------------------------------------------------------------------------- dispatch

constexpr size_t kMaxGrid = size_t(1) << 22;  // workgroups; beyond this the one-shot kernels grid-stride

template <typename D, int W>
hipError_t oneshot_w(const RankPtrs& in, char* out, const ReduceShape& sh, hipStream_t st) {
  if (sh.vec) {
    const size_t tile = static_cast<size_t>(kBlock) * kOneShotU;
    const size_t ntiles = (sh.npacks + tile - 1) / tile;
    size_t grid = ntiles < kMaxGrid ? ntiles : kMaxGrid;
    if (grid == 0) grid = 1;  // edges only
    hipLaunchKernelGGL((oneshot_vec<D, W>), dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, st, in, out, sh, ntiles);
  } else {
    const size_t need = (sh.n + kBlock - 1) / kBlock;
    const size_t grid = need < kMaxGrid ? need : kMaxGrid;
    hipLaunchKernelGGL((oneshot_elem<D, W>), dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, st, in, out, sh.n);
  }
  return hipGetLastError();
}

template <typename D, int W>
hipError_t twoshot_w(const RankPtrs& in, char* out, char* stage, Ctrl* ctrl, const ReduceShape& sh,
                     const TwoShotPlan& pl, hipStream_t st) {
  const unsigned grid = pl.n1 + pl.n2;
  if (sh.vec)
    hipLaunchKernelGGL((twoshot_vec<D, W>), dim3(grid), dim3(kBlock), 0, st, in, out, stage, ctrl, sh, pl);
  else
    hipLaunchKernelGGL((twoshot_elem<D, W>), dim3(grid), dim3(kBlock), 0, st, in, out, stage, ctrl, sh, pl);
  return hipGetLastError();
}

#define MR_W_CASES(F, D, ...)       \
  switch (W) {                      \
    case 1: return F<D, 1>(__VA_ARGS__);   \
    case 2: return F<D, 2>(__VA_ARGS__);   \
    case 3: return F<D, 3>(__VA_ARGS__);   \
    case 4: return F<D, 4>(__VA_ARGS__);   \
    case 5: return F<D, 5>(__VA_ARGS__);   \
    case 6: return F<D, 6>(__VA_ARGS__);   \
    case 7: return F<D, 7>(__VA_ARGS__);   \
    case 8: return F<D, 8>(__VA_ARGS__);   \
    case 9: return F<D, 9>(__VA_ARGS__);   \
    case 10: return F<D, 10>(__VA_ARGS__); \
    case 11: return F<D, 11>(__VA_ARGS__); \
    case 12: return F<D, 12>(__VA_ARGS__); \
    case 13: return F<D, 13>(__VA_ARGS__); \
    case 14: return F<D, 14>(__VA_ARGS__); \
    case 15: return F<D, 15>(__VA_ARGS__); \
    case 16: return F<D, 16>(__VA_ARGS__); \
    default: return hipErrorInvalidValue;  \
  }

template <typename D>
hipError_t oneshot_d(const RankPtrs& in, int W, char* out, const ReduceShape& sh, hipStream_t st) {
  MR_W_CASES(oneshot_w, D, in, out, sh, st)
}

template <typename D>
hipError_t twoshot_d(const RankPtrs& in, int W, char* out, char* stage, Ctrl* ctrl, const ReduceShape& sh,
                     const TwoShotPlan& pl, hipStream_t st) {
  MR_W_CASES(twoshot_w, D, in, out, stage, ctrl, sh, pl, st)
}

}  // namespace

hipError_t launch_oneshot(const RankPtrs& in, int W, mr_dtype dt, char* out, const ReduceShape& sh,
                          hipStream_t st) {
  switch (dt) {
    case MR_BF16: return oneshot_d<Bf16>(in, W, out, sh, st);
    case MR_FP16: return oneshot_d<Fp16>(in, W, out, sh, st);
    case MR_FP32: return oneshot_d<Fp32>(in, W, out, sh, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_twoshot(const RankPtrs& in, int W, mr_dtype dt, char* out, char* stage, Ctrl* ctrl,
                          const ReduceShape& sh, const TwoShotPlan& pl, hipStream_t st) {
  switch (dt) {
    case MR_BF16: return twoshot_d<Bf16>(in, W, out, stage, ctrl, sh, pl, st);
    case MR_FP16: return twoshot_d<Fp16>(in, W, out, stage, ctrl, sh, pl, st);
    case MR_FP32: return twoshot_d<Fp32>(in, W, out, stage, ctrl, sh, pl, st);
    default: return hipErrorInvalidValue;
  }
}

// Chunk c holds ceil(units / W) consecutive 16-byte packs of the body (elements on the element-wise
// path), so every chunk boundary is 16-byte aligned and, when n is a multiple of the pack, chunk c is
// exactly elements [c*C, (c+1)*C) with C = ceil(n/W) rounded up to a whole pack.  The last chunks may
// be short or empty.  The few elements outside the body (an unaligned head, a tail shorter than a
// pack) ride with the first tile of each phase.
TwoShotPlan plan_twoshot(int W, const ReduceShape& sh, uint32_t spin_limit) {
  TwoShotPlan pl{};
  pl.chunks = static_cast<uint32_t>(W);
  const size_t units = sh.vec ? sh.npacks : sh.n;
  pl.chunk_packs = (units + W - 1) / W;
  const size_t t1 = static_cast<size_t>(kBlock) * kTwoShotU1;
  const size_t t2 = static_cast<size_t>(kBlock) * kTwoShotU2;
  size_t tiles1 = (pl.chunk_packs + t1 - 1) / t1;
  size_t tiles2 = (pl.chunk_packs + t2 - 1) / t2;
  if (tiles1 == 0) tiles1 = 1;  // an edges-only call still needs one tile of each phase
  if (tiles2 == 0) tiles2 = 1;
  pl.tiles1_per_chunk = static_cast<uint32_t>(tiles1);
  pl.tiles2_per_chunk = static_cast<uint32_t>(tiles2);
  pl.n1 = static_cast<uint32_t>(tiles1 * W);
  pl.n2 = static_cast<uint32_t>(tiles2 * W);
  pl.spin_limit = spin_limit;
  return pl;
}

hipError_t launch_zero_ctrl(Ctrl* ctrl, hipStream_t st) {
  hipLaunchKernelGGL(zero_ctrl, dim3(1), dim3(kCtrlBytes / 4), 0, st, ctrl);
  return hipGetLastError();
}

}  // namespace mr
