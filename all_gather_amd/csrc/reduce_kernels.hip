// W-way elementwise sum-reduce kernels for gfx950: one-shot and two-shot.
//
// The sum is the one a custom all-reduce forms per element (page "Question and suggestions about
// custom allreduce": the quoted one-shot schedule pulls a chunk from every peer and sums it; the same
// page's two-shot question: reduce-scatter, then gather).  Each term is widened exactly to fp32 and
// added in rank order 0..W-1 with fp32 round-to-nearest-even adds; the sum is rounded to nearest even
// into the buffer dtype.  The work is HBM streaming ((W+1) bytes moved per output byte, at most W-1
// adds per element), so the kernels are shaped for memory-level parallelism: one 16-byte load per
// lane per rank buffer, all of a lane's loads issued before any arithmetic, large workgroups (fewer
// groups to dispatch and drain), non-temporal hints because no byte is touched twice.  No LDS, no MFMA.

#include "mr_internal.h"

namespace mr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer loads/stores, used for the two-shot stage because they carry an explicit cache policy.
__device__ i32x4 raw_buffer_load_v4(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ void raw_buffer_store_v4(i32x4 data, i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i32");

// Cache policy of the stage accesses: sc1, device-scope coherence (stores write through the XCD's
// L2, loads do not return a line another XCD may have changed).  Adding nt measured 2-3% slower.
#ifndef MR_TS_STORE_AUX
#define MR_TS_STORE_AUX (1 << 4)
#endif
#ifndef MR_TS_LOAD_AUX
#define MR_TS_LOAD_AUX (1 << 4)
#endif
#ifndef MR_TS_RATIO
#define MR_TS_RATIO 4
#endif
constexpr int kStageStoreAux = MR_TS_STORE_AUX;
constexpr int kStageLoadAux = MR_TS_LOAD_AUX;

// Buffer resource for `bytes` bytes at `base` (raw, stride 0; gfx9 data-format word).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = static_cast<int32_t>(static_cast<uint32_t>(a));
  r[1] = static_cast<int32_t>((a >> 32) & 0xffffu);
  r[2] = static_cast<int32_t>(bytes);
  r[3] = 0x00020000;
  return r;
}

// ------------------------------------------------------------------------------------- dtype traits

// bf16 = upper half of an fp32, so widening is a shift.  Narrowing uses gfx950's packed convert
// (v_cvt_pk_bf16_f32: two fp32 to two bf16, round to nearest even under the default rounding mode,
// subnormals kept under the fp32 denormal mode this library is built with, values past the largest bf16
// to infinity).  It replaced an integer rounding (add 0x7fff plus the lowest kept bit, drop 16 bits)
// that cost several ALU operations per element: same-GPU A/B of the W=8 one-shot, three interleaved
// repeats, 16 MiB per rank 26.1-26.3 -> 25.6-25.7 us, 256 KiB 2.40 -> 2.27 us, 1 MiB 3.46 -> 3.30 us.
// NaN stays NaN (its payload is not part of the contract).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

struct Bf16 {
  static constexpr int kSize = 2;
  static constexpr int V = 8;
  __device__ static float widen1(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static uint32_t narrow1(float f) { return bf16x2_rne(f, 0.0f) & 0xffffu; }
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
    for (int i = 0; i < 4; ++i) w[i] = bf16x2_rne(f[2 * i], f[2 * i + 1]);
    return w;
  }
};

// fp16 <-> fp32 through the hardware converts: exact widening, round-to-nearest-even narrowing
// (the default rounding mode) with fp16 subnormals kept (the default fp16 denormal mode).
struct Fp16 {
  static constexpr int kSize = 2;
  static constexpr int V = 8;
  __device__ static float widen1(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  __device__ static uint32_t narrow1(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }
  __device__ static void widen(const u32x4& w, float (&f)[V]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = widen1(w[i] & 0xffffu);
      f[2 * i + 1] = widen1(w[i] >> 16);
    }
  }
  __device__ static u32x4 narrow(const float (&f)[V]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = narrow1(f[2 * i]) | (narrow1(f[2 * i + 1]) << 16);
    return w;
  }
};

struct Fp32 {
  static constexpr int kSize = 4;
  static constexpr int V = 4;
  __device__ static float widen1(uint32_t b) { return __uint_as_float(b); }
  __device__ static uint32_t narrow1(float f) { return __float_as_uint(f); }
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

// Raw element bits.  `Dev` accesses are relaxed agent-scope atomics: device-coherent (sc1) loads and
// write-through stores, used for the two-shot stage.
template <int S, bool Dev>
__device__ __forceinline__ uint32_t load_bits(const char* p) {
  if (S == 2) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return Dev ? __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *q;
  }
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  return Dev ? __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *q;
}
template <int S, bool Dev>
__device__ __forceinline__ void store_bits(char* p, uint32_t b) {
  if (S == 2) {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
    if (Dev) __hip_atomic_store(q, static_cast<uint16_t>(b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *q = static_cast<uint16_t>(b);
    return;
  }
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  if (Dev) __hip_atomic_store(q, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *q = b;
}

// Element bits through single-byte accesses only (pointers that are not multiples of the element size:
// no unaligned multi-byte access is ever issued).  Little-endian, as the element's bytes sit in memory.
template <int S>
__device__ __forceinline__ uint32_t load_bytes(const char* p) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < S; ++i) v |= static_cast<uint32_t>(static_cast<uint8_t>(p[i])) << (8 * i);
  return v;
}
template <int S>
__device__ __forceinline__ void store_bytes(char* p, uint32_t v) {
#pragma unroll
  for (int i = 0; i < S; ++i) p[i] = static_cast<char>(static_cast<uint8_t>(v >> (8 * i)));
}

// ---------------------------------------------------------------------------------- shared bodies

// One element: fp32 accumulation in rank order.  BYTES: inputs read (and out written, unless Dev) one
// byte at a time; Dev: written to the stage with a device-coherent store (the stage is always aligned).
template <typename D, int W, bool Dev, bool BYTES = false>
__device__ __forceinline__ void reduce_elem(const RankPtrs& in, char* dst, size_t e) {
  const size_t off = e * D::kSize;
  auto ld = [&](const char* q) { return BYTES ? load_bytes<D::kSize>(q) : load_bits<D::kSize, false>(q); };
  float acc = D::widen1(ld(in.p[0] + off));
#pragma unroll
  for (int r = 1; r < W; ++r) acc = acc + D::widen1(ld(in.p[r] + off));
  if (BYTES && !Dev) store_bytes<D::kSize>(dst + off, D::narrow1(acc));
  else store_bits<D::kSize, Dev>(dst + off, D::narrow1(acc));
}

// Bytes d .. d+15 of the 32 bytes A:B (d the same in every lane), with selects only: no branch, so the
// loads of every rank can be in flight before any realignment.  Used for an input whose 16-byte phase is
// d bytes past out's: A and B are the two aligned packs an output pack's bytes straddle.
__device__ __forceinline__ u32x4 realign_rt(const u32x4& A, const u32x4& B, uint32_t d) {
  const bool h8 = (d & 8u) != 0, h4 = (d & 4u) != 0;
  const uint32_t w0 = h8 ? A[2] : A[0], w1 = h8 ? A[3] : A[1], w2 = h8 ? B[0] : A[2];
  const uint32_t w3 = h8 ? B[1] : A[3], w4 = h8 ? B[2] : B[0], w5 = h8 ? B[3] : B[1];
  const uint32_t x0 = h4 ? w1 : w0, x1 = h4 ? w2 : w1, x2 = h4 ? w3 : w2, x3 = h4 ? w4 : w3, x4 = h4 ? w5 : w4;
  const uint32_t sh = d & 3u;
  u32x4 o;
  o[0] = __builtin_amdgcn_alignbyte(x1, x0, sh);
  o[1] = __builtin_amdgcn_alignbyte(x2, x1, sh);
  o[2] = __builtin_amdgcn_alignbyte(x3, x2, sh);
  o[3] = __builtin_amdgcn_alignbyte(x4, x3, sh);
  return o;
}

// The two aligned packs that output pack i (on out's 16-byte grid) of rank r straddles, for an input
// in.shift[r] = d bytes past out's phase.  The second is pack i + 1 when d != 0 -- it then holds bytes of
// the output pack itself, so no load leaves the input's pages -- and pack i again when d == 0, so the
// address needs no branch.
__device__ __forceinline__ void load_pack_pair(const RankPtrs& in, int r, size_t hb, size_t i, u32x4& a, u32x4& b) {
  const uint32_t d = in.shift[r];
  const u32x4* base = reinterpret_cast<const u32x4*>(in.p[r] + hb - d);
  a = __builtin_nontemporal_load(base + i);
  b = base[i + (d != 0 ? 1 : 0)];
}

// Neighbour packs on the realigned path.  In the wave-contiguous layout below, lane l's pack u is pack
// i, and pack i + 1 is lane l + 1's pack u or, for lane 63, lane 0's pack u + 1: so the second aligned
// pack an output pack straddles is moved over from the neighbouring lane instead of loaded again.
// wave_shl:1 gives lane l the value of lane l + 1 and leaves lane 63 at `old`; wave_rol:1 gives lane 63
// the value of lane 0.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), 0x130, 0xf, 0xf, false));
}
__device__ __forceinline__ uint32_t lane0_to_lane63(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x134, 0xf, 0xf, false));
}

// Wave-contiguous tile layout: a workgroup of B lanes owns B*P consecutive 16-byte packs starting at
// `first`; wave w owns P*64 of them and lane l's u-th pack is first + w*64*P + u*64 + l, so each wave
// instruction covers 1 KiB and a wave's P instructions for one rank cover P KiB contiguous.
template <int B, int P>
__device__ __forceinline__ size_t wc_pack(size_t first, int u) {
  return first + static_cast<size_t>(threadIdx.x >> 6) * (64 * P) + static_cast<size_t>(u) * 64 + (threadIdx.x & 63);
}

// Realigned inputs, a full tile: every lane loads the aligned pack its output pack starts in (rank by
// rank, all in flight), lane 63 also the one after its last pack; the second aligned pack of each is
// then taken from the neighbouring lane (see from_next_lane).  A tile that reaches past the body's end
// (one per launch at most), and every tile for W > 8 (whose loads would not fit the registers), loads
// both aligned packs of every output pack, one row at a time.
template <typename D, int W, int B, int P, typename Store>
__device__ __forceinline__ void reduce_tile_realigned(const RankPtrs& in, size_t hb, size_t first, size_t end,
                                                      Store st) {
  if constexpr (W <= 8) {
  if (first + static_cast<size_t>(B) * P <= end) {
    const bool l63 = (threadIdx.x & 63) == 63;
    u32x4 v[P][W];
    u32x4 nxt[W];
#pragma unroll
    for (int r = 0; r < W; ++r) {
      const uint32_t d = in.shift[r];
      const u32x4* base = reinterpret_cast<const u32x4*>(in.p[r] + hb - d);
#pragma unroll
      for (int u = 0; u < P; ++u) v[u][r] = __builtin_nontemporal_load(base + wc_pack<B, P>(first, u));
      nxt[r] = u32x4{0u, 0u, 0u, 0u};
      // the pack after lane 63's last one holds bytes of that lane's output pack when d != 0
      if (l63) nxt[r] = base[wc_pack<B, P>(first, P - 1) + (d != 0 ? 1 : 0)];
    }
#pragma unroll
    for (int u = 0; u < P; ++u) {
      auto pack = [&](int r) {
        u32x4 b;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          b[k] = from_next_lane(u + 1 < P ? lane0_to_lane63(v[u + 1 < P ? u + 1 : u][r][k]) : nxt[r][k], v[u][r][k]);
        return realign_rt(v[u][r], b, in.shift[r]);
      };
      float acc[D::V];
      D::widen(pack(0), acc);
#pragma unroll
      for (int r = 1; r < W; ++r) {
        float t[D::V];
        D::widen(pack(r), t);
#pragma unroll
        for (int k = 0; k < D::V; ++k) acc[k] = acc[k] + t[k];
      }
      st(u, wc_pack<B, P>(first, u), D::narrow(acc));
    }
    return;
  }
  }
#pragma unroll 1
  for (int u = 0; u < P; ++u) {
    const size_t i = wc_pack<B, P>(first, u);
    if (i < end) {
      u32x4 a[W], b[W];
#pragma unroll
      for (int r = 0; r < W; ++r) load_pack_pair(in, r, hb, i, a[r], b[r]);
      float acc[D::V];
      D::widen(realign_rt(a[0], b[0], in.shift[0]), acc);
#pragma unroll
      for (int r = 1; r < W; ++r) {
        float t[D::V];
        D::widen(realign_rt(a[r], b[r], in.shift[r]), t);
#pragma unroll
        for (int k = 0; k < D::V; ++k) acc[k] = acc[k] + t[k];
      }
      st(u, i, D::narrow(acc));
    }
  }
}

// Reduce a wave-contiguous tile of B*P packs (i < end), PC packs at a time: all W*PC loads in flight,
// rank by rank, before the adds; each result goes to st(u, i, pack).
// One pack's sum over the W ranks: widened to fp32, added in rank order, narrowed (the arithmetic of
// reduce_tile, for kernels that issue their loads apart from the sums).
template <typename D, int W>
__device__ __forceinline__ u32x4 sum_ranks(const u32x4 (&v)[W]) {
  float acc[D::V];
  D::widen(v[0], acc);
#pragma unroll
  for (int r = 1; r < W; ++r) {
    float t[D::V];
    D::widen(v[r], t);
#pragma unroll
    for (int k = 0; k < D::V; ++k) acc[k] = acc[k] + t[k];
  }
  return D::narrow(acc);
}

template <typename D, int W, int B, int P, typename Store, bool RA = false, bool FULL = false>
__device__ __forceinline__ void reduce_tile(const RankPtrs& in, size_t hb, size_t first, size_t end, Store st) {
  if constexpr (RA) {
    reduce_tile_realigned<D, W, B, P, Store>(in, hb, first, end, st);
    return;
  }
  constexpr int PC = (W <= 8 || P == 1) ? P : 2;  // wide W: fewer packs in flight per lane
  static_assert(P % PC == 0, "pack groups");
  if (FULL && first + static_cast<size_t>(B) * P <= end) {
    // A tile wholly inside the packs, without per-lane checks: straight-line code, so the compiler
    // waits for each rank's packs in turn and the sums start while later loads are in flight.
#pragma unroll
    for (int u0 = 0; u0 < P; u0 += PC) {
      u32x4 v[PC][W];
#pragma unroll
      for (int r = 0; r < W; ++r)
#pragma unroll
        for (int u = 0; u < PC; ++u)
          v[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in.p[r] + hb) + wc_pack<B, P>(first, u0 + u));
#pragma unroll
      for (int u = 0; u < PC; ++u) st(u0 + u, wc_pack<B, P>(first, u0 + u), sum_ranks<D, W>(v[u]));
    }
    return;
  }
#pragma unroll
  for (int u0 = 0; u0 < P; u0 += PC) {
    u32x4 v[PC][W];
    u32x4 vb[RA ? PC : 1][RA ? W : 1];  // RA: the second aligned pack of each
#pragma unroll
    for (int r = 0; r < W; ++r)
#pragma unroll
      for (int u = 0; u < PC; ++u) {
        const size_t i = wc_pack<B, P>(first, u0 + u);
        if (i < end) {
          if constexpr (RA) load_pack_pair(in, r, hb, i, v[u][r], vb[u][r]);
          else v[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in.p[r] + hb) + i);
        }
      }
#pragma unroll
    for (int u = 0; u < PC; ++u) {
      const size_t i = wc_pack<B, P>(first, u0 + u);
      if (i < end) {
        auto pack = [&](int r) {
          if constexpr (RA) return realign_rt(v[u][r], vb[u][r], in.shift[r]);
          else return v[u][r];
        };
        float acc[D::V];
        D::widen(pack(0), acc);
#pragma unroll
        for (int r = 1; r < W; ++r) {
          float t[D::V];
          D::widen(pack(r), t);
#pragma unroll
          for (int k = 0; k < D::V; ++k) acc[k] = acc[k] + t[k];
        }
        st(u0 + u, i, D::narrow(acc));
      }
    }
  }
}

// Elements outside the 16-byte body: [0, head) and [head + npacks*V, n).  At most 2V-2 of them.
template <typename D, int W, bool Dev>
__device__ __forceinline__ void reduce_edges(const RankPtrs& in, char* dst, const ReduceShape& sh) {
  const size_t tail0 = sh.head + sh.npacks * D::V;
  const size_t count = sh.head + (sh.n - tail0);
  for (size_t k = threadIdx.x; k < count; k += blockDim.x)
    reduce_elem<D, W, Dev>(in, dst, k < sh.head ? k : tail0 + (k - sh.head));
}

template <typename D>
__device__ __forceinline__ void copy_edges_from_stage(const char* stage, char* dst, const ReduceShape& sh) {
  const size_t tail0 = sh.head + sh.npacks * D::V;
  const size_t count = sh.head + (sh.n - tail0);
  for (size_t k = threadIdx.x; k < count; k += blockDim.x) {
    const size_t off = (k < sh.head ? k : tail0 + (k - sh.head)) * D::kSize;
    store_bits<D::kSize, false>(dst + off, load_bits<D::kSize, true>(stage + off));
  }
}

// ---------------------------------------------------------------------------------------- one-shot

// One-shot tile shapes (lanes x packs per lane, wave-contiguous).  The wide tile is the large-message
// shape: same-GPU A/B at W=8 bf16, 16 MiB per rank: 256 lanes x 4 packs wave-contiguous 26.2 us; 512 x 1
// lane-interleaved 26.3; 512 x 2 interleaved 26.5; 1024 x 2 wave-contiguous 26.9; 512 x 2
// wave-contiguous 27.0; 1024 x 1 interleaved 27.5.  Smaller messages take the medium (256 x 1) or
// narrow (64 x 1) tile so that the grid still has enough workgroups to keep every CU's loads in flight.
#ifndef MR_OS_BLOCK
#define MR_OS_BLOCK 256
#endif
#ifndef MR_OS_U
#define MR_OS_U 4
#endif
constexpr int kOneShotBlock = MR_OS_BLOCK;
template <int W> struct OneShotU { static constexpr int value = W <= 8 ? MR_OS_U : 1; };

// XCD-aware tile order.  Workgroups are handed to the 8 XCDs round-robin, so workgroup b runs on XCD
// b % 8; xcd_tile is a bijection of [0, ntiles) that gives XCD x one contiguous run of tiles.  Whether
// it pays depends on the grid (same-GPU A/B at W=8 bf16, three interleaved repeats, tile = b against
// xcd_tile): it wins while the grid is small (256 KiB per rank, 256 tiles: 3.11 -> 2.41 us; 512 KiB:
// 3.22 -> 2.73; 3 MiB, 768 tiles: 6.45 -> 6.23) and on the 1024 wide tiles of 16 MiB (26.8 -> 26.6),
// and loses on larger grids (4 MiB as 1024 medium tiles: 8.0 -> 9.1; 32 MiB, 2048 tiles: 51.7 -> 52.8;
// 64 MiB: 102 -> 109).  The host sets `xcd` from that (oneshot_vec_launch).
__device__ __forceinline__ size_t xcd_tile(size_t b, size_t ntiles) {
  constexpr size_t kXcds = 8;
  const size_t q = ntiles / kXcds, rem = ntiles % kXcds, x = b % kXcds;
  return x * q + (x < rem ? x : rem) + b / kXcds;
}

template <typename D, int W, int B, int U, bool RA = false, bool FULL = false>
__global__ __launch_bounds__(B) void oneshot_vec(RankPtrs in, char* out, ReduceShape sh, size_t ntiles, int xcd) {
  const size_t hb = sh.head * D::kSize;
  u32x4* dst = reinterpret_cast<u32x4*>(out + hb);
  auto store = [&](int, size_t i, const u32x4& o) { __builtin_nontemporal_store(o, dst + i); };
  for (size_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
    const size_t t = xcd ? xcd_tile(b, ntiles) : b;
    reduce_tile<D, W, B, U, decltype(store), RA, FULL>(in, hb, t * (B * U), sh.npacks, store);
  }
  if (blockIdx.x == 0) reduce_edges<D, W, false>(in, out, sh);
}

// Wide tiles, pipelined (W <= 8, 16 to 64 MiB per rank buffer): a persistent grid of as many
// workgroups as are resident on the chip at once (161 VGPRs at W=8: three per CU); workgroup b walks
// tiles b, b + grid, ...  For each tile it issues every load, then stores the previous tile's results
// while those loads are in flight, then sums.  It replaced pairs of tiles per workgroup (first tile's
// results held until the second was summed; 170 VGPRs, two per CU), which had beaten one tile per
// workgroup by 2-3% from 16 to 64 MiB.  Same-GPU A/B against the pairs, alternating processes, best of
// three, two GPUs: W=8 bf16 16 MiB per rank 24.89-24.92 -> 24.55-24.67 us and 24.94-25.08 -> 24.67-24.73,
// 24 MiB 37.09-37.24 -> 36.33-36.38, 32 MiB 49.01-49.16 -> 48.04-48.28 and 48.95-49.09 -> 48.23-48.36,
// 64 MiB 99.4-100.0 -> 98.7-99.2 and 98.8-99.5 -> 99.4-99.7; fp32 16 MiB 24.75-24.81 -> 24.61-24.68;
// W=4 bf16 16 MiB 15.16-15.21 -> 15.06-15.07.  With 640 workgroups (not every slot filled) it lost 5%,
// with XCD-contiguous tiles it lost at 24 MiB and beyond, and at 256 MiB it lost to one tile per
// workgroup (411 -> 419 us).  Full tiles without bounds checks (below) then gained 0.3-1.5%: W=8 bf16
// 16 MiB 24.77-24.83 -> 24.55-24.57 us, 64 MiB 99.8-101.0 -> 98.3-99.5, W=4 bf16 16 MiB 15.09-15.14 ->
// 14.86-14.90.  XCD-contiguous tile runs on this unchecked kernel lost at 16 MiB too (24.49-24.54 ->
// 25.71-25.93 us; 32 MiB 48.05-48.16 -> 50.75-51.12 us).
template <typename D, int W, int B, int U>
__global__ __launch_bounds__(B) void oneshot_pipe(RankPtrs in, char* out, ReduceShape sh, size_t ntiles) {
  const size_t hb = sh.head * D::kSize;
  u32x4* dst = reinterpret_cast<u32x4*>(out + hb);
  const size_t nfull = sh.npacks / (B * U);  // tiles wholly inside the packs
  u32x4 res[U];
  size_t prev = ~size_t(0);  // first pack of the tile whose sums res holds
  size_t t = blockIdx.x;
  // Full tiles need no per-lane bounds checks, so the loop is straight-line code: the compiler then
  // waits for each rank's packs in turn (the sums start while later ranks' loads are in flight) and
  // never for the previous tile's stores.  With the checks it waited for everything before summing.
  for (; t < nfull; t += gridDim.x) {
    const size_t first = t * (B * U);
    u32x4 v[U][W];
#pragma unroll
    for (int r = 0; r < W; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in.p[r] + hb) + wc_pack<B, U>(first, u));
    __asm__ volatile("" ::: "memory");  // the loads are issued before the stores below (the measured order)
    if (prev != ~size_t(0)) {
#pragma unroll
      for (int u = 0; u < U; ++u) __builtin_nontemporal_store(res[u], dst + wc_pack<B, U>(prev, u));
    }
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < U; ++u) res[u] = sum_ranks<D, W>(v[u]);
    prev = first;
  }
  if (prev != ~size_t(0)) {
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(res[u], dst + wc_pack<B, U>(prev, u));
  }
  if (t < ntiles) {  // the partial last tile (t == nfull), on the checked path
    auto st = [&](int, size_t i, const u32x4& o) { __builtin_nontemporal_store(o, dst + i); };
    reduce_tile<D, W, B, U, decltype(st)>(in, hb, t * (B * U), sh.npacks, st);
  }
  if (blockIdx.x == 0) reduce_edges<D, W, false>(in, out, sh);
}

template <typename D, int W, bool BYTES>
__global__ __launch_bounds__(kBlock) void oneshot_elem(RankPtrs in, char* out, size_t n) {
  for (size_t e = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * kBlock)
    reduce_elem<D, W, false, BYTES>(in, out, e);
}

// ---------------------------------------------------------------------------------------- two-shot
//
// Phase 1 (reduce-scatter): chunk c = 0..W-1 of the message (a 1/W share, whole 16-byte packs) is
// reduced into the stage buffer in tiles.  Phase 2 (gather-copy): the stage is copied into out in
// tiles of `ratio` phase-1 tiles, so a phase-2 workgroup copies bytes that other workgroups reduced.
//
// Start order.  A workgroup's role comes from a ticket taken when it starts, not from its index: with
// the tile and chunk barriers, workgroup b belongs to chunk c = b % W and takes the next ticket of
// that chunk's counter (tickets < t1 reduce phase-1 tile `ticket`, the rest copy phase-2 tiles); with
// the grid barrier one counter orders every workgroup.  A phase-2 tile only waits for phase-1 tiles
// whose tickets were handed out before its own, so their workgroups are already running and never
// wait themselves: the wait ends whether or not the grid fits the GPU at once, and two such kernels
// may share the GPU.  Each wait is still bounded (spin_limit polls), after which it sets an error bit.
//
// Release and acquire.  Phase-1 stage stores write through the XCD's L2 (device-scope coherence,
// sc1); every lane waits for its stores to be acknowledged (vmcnt 0) before the workgroup barrier, and
// only then does one lane publish the tile with a relaxed agent-scope atomic (performed at the device
// coherence point).  Phase-2 lanes read the stage with device-scope loads (sc1), which do not return
// a line another XCD may have changed.  That is release/acquire for exactly the stage bytes; the
// compiler's agent-scope release would instead write back every dirty line of the whole L2 once per
// workgroup, which costs several times the reduce itself.
//
// Barrier granularity (sync):
//   tile  -- phase-2 tile q of chunk c waits for the flags of phase-1 tiles [q*ratio, (q+1)*ratio) of
//            chunk c and clears them; the claim counter is cleared by the holder of the last ticket.
//   chunk -- waits until done1[c] counts all t1 phase-1 tiles of chunk c.
//   grid  -- waits until done1[x] counts all t1 phase-1 tiles of every chunk x (lanes 0..W-1 of the
//            first wave wait for one chunk each).  Work comes from per-chunk pools (claim[c]: phase-1
//            tiles, done2[c]: phase-2 groups): a workgroup tries its own chunk's pool first and the
//            others after it, and takes phase-2 work only once it found every phase-1 pool empty, so
//            every phase-1 tile has started before anyone waits.  The pools overshoot, so the last
//            workgroup to finish (gdone counts all of them) clears every word.
//   last  -- no phase-2 workgroups and no waiting: flags[c*t2 + q] counts the releases of group q of
//            chunk c, and the workgroup whose release completes the group re-arms it and copies it.
// In every mode the words return to zero by the end of the launch, so back-to-back launches on one
// stream need no host reset.

constexpr uint32_t kNoWork = 0xffffffffu;  // ticket of a workgroup that found no work (cannot happen:
                                           // the grid holds exactly one workgroup per work item)

__device__ __forceinline__ void take_ticket(Ctrl* ctrl, const TwoShotPlan& pl, uint32_t& c, uint32_t& k) {
  __shared__ uint32_t s_c, s_k;
  if (threadIdx.x == 0) {
    const uint32_t per = pl.t1 + pl.t2;
    if (pl.sync == kSyncGrid) {
      // one fetch-and-add per pool tried; a pool is empty once its counter reached its size, and
      // stays so (the counters only grow during a launch)
      const uint32_t c0 = blockIdx.x % pl.chunks;
      s_c = 0;
      s_k = kNoWork;
      bool got = false;
      for (uint32_t i = 0; i < pl.chunks && !got; ++i) {
        const uint32_t cc = c0 + i < pl.chunks ? c0 + i : c0 + i - pl.chunks;
        const uint32_t t = __hip_atomic_fetch_add(&ctrl->claim[cc][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t < pl.t1) {
          s_c = cc;
          s_k = t;
          got = true;
        }
      }
      for (uint32_t i = 0; i < pl.chunks && !got; ++i) {
        const uint32_t cc = c0 + i < pl.chunks ? c0 + i : c0 + i - pl.chunks;
        const uint32_t t = __hip_atomic_fetch_add(&ctrl->done2[cc][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t < pl.t2) {
          s_c = cc;
          s_k = pl.t1 + t;
          got = true;
        }
      }
    } else {
      const uint32_t cc = blockIdx.x % pl.chunks;
      const uint32_t t = __hip_atomic_fetch_add(&ctrl->claim[cc][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == per - 1) __hip_atomic_store(&ctrl->claim[cc][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_c = cc;
      s_k = t;
    }
  }
  __syncthreads();
  c = s_c;
  k = s_k;
}

__device__ __forceinline__ void publish_phase1(Ctrl* ctrl, uint32_t* flags, const TwoShotPlan& pl, uint32_t c, uint32_t k) {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this lane's write-through stage stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0 && pl.sync != kSyncLast) {
    if (pl.sync == kSyncTile)
      __hip_atomic_fetch_add(&flags[static_cast<size_t>(c) * pl.t1 + k], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else  // chunk and grid barriers count per chunk (W words instead of one contended word)
      __hip_atomic_fetch_add(&ctrl->done1[c][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Thread 0 polls `word` until it reaches `target` (compared as signed: a word a consumer has already
// given back reads negative until its late producer arrives); false if it gave up.
__device__ __forceinline__ bool wait_at_least(uint32_t* word, uint32_t target, uint32_t spin_limit) {
  uint32_t spins = 0;
  while (static_cast<int32_t>(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
         static_cast<int32_t>(target)) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > spin_limit) return false;
  }
  return true;
}

__device__ __forceinline__ void wait_phase1(Ctrl* ctrl, uint32_t* flags, const TwoShotPlan& pl, uint32_t c, uint32_t q) {
  if (pl.sync == kSyncTile) {
    // lanes 0..ratio-1 of the first wave each wait for one producer flag, so the waits overlap
    const uint32_t j = q * pl.ratio + threadIdx.x;
    if (threadIdx.x < pl.ratio && j < pl.t1) {
      uint32_t* f = &flags[static_cast<size_t>(c) * pl.t1 + j];
      if (!wait_at_least(f, 1u, pl.spin_limit))
        __hip_atomic_fetch_or(&ctrl->err[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // consumed: give the release back.  After a timeout this leaves -1, and the late producer's +1
      // (still inside this launch) brings the flag back to zero, so it cannot satisfy a later launch.
      __hip_atomic_fetch_sub(f, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (pl.sync == kSyncChunk) {
    if (threadIdx.x == 0 && !wait_at_least(&ctrl->done1[c][0], pl.t1, pl.spin_limit))
      __hip_atomic_fetch_or(&ctrl->err[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x < pl.chunks) {
    // grid barrier: lane x of the first wave waits for chunk x, so the W waits overlap
    if (!wait_at_least(&ctrl->done1[threadIdx.x][0], pl.t1, pl.spin_limit))
      __hip_atomic_fetch_or(&ctrl->err[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// End of a workgroup's two-shot work (k = its ticket).  Chunk barrier: the last phase-2 tile of chunk c
// re-arms that chunk's words.  Grid barrier: every workgroup counts itself out, and the last one re-arms
// the pools and counters of every chunk (no workgroup can still be claiming work then).  The words that
// only count with returning atomics (pools, done2, gdone) have seen every increment of the launch and
// are stored to zero; the release counts done1 get non-returning increments, which may still be in
// flight (or, after a timeout, still to come), so t1 is subtracted instead: the count reaches zero once
// every phase-1 tile of the launch has released, in whatever order the atomics land.
__device__ __forceinline__ void finish_twoshot(Ctrl* ctrl, const TwoShotPlan& pl, uint32_t c, uint32_t k) {
  if (threadIdx.x != 0) return;
  if (pl.sync == kSyncChunk && k >= pl.t1) {
    const uint32_t d = __hip_atomic_fetch_add(&ctrl->done2[c][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == pl.t2 - 1) {
      __hip_atomic_fetch_sub(&ctrl->done1[c][0], pl.t1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->done2[c][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (pl.sync == kSyncGrid) {
    const uint32_t d = __hip_atomic_fetch_add(&ctrl->gdone[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == pl.chunks * (pl.t1 + pl.t2) - 1) {
      for (uint32_t x = 0; x < pl.chunks; ++x) {
        __hip_atomic_store(&ctrl->claim[x][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_sub(&ctrl->done1[x][0], pl.t1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctrl->done2[x][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(&ctrl->gdone[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

constexpr uint32_t kRatio = MR_TS_RATIO;  // phase-1 tiles per phase-2 tile
static_assert(kRatio >= 1 && kRatio <= 64, "one lane of the first wave waits for each producer flag");
// Phase-1 tile = TB lanes x 1 pack; phase-2 tile = TB lanes x ratio packs.  Large messages use TB=1024
// (same-GPU A/B at W=8 bf16, 16 MiB per rank, per-tile flags: 1024 lanes x 1 pack 35.4 us, 512 x 2
// 39.2 us, 256 x 4 39.8 us; each publish waits for its stores); smaller ones TB=256 or 64, so that
// each chunk still splits into enough tiles to fill the CUs.
constexpr int kTBlock = static_cast<int>(kTwoShotWideTile);  // the planner sizes wide tiles by it too
constexpr int kP2 = kRatio;  // packs per lane, phase 2
// Element-wise path (pointers in different 16-byte phases): elements per lane per phase-1 tile.  Same-GPU
// A/B, W=8 bf16, 16 MiB per rank, inputs at alternating 2-byte phases: one element per lane with the
// loads issued one element at a time 92 us; with a lane's loads all in flight first, 1 / 2 / 4 / 8
// elements per lane 88.5 / 94.7 / 86.5 / 137 us (eight ranks of eight elements outrun the 63
// outstanding loads a wave can count).  The 16-byte path takes 35.6 us.
constexpr int kElemPer = 4;

// Phase 2 of one group: copy the TB*P2 packs from `first` (clipped to cend) from the stage to out with
// device-scope stage loads, P2 packs per lane, wave-contiguous.
template <typename D, int TB, int P2, int LAUX = kStageLoadAux>
__device__ __forceinline__ void copy_group(char* out, char* stage, const ReduceShape& sh, size_t first, size_t cend,
                                           bool with_edges) {
  const size_t hb = sh.head * D::kSize;
  const i32x4 rs = make_rsrc(stage + hb + first * 16, TB * P2 * 16);
  u32x4 v[P2];
#pragma unroll
  for (int u = 0; u < P2; ++u) {
    const size_t i = wc_pack<TB, P2>(first, u);
    if (i < cend) v[u] = __builtin_bit_cast(u32x4, raw_buffer_load_v4(rs, static_cast<int>((i - first) * 16), 0, LAUX));
  }
#pragma unroll
  for (int u = 0; u < P2; ++u) {
    const size_t i = wc_pack<TB, P2>(first, u);
    if (i < cend) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(out + hb) + i);
  }
  if (with_edges) copy_edges_from_stage<D>(stage, out, sh);
}

// Last-arriver hand-off: after publishing its tile, the workgroup bumps the arrival count of its group
// of `ratio` tiles; the one that completes the group (it has seen every other member's release in the
// atomic's order) re-arms the count and copies the group.  Nobody waits.
__device__ __forceinline__ bool arrive_last(uint32_t* counts, const TwoShotPlan& pl, uint32_t c, uint32_t k) {
  __shared__ uint32_t s_last;
  if (threadIdx.x == 0) {
    const uint32_t q = k / pl.ratio;
    const uint32_t members = (q + 1) * pl.ratio <= pl.t1 ? pl.ratio : pl.t1 - q * pl.ratio;
    uint32_t* cnt = &counts[static_cast<size_t>(c) * pl.t2 + q];
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == members - 1;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// Built once per hand-off (SYNC): with the mode a compile-time constant the other modes' code drops
// out.  Same-GPU A/B against one build for all modes, W=8 bf16: 4 MiB per rank tile 16.0 -> 15.65 us,
// chunk 16.3 -> 15.85, last arriver 11.8 -> 11.55, grid 17.2 -> 17.6; 16 MiB last 38.1 -> 37.7, grid
// 38.2 -> 37.7.
template <typename D, int W, int TB, int SYNC, bool RA = false>
__global__ __launch_bounds__(TB) void twoshot_vec(RankPtrs in, char* out, char* stage, Ctrl* ctrl, uint32_t* flags,
                                                  ReduceShape sh, TwoShotPlan pl_arg) {
  TwoShotPlan pl = pl_arg;
  pl.sync = SYNC;
  uint32_t c, k;
  if (pl.sync == kSyncLast) {  // phase-1 workgroups only; consecutive workgroups take one chunk's tiles
    c = blockIdx.x / pl.t1;
    k = blockIdx.x % pl.t1;
  } else {
    take_ticket(ctrl, pl, c, k);
  }
  const size_t hb = sh.head * D::kSize;
  const size_t c0 = static_cast<size_t>(c) * pl.chunk_units;
  const size_t cend = c0 + pl.chunk_units < sh.npacks ? c0 + pl.chunk_units : sh.npacks;
  if (k < pl.t1) {
    const size_t first = c0 + static_cast<size_t>(k) * TB;
    const i32x4 rs = make_rsrc(stage + hb + first * 16, TB * 16);
    auto store = [&](int, size_t i, const u32x4& o) {
      raw_buffer_store_v4(__builtin_bit_cast(i32x4, o), rs, static_cast<int>((i - first) * 16), 0, kStageStoreAux);
    };
    reduce_tile<D, W, TB, 1, decltype(store), RA>(in, hb, first, cend, store);
    if (c == 0 && k == 0) reduce_edges<D, W, true>(in, stage, sh);
    publish_phase1(ctrl, flags, pl, c, k);
    if (pl.sync == kSyncLast && arrive_last(flags, pl, c, k)) {
      const uint32_t q = k / pl.ratio;
      copy_group<D, TB, kP2>(out, stage, sh, c0 + static_cast<size_t>(q) * (TB * kRatio), cend, c == 0 && q == 0);
    }
  } else if (k < pl.t1 + pl.t2) {
    const uint32_t q = k - pl.t1;
    wait_phase1(ctrl, flags, pl, c, q);
    copy_group<D, TB, kP2>(out, stage, sh, c0 + static_cast<size_t>(q) * (TB * kRatio), cend, c == 0 && q == 0);
  }
  finish_twoshot(ctrl, pl, c, k);
}

// XCD-local two-shot with per-unit producer flags (16-byte path, W <= 8; the per-tile hand-off from
// 16 MiB per rank buffer).
//
// Units.  The message is cut into units of one wide tile (256 lanes x 4 packs, 16 KiB of output; the
// last-arriver form takes 4 KiB or 1 KiB units below 8 MiB per rank buffer) and the units into kXcds
// runs of `run` consecutive units, one run per XCD.  Workgroup b belongs to run
// x = b % kXcds, because workgroups are dealt to the XCDs in turn; its index s = b / kXcds inside the
// run gives its role: s < run_padded reduces unit s of the run into the stage (phase 1), larger s copy
// a group of kXcdGroup consecutive units of the run from the stage to out (phase 2, always units that
// other workgroups reduced).  Roles come from the index, so no ticket atomic delays a workgroup's loads.
//
// Hand-off inside one XCD.  A producer writes its unit to the stage with ordinary write-back stores,
// waits until the XCD's L2 has acknowledged every one of them (vmcnt 0) and then publishes the unit by
// exchanging its flag word for 1 + the XCC id it runs on (a relaxed agent-scope atomic).  A copier
// polls the flags of its group; a flag holding 1 + its own XCC id means the unit sits in the L2 it
// reads through.  One L2 serves every CU of an XCD, so the stores need no write-back past it and no
// write-through.  The copier's loads (sc0, workgroup-scope coherence) may be served by its CU's L1, but
// no L1 can hold an old copy of the unit: stream order already makes a launch see every earlier write,
// so an L1 could only return a stage line that the same CU loaded earlier in this launch, and every
// stage line is loaded once per launch, by the copier of its unit, after the flag (units start on
// 256-byte boundaries of the stage, so no cache line holds bytes of two units).
//
// Nothing rests on where the dispatcher places workgroups or in which order it starts them.  A unit
// whose flag names another XCD, or whose producer has not published within the spin limit, is
// recomputed by the copier from the rank buffers straight into out (same arithmetic, same bits).  On a
// timeout the copier first claims the flag (compare-and-swap 0 -> kTaken); a producer that publishes
// later finds kTaken and clears it, and a copier that finds a published value clears it, so every flag
// is zero again when the launch ends and a late release can never satisfy a later launch.  The error
// word records these rare paths (bit 1: recomputed after a timeout, bit 2: producer on another XCD);
// the output stays valid in both.
//
// Same-GPU A/B against the ticketed 1024-lane tile kernel (W=8, rotating buffer sets, three repeats):
// bf16 16 MiB per rank 35.1 -> 34.1-34.3 us and 35.4 -> 33.0 us on two GPUs, 32 MiB 66.3 -> 63.5-64.4,
// 64 MiB 119-129 -> 118-119; fp32 16 MiB 35.1 -> 34.1-34.3, 64 MiB 124.6 -> 119.3.  Units of two wide
// tiles (one round of 512 workgroups at 16 MiB), a copy group of 1 or 3 units, a non-temporal stage
// load, and copies interleaved into the dispatch order after a lag of 24-192 units per run all
// measured the same or slower; the interleaved copies wait and hold slots.
constexpr uint32_t kTaken = 0xffffffffu;  // flag claimed by a copier that stopped waiting
constexpr int kXcdStageLoadAux = 1;       // sc0: workgroup-scope coherent stage loads (see above)

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 0xfu;
}

// Lanes 0..kXcdGroup-1 of the first wave settle one unit each: 0 nothing (past the end), 1 copy it from
// the stage, 2 recompute it.
__device__ __forceinline__ uint32_t settle_unit(Ctrl* ctrl, uint32_t* flags, size_t u, uint32_t spin_limit) {
  uint32_t* f = &flags[u];
  uint32_t v, spins = 0;
  while ((v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > spin_limit) {
      uint32_t expect = 0u;
      v = __hip_atomic_compare_exchange_strong(f, &expect, kTaken, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
              ? kTaken
              : expect;  // published meanwhile
      break;
    }
  }
  if (v == kTaken) {  // our claim: the producer clears it when it publishes
    __hip_atomic_fetch_or(&ctrl->err[0], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 2u;
  }
  __hip_atomic_store(f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // consumed: re-arm
  if (v == 1u + xcc_id()) return 1u;
  __hip_atomic_fetch_or(&ctrl->err[0], 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 2u;
}

// Last-arriver form (LAST; no copier workgroups and no waiting): the 64-bit word g of run x in the flag
// area is the arrival word of copy group g (kXcdLastGroup units) of that run.  Its low 8 bits count
// the members that have published, and a 4-bit field per XCC (from bit 8) counts those that ran there.
// The producer whose arrival completes the group re-arms the word and copies the group from the stage
// at once; if some member ran on another XCC it recomputes the group from the rank buffers instead
// (error word bit 2, output valid).
__device__ __forceinline__ uint64_t xcd_arrival(uint32_t xcc) {
  return 1u + (xcc < kXcds ? uint64_t{1} << (8 + 4 * xcc) : 0u);
}
static_assert(8 + 4 * kXcds <= 64 && kXcdLastGroup >= 1 && kXcdLastGroup <= 15, "arrival word fields");

// B lanes x U packs per unit: the wide tile (256 x 4, 16 KiB of output) from 8 MiB per rank buffer,
// and for the last arriver on smaller messages the medium (256 x 1) or narrow (64 x 1) tile, so that a
// small message still spreads over every CU (twoshot_xcd_unit_packs picks it).
template <typename D, int W, bool LAST, bool RA = false, int B = kOneShotBlock, int U = 4>
__global__ __launch_bounds__(B) void twoshot_xcd(RankPtrs in, char* out, char* stage, Ctrl* ctrl,
                                                 uint32_t* flags, ReduceShape sh, TwoShotPlan pl) {
  static_assert(LAST || !RA, "realigned inputs take the last-arriver hand-off only");
  static_assert(LAST || (B == kOneShotBlock && U == 4), "copier workgroups run on wide units");
  constexpr int R = static_cast<int>(LAST ? kXcdLastGroup : kXcdGroup);  // units per copy
  constexpr size_t UP = static_cast<size_t>(B) * U;  // packs per unit
  static_assert(UP * 16 % 256 == 0, "units start on 256-byte boundaries of the stage body");
  const size_t hb = sh.head * D::kSize;
  const uint32_t x = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
  const size_t run0 = static_cast<size_t>(x) * pl.run;  // first unit of this run
  const size_t in_run = run0 < pl.units ? (pl.units - run0 < pl.run ? pl.units - run0 : pl.run) : 0;
  u32x4* dst = reinterpret_cast<u32x4*>(out + hb);
  __shared__ uint32_t s_mode[R];
  uint32_t g;  // copy group of this run
  if (s < pl.run_padded) {
    const size_t u = run0 + s;
    if (s >= in_run) return;  // padding
    const size_t first = u * UP;
    const i32x4 rs = make_rsrc(stage + hb + first * 16, static_cast<uint32_t>(UP * 16));
    auto store = [&](int, size_t i, const u32x4& o) {
      raw_buffer_store_v4(__builtin_bit_cast(i32x4, o), rs, static_cast<int>((i - first) * 16), 0, 0);
    };
    reduce_tile<D, W, B, U, decltype(store), RA>(in, hb, first, sh.npacks, store);
    if (u == 0) reduce_edges<D, W, false>(in, out, sh);  // the few elements outside the packs: straight to out
    __builtin_amdgcn_s_waitcnt(0x0f70);                 // vmcnt(0): the L2 holds this lane's stage stores
    __syncthreads();
    if constexpr (!LAST) {
      if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_exchange(&flags[u], 1u + xcc_id(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == kTaken) __hip_atomic_store(&flags[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    } else {
      g = s / R;
      if (threadIdx.x == 0) {
        const uint32_t members = in_run - static_cast<size_t>(g) * R < R ? static_cast<uint32_t>(in_run - static_cast<size_t>(g) * R) : R;
        uint64_t* word = reinterpret_cast<uint64_t*>(flags) + static_cast<size_t>(x) * ((pl.run + R - 1) / R) + g;
        const uint32_t me = xcc_id();
        const uint64_t add = xcd_arrival(me);
        const uint64_t old = __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t go = 0u;
        if ((old & 0xffu) == members - 1) {  // every member has published: re-arm, then copy the group
          __hip_atomic_store(word, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          go = me < kXcds && (((old + add) >> (8 + 4 * me)) & 15u) == members ? 1u : 2u;
          if (go == 2u) __hip_atomic_fetch_or(&ctrl->err[0], 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) s_mode[r] = static_cast<uint32_t>(r) < members ? go : 0u;
      }
      __syncthreads();
      if (s_mode[0] == 0u) return;
    }
  } else {
    if constexpr (LAST) return;  // not launched: the last-arriver grid holds producers only
    g = s - pl.run_padded;
    if (threadIdx.x < R) {
      const size_t i = static_cast<size_t>(g) * R + threadIdx.x;
      s_mode[threadIdx.x] = i < in_run ? settle_unit(ctrl, flags, run0 + i, pl.spin_limit) : 0u;
    }
    __syncthreads();
  }
  const size_t first = (run0 + static_cast<size_t>(g) * R) * UP;
  bool from_stage = true;
#pragma unroll
  for (int r = 0; r < R; ++r) from_stage = from_stage && s_mode[r] != 2u;
  if (from_stage) {  // the common case: every unit from the stage, all loads in flight before the stores
    const i32x4 rs = make_rsrc(stage + hb + first * 16, static_cast<uint32_t>(UP * R * 16));
    u32x4 v[R * U];
    if (s_mode[R - 1] == 1u && first + R * UP <= sh.npacks) {
      // A whole group (every member present, inside the packs) without per-lane checks: straight-line
      // code, so each store waits only for its own load.  Same-GPU A/B, W=8 bf16, last arriver: 1 MiB
      // per rank 5.81 -> 5.19 us, 4 MiB 10.86 -> 9.87, 16 MiB 31.9 -> 31.3, 32 MiB 63.1 -> 62.0; fp32
      // 16 MiB 31.6 -> 30.8.
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int uu = 0; uu < U; ++uu)
          v[r * U + uu] = __builtin_bit_cast(
              u32x4, raw_buffer_load_v4(rs, static_cast<int>((wc_pack<B, U>(first + r * UP, uu) - first) * 16), 0,
                                        kXcdStageLoadAux));
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int uu = 0; uu < U; ++uu) __builtin_nontemporal_store(v[r * U + uu], dst + wc_pack<B, U>(first + r * UP, uu));
      return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const size_t i = wc_pack<B, U>(first + r * UP, uu);
        if (s_mode[r] == 1u && i < sh.npacks)
          v[r * U + uu] = __builtin_bit_cast(u32x4, raw_buffer_load_v4(rs, static_cast<int>((i - first) * 16), 0, kXcdStageLoadAux));
      }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const size_t i = wc_pack<B, U>(first + r * UP, uu);
        if (s_mode[r] == 1u && i < sh.npacks) __builtin_nontemporal_store(v[r * U + uu], dst + i);
      }
    return;
  }
#pragma unroll 1
  for (int r = 0; r < R; ++r) {  // some unit recomputed: one unit at a time
    const size_t f = first + r * UP;
    if (s_mode[r] == 1u)
      copy_group<D, B, U, kXcdStageLoadAux>(out, stage, sh, f, sh.npacks, false);
    else if (s_mode[r] == 2u) {
      auto st = [&](int, size_t i, const u32x4& o) { __builtin_nontemporal_store(o, dst + i); };
      reduce_tile<D, W, B, U, decltype(st), RA>(in, hb, f, sh.npacks, st);
    }
  }
}

// Element-wise two-shot for pointers that do not share one 16-byte alignment (units are elements;
// a phase-2 group copies ratio phase-1 tiles, kElemPer elements per lane each).
template <typename D, bool BYTES>
__device__ __forceinline__ void copy_group_elem(char* out, const char* stage, size_t first, size_t cend) {
  constexpr int N = kRatio * kElemPer;  // elements per lane
  uint32_t v[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const size_t e = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (e < cend) v[u] = load_bits<D::kSize, true>(stage + e * D::kSize);
  }
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const size_t e = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (e < cend) {
      if (BYTES) store_bytes<D::kSize>(out + e * D::kSize, v[u]);
      else store_bits<D::kSize, false>(out + e * D::kSize, v[u]);
    }
  }
}

// Phase-1 tile of the element-wise path: kElemPer elements per lane at stride kBlock (each step
// coalesced), every rank's loads in flight before the adds.
template <typename D, int W, bool BYTES>
__device__ __forceinline__ void reduce_tile_elem(const RankPtrs& in, char* stage, size_t first, size_t cend) {
  uint32_t v[kElemPer][W];
#pragma unroll
  for (int r = 0; r < W; ++r)
#pragma unroll
    for (int u = 0; u < kElemPer; ++u) {
      const size_t e = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
      if (e < cend) v[u][r] = BYTES ? load_bytes<D::kSize>(in.p[r] + e * D::kSize) : load_bits<D::kSize, false>(in.p[r] + e * D::kSize);
    }
#pragma unroll
  for (int u = 0; u < kElemPer; ++u) {
    const size_t e = first + static_cast<size_t>(u) * kBlock + threadIdx.x;
    if (e < cend) {
      float acc = D::widen1(v[u][0]);
#pragma unroll
      for (int r = 1; r < W; ++r) acc = acc + D::widen1(v[u][r]);
      store_bits<D::kSize, true>(stage + e * D::kSize, D::narrow1(acc));
    }
  }
}

template <typename D, int W, bool BYTES>
__global__ __launch_bounds__(kBlock) void twoshot_elem(RankPtrs in, char* out, char* stage, Ctrl* ctrl,
                                                       uint32_t* flags, ReduceShape sh, TwoShotPlan pl) {
  uint32_t c, k;
  if (pl.sync == kSyncLast) {
    c = blockIdx.x / pl.t1;
    k = blockIdx.x % pl.t1;
  } else {
    take_ticket(ctrl, pl, c, k);
  }
  constexpr size_t kTileE = static_cast<size_t>(kBlock) * kElemPer;  // elements per phase-1 tile
  const size_t c0 = static_cast<size_t>(c) * pl.chunk_units;
  const size_t cend = c0 + pl.chunk_units < sh.n ? c0 + pl.chunk_units : sh.n;
  if (k < pl.t1) {
    reduce_tile_elem<D, W, BYTES>(in, stage, c0 + static_cast<size_t>(k) * kTileE, cend);
    publish_phase1(ctrl, flags, pl, c, k);
    if (pl.sync == kSyncLast && arrive_last(flags, pl, c, k))
      copy_group_elem<D, BYTES>(out, stage, c0 + static_cast<size_t>(k / pl.ratio) * (kTileE * kRatio), cend);
  } else if (k < pl.t1 + pl.t2) {
    const uint32_t q = k - pl.t1;
    wait_phase1(ctrl, flags, pl, c, q);
    copy_group_elem<D, BYTES>(out, stage, c0 + static_cast<size_t>(q) * (kTileE * kRatio), cend);
  }
  finish_twoshot(ctrl, pl, c, k);
}

__global__ void zero_words(uint32_t* p, size_t words) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------------------------------- dispatch

constexpr size_t kMaxGrid = size_t(1) << 20;  // workgroups; beyond this the one-shot kernels grid-stride

template <typename D, int W, int B, int U, bool RA = false, bool FULL = false>
hipError_t oneshot_vec_launch(const RankPtrs& in, char* out, const ReduceShape& sh, hipStream_t st) {
  constexpr size_t tile = static_cast<size_t>(B) * U;
  const size_t ntiles = (sh.npacks + tile - 1) / tile;
  size_t grid = ntiles < kMaxGrid ? ntiles : kMaxGrid;
  if (grid == 0) grid = 1;  // edges only
  // XCD-contiguous tile order on small grids and on the wide tiles up to 1024 of them (see xcd_tile)
  const int xcd = grid == ntiles && (ntiles <= 512 || (tile == 1024 && ntiles <= 1024)) ? 1 : 0;
  hipLaunchKernelGGL((oneshot_vec<D, W, B, U, RA, FULL>), dim3(static_cast<unsigned>(grid)), dim3(B), 0, st, in, out,
                     sh, ntiles, xcd);
  return hipGetLastError();
}

template <typename D, int W>
hipError_t oneshot_pipe_launch(const RankPtrs& in, char* out, const ReduceShape& sh, hipStream_t st) {
  constexpr int B = kOneShotBlock, U = OneShotU<W>::value;
  const size_t ntiles = (sh.npacks + B * U - 1) / (B * U);
  const size_t resident = resident_workgroups(oneshot_pipe<D, W, B, U>, B);
  size_t grid = resident && resident < ntiles ? resident : ntiles;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid == 0) grid = 1;  // edges only
  hipLaunchKernelGGL((oneshot_pipe<D, W, B, U>), dim3(static_cast<unsigned>(grid)), dim3(B), 0, st, in, out, sh, ntiles);
  return hipGetLastError();
}

// Realigned 16-byte path (inputs in other 16-byte phases than out): the wide tile's four packs per lane
// for W <= 8, the second aligned pack of each moved over from the neighbouring lane (reduce_tile_realigned;
// 234 VGPRs, two waves per SIMD).  Same-GPU A/B, W=8, 16 MiB per rank, inputs at alternating phases:
// two packs per lane with both aligned packs loaded 30.3 us (bf16); two packs per lane, neighbour moves
// 27.4; four packs per lane, neighbour moves 26.2 (the aligned wide one-shot: 25.6).  One pack for W > 8.
// The aligned one-shot's pipelined persistent schedule does not carry over: a resident grid storing one
// realigned tile's sums while the next tile loads ran slower at both widths (same GPU, three interleaved
// repeats, W=8, odd ranks one element off: bf16 16 MiB 26.9-27.3 -> 28.5-28.6 us with four packs per
// lane, 224 VGPRs, and 28.6-29.0 us with two, 160 VGPRs; bf16 63 MiB 96.6-97.0 -> 100.5-100.9 us).
#ifndef MR_RA_U
#define MR_RA_U 4
#endif
template <int W> struct RealignU { static constexpr int value = W <= 8 ? MR_RA_U : 1; };

template <typename D, int W>
hipError_t oneshot_w(const RankPtrs& in, char* out, const ReduceShape& sh, uint32_t shape, hipStream_t st) {
  if (sh.vec && sh.realign) return oneshot_vec_launch<D, W, kOneShotBlock, RealignU<W>::value, true>(in, out, sh, st);
  if (sh.vec) {
    if constexpr (W <= 8) {
      if (shape == kShapeWidePair) return oneshot_pipe_launch<D, W>(in, out, sh, st);
    }
    switch (shape) {
      case kShapeNarrow: return oneshot_vec_launch<D, W, 64, 1>(in, out, sh, st);
      case kShapeMedium: return oneshot_vec_launch<D, W, 256, 1>(in, out, sh, st);
      default:
        // beyond the pipelined kernel's range, full wide tiles on the unchecked path: same-GPU A/B, W=8
        // bf16, 128 MiB per rank 202.3-202.6 -> 199.2-200.9 us, 256 MiB 413.0-413.8 -> 404.4-406.2 us;
        // at 8 MiB it lost (13.7 -> 15.4 us), so smaller messages keep the checked path
        if (sh.npacks > kPipeMaxPacks)
          return oneshot_vec_launch<D, W, kOneShotBlock, OneShotU<W>::value, false, true>(in, out, sh, st);
        return oneshot_vec_launch<D, W, kOneShotBlock, OneShotU<W>::value>(in, out, sh, st);
    }
  }
  const size_t need = (sh.n + kBlock - 1) / kBlock;
  const size_t grid = need < kMaxGrid ? need : kMaxGrid;
  if (sh.bytes)
    hipLaunchKernelGGL((oneshot_elem<D, W, true>), dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, st, in, out, sh.n);
  else
    hipLaunchKernelGGL((oneshot_elem<D, W, false>), dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, st, in, out, sh.n);
  return hipGetLastError();
}

template <typename D, int W, int TB>
hipError_t twoshot_vec_launch(const RankPtrs& in, char* out, char* stage, Ctrl* ctrl, uint32_t* flags,
                              const ReduceShape& sh, const TwoShotPlan& pl, unsigned grid, hipStream_t st) {
  switch (pl.sync) {
    case kSyncTile:
      hipLaunchKernelGGL((twoshot_vec<D, W, TB, kSyncTile>), dim3(grid), dim3(TB), 0, st, in, out, stage, ctrl, flags, sh, pl);
      break;
    case kSyncChunk:
      hipLaunchKernelGGL((twoshot_vec<D, W, TB, kSyncChunk>), dim3(grid), dim3(TB), 0, st, in, out, stage, ctrl, flags, sh, pl);
      break;
    case kSyncGrid:
      hipLaunchKernelGGL((twoshot_vec<D, W, TB, kSyncGrid>), dim3(grid), dim3(TB), 0, st, in, out, stage, ctrl, flags, sh, pl);
      break;
    default:
      hipLaunchKernelGGL((twoshot_vec<D, W, TB, kSyncLast>), dim3(grid), dim3(TB), 0, st, in, out, stage, ctrl, flags, sh, pl);
      break;
  }
  return hipGetLastError();
}

template <typename D, int W>
hipError_t twoshot_w(const RankPtrs& in, char* out, char* stage, Ctrl* ctrl, uint32_t* flags, const ReduceShape& sh,
                     const TwoShotPlan& pl, hipStream_t st) {
  if constexpr (W <= 8) {
    if (sh.vec && pl.xcd && pl.sync == kSyncLast) {
      const dim3 g(static_cast<unsigned>(twoshot_grid(pl)));
      if (sh.realign) {
        if (pl.unit1 == 64)
          hipLaunchKernelGGL((twoshot_xcd<D, W, true, true, 64, 1>), g, dim3(64), 0, st, in, out, stage, ctrl, flags,
                             sh, pl);
        else if (pl.unit1 == 256)
          hipLaunchKernelGGL((twoshot_xcd<D, W, true, true, 256, 1>), g, dim3(256), 0, st, in, out, stage, ctrl, flags,
                             sh, pl);
        else
          hipLaunchKernelGGL((twoshot_xcd<D, W, true, true>), g, dim3(kOneShotBlock), 0, st, in, out, stage, ctrl,
                             flags, sh, pl);
      } else {
        if (pl.unit1 == 64)
          hipLaunchKernelGGL((twoshot_xcd<D, W, true, false, 64, 1>), g, dim3(64), 0, st, in, out, stage, ctrl, flags,
                             sh, pl);
        else if (pl.unit1 == 256)
          hipLaunchKernelGGL((twoshot_xcd<D, W, true, false, 256, 1>), g, dim3(256), 0, st, in, out, stage, ctrl,
                             flags, sh, pl);
        else
          hipLaunchKernelGGL((twoshot_xcd<D, W, true>), g, dim3(kOneShotBlock), 0, st, in, out, stage, ctrl, flags, sh,
                             pl);
      }
      return hipGetLastError();
    }
    if (sh.vec && pl.xcd) {
      hipLaunchKernelGGL((twoshot_xcd<D, W, false>), dim3(static_cast<unsigned>(twoshot_grid(pl))),
                         dim3(kOneShotBlock), 0, st, in, out, stage, ctrl, flags, sh, pl);
      return hipGetLastError();
    }
  }
  const unsigned grid = static_cast<unsigned>(twoshot_grid(pl));
  if (sh.vec && sh.realign) {  // the planner fixes the last-arriver hand-off and wide tiles here
    hipLaunchKernelGGL((twoshot_vec<D, W, kTBlock, kSyncLast, true>), dim3(grid), dim3(kTBlock), 0, st, in, out, stage,
                       ctrl, flags, sh, pl);
    return hipGetLastError();
  }
  if (sh.vec && pl.unit1 == 64)
    return twoshot_vec_launch<D, W, 64>(in, out, stage, ctrl, flags, sh, pl, grid, st);
  if (sh.vec && pl.unit1 == 256)
    return twoshot_vec_launch<D, W, 256>(in, out, stage, ctrl, flags, sh, pl, grid, st);
  if (sh.vec)
    return twoshot_vec_launch<D, W, kTBlock>(in, out, stage, ctrl, flags, sh, pl, grid, st);
  if (sh.bytes)
    hipLaunchKernelGGL((twoshot_elem<D, W, true>), dim3(grid), dim3(kBlock), 0, st, in, out, stage, ctrl, flags, sh, pl);
  else
    hipLaunchKernelGGL((twoshot_elem<D, W, false>), dim3(grid), dim3(kBlock), 0, st, in, out, stage, ctrl, flags, sh, pl);
  return hipGetLastError();
}

#define MR_W_CASES(F, D, ...)              \
  switch (W) {                             \
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
hipError_t oneshot_d(const RankPtrs& in, int W, char* out, const ReduceShape& sh, uint32_t shape, hipStream_t st) {
  MR_W_CASES(oneshot_w, D, in, out, sh, shape, st)
}

template <typename D>
hipError_t twoshot_d(const RankPtrs& in, int W, char* out, char* stage, Ctrl* ctrl, uint32_t* flags,
                     const ReduceShape& sh, const TwoShotPlan& pl, hipStream_t st) {
  MR_W_CASES(twoshot_w, D, in, out, stage, ctrl, flags, sh, pl, st)
}

}  // namespace

hipError_t launch_oneshot(const RankPtrs& in, int W, mr_dtype dt, char* out, const ReduceShape& sh,
                          uint32_t shape, hipStream_t st) {
  switch (dt) {
    case MR_BF16: return oneshot_d<Bf16>(in, W, out, sh, shape, st);
    case MR_FP16: return oneshot_d<Fp16>(in, W, out, sh, shape, st);
    case MR_FP32: return oneshot_d<Fp32>(in, W, out, sh, shape, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_twoshot(const RankPtrs& in, int W, mr_dtype dt, char* out, char* stage, Ctrl* ctrl,
                          uint32_t* flags, const ReduceShape& sh, const TwoShotPlan& pl, hipStream_t st) {
  switch (dt) {
    case MR_BF16: return twoshot_d<Bf16>(in, W, out, stage, ctrl, flags, sh, pl, st);
    case MR_FP16: return twoshot_d<Fp16>(in, W, out, stage, ctrl, flags, sh, pl, st);
    case MR_FP32: return twoshot_d<Fp32>(in, W, out, stage, ctrl, flags, sh, pl, st);
    default: return hipErrorInvalidValue;
  }
}

// Chunk c holds ceil(units / W) consecutive units: 16-byte packs of the body (elements on the
// element-wise path).  When n is a multiple of the pack, chunk c is exactly elements [c*C, (c+1)*C)
// with C = ceil(n/W) rounded up to a whole pack, so every chunk boundary is 16-byte aligned; the last
// chunks may be short or empty.  The few elements outside the body (an unaligned head, a tail shorter
// than a pack) ride with phase-1 tile 0 and phase-2 tile 0 of chunk 0.
TwoShotPlan plan_twoshot(int W, const ReduceShape& sh, uint32_t sync, uint32_t spin_limit, uint32_t shape) {
  TwoShotPlan pl{};
  if (sh.vec && sh.realign) {  // realigned inputs: the last-arriver hand-off, on XCD-local units or wide tiles
    sync = kSyncLast;
    if (!twoshot_xcd_units(sh.vec, W, sh.npacks, sync, shape)) shape = kShapeWide;
  }
  pl.chunks = static_cast<uint32_t>(W);
  const size_t units = sh.vec ? sh.npacks : sh.n;
  pl.chunk_units = (units + W - 1) / W;
  pl.unit1 = sh.vec ? twoshot_tile_packs(sh.npacks, sync, shape) : kBlock * kElemPer;
  pl.ratio = kRatio;
  pl.unit2 = pl.unit1 * kRatio;
  size_t t1 = (pl.chunk_units + pl.unit1 - 1) / pl.unit1;
  if (t1 == 0) t1 = 1;  // an edges-only call still has one tile of each phase
  const size_t t2 = (t1 + kRatio - 1) / kRatio;
  pl.t1 = static_cast<uint32_t>(t1);
  pl.t2 = static_cast<uint32_t>(t2);
  pl.sync = sync;
  pl.spin_limit = spin_limit;
  if (twoshot_xcd_units(sh.vec, W, sh.npacks, sync, shape)) {  // XCD-local units replace the chunk tiles
    const size_t UP = twoshot_xcd_unit_packs(sh.npacks, sync, shape);
    pl.unit1 = static_cast<uint32_t>(UP);
    pl.xcd = 1;
    pl.units = sh.npacks ? (sh.npacks + UP - 1) / UP : 1;  // an edges-only call still has one unit
    pl.run = static_cast<uint32_t>((pl.units + kXcds - 1) / kXcds);
    pl.run_padded = (pl.run + kXcdGroup - 1) / kXcdGroup * kXcdGroup;
  }
  return pl;
}

hipError_t launch_zero_words(void* p, size_t words, hipStream_t st) {
  if (words == 0) return hipSuccess;
  size_t grid = (words + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(zero_words, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace mr
