// Device code of the layout-aware FSDP2 collective local stages for MI355X
// (gfx950, CDNA4), after "The Endgame of FSDP Communication: Layout-Aware
// Collectives on Copy Engines, RDMA, and NVSwitch" (Wang et al.).
//
//   rs_local_kernel    reduce-scatter local stage (Section 4, Equation 5;
//                      Section 4.1 "Level 1: Node-Local Reduction"): W ranks'
//                      bf16 (or fp32) gradients -> W packed fp32 shards,
//                      summed in rank order in fp32 (Section 4.3), then
//                      Equation 5's alpha and accumulate; padding rows are
//                      rows of zeros.
//   ag_copyout_kernel  all-gather copy-out (Section 2.1): rank-major bf16
//                      buffer -> per-parameter tensors.
//   ag_copyin_kernel   all-gather copy-in (Sections 2.1, 3.1): every rank's
//                      local shards (fp32 cast to bf16, or bf16) -> the
//                      rank-major bf16 buffer, padding +0.
//   stock_pack_kernel  stock FSDP2's gradient pack of one rank (Section 2.1,
//                      Equation 3): slice, zero-pad, widen to fp32 and place
//                      rank-major; the baseline that the reduce-scatter above
//                      makes unnecessary.
//
// All are HBM-bandwidth bound: no MFMA, no atomics, no communication between
// waves.  Structure (shared):
//   * The plan's segments are cut into fixed-size chunks.  Every wave of the
//     grid is an independent worker, and chunks are dealt to waves round
//     robin (wave w takes chunks w, w + NW, w + 2 NW, ...), so at any moment
//     the whole grid streams through one compact window of each tensor.
//     (Measured on MI355X: this order keeps HBM 10-25% busier than giving
//     each workgroup a contiguous range of the tensors.)
//   * The chunk -> segment index (the segments' first-chunk table) is staged
//     in LDS once per workgroup; a wave finds the segment of its next chunk
//     with one 64-lane compare and ballot.  The segment's header and pointers
//     are then fetched with scalar loads one chunk ahead, so the scalar
//     fetch overlaps the vector loads of the current chunk.
//   * Vector bodies use non-temporal loads and contiguous 8- or 16-byte
//     stores; heads and tails of misaligned tensors take a scalar path, and a
//     source at another 16-byte phase than its destination is realigned in
//     registers (two aligned blocks per group, shifted).
//   * One launch covers a span of chunks; the host splits a long operation
//     into several launches, so that the waves of one launch cannot drift far
//     apart (which would widen the window).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <type_traits>

#include "tide_internal.h"

namespace {

using tide::CallHdr;
using tide::ChunkSpan;
using tide::KernelArgs;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Every tensor is in global memory; saying so (address space 1) makes the
// compiler emit global_* rather than flat_* accesses.
#define TIDE_GLOBAL __attribute__((address_space(1)))

template <typename T, bool CACHED>
__device__ __forceinline__ T load(const void* p) {
  const TIDE_GLOBAL T* q = (const TIDE_GLOBAL T*)(p);
  if constexpr (CACHED) {
    return *q;
  } else {
    return __builtin_nontemporal_load(q);
  }
}

template <typename T, bool CACHED>
__device__ __forceinline__ void store(void* p, T v) {
  TIDE_GLOBAL T* q = (TIDE_GLOBAL T*)(p);
  if constexpr (CACHED) {
    *q = v;
  } else {
    __builtin_nontemporal_store(v, q);
  }
}

__device__ __forceinline__ uint16_t load2(const uint16_t* p) { return *(const TIDE_GLOBAL uint16_t*)(p); }
__device__ __forceinline__ void store2(uint16_t* p, uint16_t v) { *(TIDE_GLOBAL uint16_t*)(p) = v; }
__device__ __forceinline__ float load4(const float* p) { return *(const TIDE_GLOBAL float*)(p); }
__device__ __forceinline__ void store4(float* p, float v) { *(TIDE_GLOBAL float*)(p) = v; }

// bf16 is the upper half of binary32, so widening is a shift (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Values all lanes hold identically are moved to scalar registers.
__device__ __forceinline__ int32_t sgpr(int32_t v) { return int32_t(__builtin_amdgcn_readfirstlane(uint32_t(v))); }

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ int lane_id() { return int(threadIdx.x & 63); }

// Groups each lane has in flight per step (measured on MI355X: two groups of
// W loads for the reduce-scatter of bf16 gradients, one of fp32 gradients,
// whose groups are twice as long; four 16-byte loads for the bf16 copies,
// eight for the casting and widening copies, whose groups are half as long on
// one side).
constexpr int kRsUnroll = 2;
constexpr int kCoUnroll = 4;
constexpr int kCastUnroll = 8;

// ---------------------------------------------------------------------------
// Chunk dealing and segment lookup (shared by every kernel)
// ---------------------------------------------------------------------------

// The chunk -> segment search table, as far as one launch needs it: the
// first-chunk indices of segments span.seg .. span.seg_end (the last entry
// bounds the launch's last segment), indexed relative to span.seg and staged
// in LDS when it fits (it is read by every chunk of every wave).  Staging only
// the launch's slice keeps the start of every launch short on plans of many
// tensors.
extern __shared__ int32_t s_chunk_begin[];

template <bool STAGED>
__device__ __forceinline__ const int32_t* chunk_table(const int32_t* __restrict__ chunk_begin, const ChunkSpan& sp) {
  if constexpr (STAGED) {
    const int32_t n = sp.seg_end - sp.seg;
    for (int i = threadIdx.x; i <= n; i += tide::kThreads) s_chunk_begin[i] = chunk_begin[sp.seg + i];
    __syncthreads();
    return s_chunk_begin;
  } else {
    return chunk_begin + sp.seg;
  }
}

// The plan's read-only tables, passed as separate restrict-qualified kernel
// arguments so that their (wave-uniform) loads go through the scalar cache.
struct Tables {
  const CallHdr* __restrict__ hdr;
  const void* const* __restrict__ ptrs;
  int32_t nsrc, chunk;
  ChunkSpan span;  // the chunks and segments of this launch
};

// Advance `cur` (wave-uniform, non-decreasing) to the segment holding chunk
// c: the largest s with cb[s] <= c, where cb[nseg] > c.  64 candidates per
// step.
__device__ __forceinline__ int32_t seek(const int32_t* cb, int32_t nseg, int32_t cur, int32_t c) {
  while (true) {
    const int32_t idx = cur + 1 + lane_id();
    const int32_t v = idx <= nseg ? cb[idx] : INT_MAX;
    const int32_t k = __popcll(__ballot(v <= c));
    cur += k;
    if (k < 64) return sgpr(cur);
  }
}

// A wave's view of one chunk.
struct Chunk {
  int64_t lo, vlo, vhi, hi;  // scalar [lo, vlo), vector groups [vlo, vhi), scalar [vhi, hi)
};

// Chunk j of a segment of `len` elements, `nch` chunks: chunk boundaries after
// the first sit at j*chunk + h, h being the segment's aligned-body start, so
// every chunk but the first starts on the vector body; the last chunk runs to
// the end.  Which wave handles which chunk never changes any result.
__device__ __forceinline__ Chunk chunk_range(const CallHdr& h, int64_t j, int64_t nch, int64_t chunk, int group) {
  const int64_t head = h.head > 0 ? h.head : 0;
  Chunk r;
  r.lo = (j == 0) ? 0 : min64(h.len, j * chunk + head);
  r.hi = (j == nch - 1) ? h.len : min64(h.len, (j + 1) * chunk + head);
  if (h.head < 0) {
    r.vlo = r.vhi = r.hi;
  } else {
    r.vlo = (j == 0) ? min64(head, r.hi) : r.lo;
    r.vhi = r.vlo + ((r.hi - r.vlo) / group) * group;
  }
  return r;
}

// Wave index in the grid and the wave count.
// Workgroups are dispatched round robin over the 8 XCDs (workgroup b runs on
// XCD b mod 8).  When the grid is a multiple of 8, workgroup b is renumbered
// so that each XCD owns a contiguous eighth of the waves, and hence of every
// window of chunks: one XCD's L2 and translation caches then see contiguous
// addresses.  (Measured: 1-3% over the plain numbering on MI355X.)
__device__ __forceinline__ void wave_slot(int32_t* w, int32_t* nw) {
  int32_t b = int32_t(blockIdx.x);
  const int32_t G = int32_t(gridDim.x);
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  *w = sgpr(b * tide::kWavesPerGroup + int32_t(threadIdx.x >> 6));
  *nw = int32_t(gridDim.x) * tide::kWavesPerGroup;
}

// Segment descriptor of the chunk a wave is about to process (wave-uniform):
// NS source pointers (none when the kernel reads them from the table as it
// goes) and the destination.
template <int NS>
struct Desc {
  CallHdr h;
  int32_t seg, j, nch;
  const void* src[NS > 0 ? NS : 1];
  void* dst;
};

template <int NS>
__device__ __forceinline__ void fetch(const Tables& a, const int32_t* cb, int32_t* cur, int32_t c, Desc<NS>* d) {
  *cur = seek(cb, a.span.seg_end - a.span.seg, *cur, c);  // relative to span.seg
  const int32_t s = a.span.seg + *cur;
  const int32_t first = sgpr(cb[*cur]);
  d->seg = s;
  d->j = c - first;
  d->nch = sgpr(cb[*cur + 1]) - first;
  d->h = a.hdr[s];
  const void* const* row = a.ptrs + int64_t(s) * (a.nsrc + 1);
#pragma unroll
  for (int u = 0; u < NS; ++u) d->src[u] = row[u];
  d->dst = const_cast<void*>(row[a.nsrc]);
}

// The persistent loop of every kernel: deal the launch's chunks to this wave
// round robin, fetch each chunk's descriptor one chunk ahead (the scalar loads
// overlap the vector loads of the current chunk) and hand the chunk to `body`.
template <int NS, bool STAGED, typename Body>
__device__ __forceinline__ void for_each_chunk(const Tables& a, const int32_t* __restrict__ chunk_begin, Body body) {
  const int32_t* cb = chunk_table<STAGED>(chunk_begin, a.span);
  int32_t w, nw;
  wave_slot(&w, &nw);
  const int32_t end = a.span.end;
  int32_t cur = 0;
  int32_t c = a.span.first + w;
  Desc<NS> next;
  if (c < end) fetch<NS>(a, cb, &cur, c, &next);
  while (c < end) {
    const Desc<NS> d = next;
    const int32_t cn = c + nw;
    if (cn < end) fetch<NS>(a, cb, &cur, cn, &next);
    body(d);
    c = cn;
  }
}

// ---------------------------------------------------------------------------
// Reduce-scatter local stage
// ---------------------------------------------------------------------------

// Source types.  A vector group is 4 elements: 8 bytes of bf16 or 16 bytes of
// fp32 per source.  first() starts the sum with rank 0's value, add() adds
// the next rank's: one binary32 addition per element, no contraction.
template <bool F32>
struct Src;

template <>
struct Src<false> {
  using T = uint16_t;
  using V = u32x2;
  static __device__ __forceinline__ void first(V v, float a[4]) {
    a[0] = bf16_lo(v.x);
    a[1] = bf16_hi(v.x);
    a[2] = bf16_lo(v.y);
    a[3] = bf16_hi(v.y);
  }
  static __device__ __forceinline__ void add(V v, float a[4]) {
    a[0] = a[0] + bf16_lo(v.x);
    a[1] = a[1] + bf16_hi(v.x);
    a[2] = a[2] + bf16_lo(v.y);
    a[3] = a[3] + bf16_hi(v.y);
  }
  static __device__ __forceinline__ float one(const void* p, int64_t e) {
    return bf16_to_f32(load2(static_cast<const uint16_t*>(p) + e));
  }
};

template <>
struct Src<true> {
  using T = float;
  using V = f32x4;
  static __device__ __forceinline__ void first(V v, float a[4]) {
    a[0] = v.x;
    a[1] = v.y;
    a[2] = v.z;
    a[3] = v.w;
  }
  static __device__ __forceinline__ void add(V v, float a[4]) {
    a[0] = a[0] + v.x;
    a[1] = a[1] + v.y;
    a[2] = a[2] + v.z;
    a[3] = a[3] + v.w;
  }
  static __device__ __forceinline__ float one(const void* p, int64_t e) {
    return load4(static_cast<const float*>(p) + e);
  }
};

// Equation 5's scale and accumulate, applied to a finished sum: one binary32
// product, then (accumulating) one binary32 addition of the value already in
// the shard.  kPlain (alpha = 1, no accumulation) stores the sum as it is.
// The mode is uniform over the grid and chosen once per chunk, so the default
// path's loop carries no trace of the epilogue.  When accumulating, the old
// shard values are loaded together with the sources, so their latency hides
// behind the same wait, and non-temporally like them (measured on MI355X:
// 7-9% faster than cached loads of the values about to be overwritten).
enum Epi : int { kPlain = 0, kScale = 1, kScaleAcc = 2 };

template <int EPI, bool CL>
__device__ __forceinline__ f32x4 old4(const float* d) {
  if constexpr (EPI == kScaleAcc) {
    return load<f32x4, CL>(d);
  } else {
    return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

template <bool CS, int EPI>
__device__ __forceinline__ void put4(float* d, const float a[4], float alpha, f32x4 old) {
  if constexpr (EPI == kPlain) {
    store<f32x4, CS>(d, f32x4{a[0], a[1], a[2], a[3]});
  } else {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = alpha * a[i];
    if constexpr (EPI == kScaleAcc) {
      v[0] = old.x + v[0];
      v[1] = old.y + v[1];
      v[2] = old.z + v[2];
      v[3] = old.w + v[3];
    }
    store<f32x4, CS>(d, f32x4{v[0], v[1], v[2], v[3]});
  }
}

template <int EPI>
__device__ __forceinline__ void put1(float* d, float s, float alpha) {
  if constexpr (EPI == kPlain) {
    store4(d, s);
  } else {
    float v = alpha * s;
    if constexpr (EPI == kScaleAcc) v = load4(d) + v;
    store4(d, v);
  }
}

// Sum of the W sources at element e (scalar path), rank order 0..W-1.
template <bool F32>
__device__ __forceinline__ float sum_one(const void* const* src, int32_t W, int64_t e) {
  float acc = Src<F32>::one(src[0], e);
  for (int32_t u = 1; u < W; ++u) acc = acc + Src<F32>::one(src[u], e);
  return acc;
}

// One batch of NB consecutive ranks u0 .. u0+NB-1 for U groups of 4 elements
// per lane, the first at group index g0 of the chunk body starting at vlo:
// all NB*U loads first, then the additions in rank order into acc; FIRST
// starts the sums with rank u0's value.  Loads address a scalar base plus a
// 32-bit lane offset, as in the templated paths.
template <bool F32, bool CL, int U, int NB, bool FIRST>
__device__ __forceinline__ void rs_batch(const void* const* src, int32_t u0, int64_t vlo, int64_t g0,
                                         float (&acc)[U][4]) {
  using S = Src<F32>;
  using T = typename S::T;
  using V = typename S::V;
  constexpr int kGroupBytes = 4 * int(sizeof(T));
  const char* s[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) s[j] = reinterpret_cast<const char*>(static_cast<const T*>(src[u0 + j]) + vlo);
  V v[U][NB];
#pragma unroll
  for (int k = 0; k < U; ++k) {
#pragma unroll
    for (int j = 0; j < NB; ++j) v[k][j] = load<V, CL>(s[j] + uint32_t((g0 + 64 * k) * kGroupBytes));
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (FIRST && j == 0) {
        S::first(v[k][0], acc[k]);
      } else {
        S::add(v[k][j], acc[k]);
      }
    }
  }
}

// A batch of nb (1..8, wave-uniform) ranks.
template <bool F32, bool CL, int U, bool FIRST>
__device__ __forceinline__ void rs_batch_n(int32_t nb, const void* const* src, int32_t u0, int64_t vlo, int64_t g0,
                                           float (&acc)[U][4]) {
  switch (nb) {
    case 1: rs_batch<F32, CL, U, 1, FIRST>(src, u0, vlo, g0, acc); break;
    case 2: rs_batch<F32, CL, U, 2, FIRST>(src, u0, vlo, g0, acc); break;
    case 3: rs_batch<F32, CL, U, 3, FIRST>(src, u0, vlo, g0, acc); break;
    case 4: rs_batch<F32, CL, U, 4, FIRST>(src, u0, vlo, g0, acc); break;
    case 5: rs_batch<F32, CL, U, 5, FIRST>(src, u0, vlo, g0, acc); break;
    case 6: rs_batch<F32, CL, U, 6, FIRST>(src, u0, vlo, g0, acc); break;
    case 7: rs_batch<F32, CL, U, 7, FIRST>(src, u0, vlo, g0, acc); break;
    default: rs_batch<F32, CL, U, 8, FIRST>(src, u0, vlo, g0, acc); break;
  }
}

// Instances of the reduce-scatter for a W fixed at run time (WT <= 0).  Their
// steps cover twice the groups per lane of the templated W = 8 path (batches
// of up to 8 sources, often fewer in the last one; measured on MI355X: 3-15%
// faster than the W = 8 step width for every W tried, 5 to 64).
constexpr int kAnyW = 0;
// bf16, W <= 3 with chunks of at least 2048 elements: four times the groups per
// step of the W = 8 path.
constexpr int kAnyTinyW = -4;
// Any W, for calls with sum segments whose sources are off the destination's
// phase: the any-W body plus the realigned one.
constexpr int kAnyWShift = -2;

// Full steps of U groups per lane over the chunk body [vlo, vlo + 4 ng) for
// any W: batches of 8 ranks (the last one shorter), each batch's loads issued
// together; each batch's source pointers come from the call table through
// the scalar cache.  Returns where the steps stopped.
template <bool F32, bool CL, bool CS, int EPI, int U>
__device__ __forceinline__ int64_t any_steps(const void* const* src, int32_t W, float* dst, int64_t vlo, int64_t ng,
                                             int64_t g, float alpha) {
  const int32_t full = W >> 3, rest = W & 7;
  float* d = dst + vlo;
  int64_t base = 0;
  for (; base + 64 * U <= ng; base += 64 * U) {
    float acc[U][4];
    f32x4 o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) o[k] = old4<EPI, CL>(d + (base + g + 64 * k) * 4);
    if (full > 0) {
      rs_batch<F32, CL, U, 8, true>(src, 0, vlo, base + g, acc);
      for (int32_t b = 1; b < full; ++b) rs_batch<F32, CL, U, 8, false>(src, b * 8, vlo, base + g, acc);
      if (rest > 0) rs_batch_n<F32, CL, U, false>(rest, src, full * 8, vlo, base + g, acc);
    } else {
      rs_batch_n<F32, CL, U, true>(rest, src, 0, vlo, base + g, acc);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) put4<CS, EPI>(d + (base + g + 64 * k) * 4, acc[k], alpha, o[k]);
  }
  return base;
}

// Four bf16 elements starting PS elements (1..3) into the 16 bytes a, b.
template <int PS>
__device__ __forceinline__ u32x2 shift4h(u32x2 a, u32x2 b) {
  const uint32_t w[4] = {a.x, a.y, b.x, b.y};
  constexpr int q = PS >> 1;
  if constexpr ((PS & 1) != 0) {
    return u32x2{__builtin_amdgcn_alignbyte(w[q + 1], w[q], 2), __builtin_amdgcn_alignbyte(w[q + 2], w[q + 1], 2)};
  } else {
    return u32x2{w[q], w[q + 1]};
  }
}

// Four fp32 elements starting PS elements (1..3) into the 32 bytes a, b.
template <int PS>
__device__ __forceinline__ f32x4 shift4(f32x4 a, f32x4 b) {
  const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return f32x4{w[PS], w[PS + 1], w[PS + 2], w[PS + 3]};
}

// A realigned group of 4 source elements starting PS elements past a block
// boundary: the aligned blocks a (holding the first element) and b (the next).
template <bool F32, int PS>
__device__ __forceinline__ typename Src<F32>::V shift_group(typename Src<F32>::V a, typename Src<F32>::V b) {
  if constexpr (F32) {
    return shift4<PS>(a, b);
  } else {
    return shift4h<PS>(a, b);
  }
}

// rs_batch for sources PS elements (1..3) past a group boundary at the
// chunk body's start, where the destination is 16-byte aligned: each source
// group is built from the two aligned blocks that hold it (both hold
// elements of the group, so no load leaves the source's pages).
template <bool F32, bool CL, int U, int NB, bool FIRST, int PS>
__device__ __forceinline__ void rs_batch_shift(const void* const* src, int32_t u0, int64_t vlo, int64_t g0,
                                               float (&acc)[U][4]) {
  using S = Src<F32>;
  using T = typename S::T;
  using V = typename S::V;
  constexpr int kGroupBytes = 4 * int(sizeof(T));
  const char* s[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) s[j] = reinterpret_cast<const char*>(static_cast<const T*>(src[u0 + j]) + vlo - PS);
  V a[U][NB], b[U][NB];
#pragma unroll
  for (int k = 0; k < U; ++k) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      a[k][j] = load<V, CL>(s[j] + uint32_t((g0 + 64 * k) * kGroupBytes));
      b[k][j] = load<V, CL>(s[j] + uint32_t((g0 + 64 * k + 1) * kGroupBytes));
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const V v = shift_group<F32, PS>(a[k][j], b[k][j]);
      if (FIRST && j == 0) {
        S::first(v, acc[k]);
      } else {
        S::add(v, acc[k]);
      }
    }
  }
}

template <bool F32, bool CL, int U, bool FIRST, int PS>
__device__ __forceinline__ void rs_batch_shift_n(int32_t nb, const void* const* src, int32_t u0, int64_t vlo,
                                                 int64_t g0, float (&acc)[U][4]) {
  switch (nb) {
    case 1: rs_batch_shift<F32, CL, U, 1, FIRST, PS>(src, u0, vlo, g0, acc); break;
    case 2: rs_batch_shift<F32, CL, U, 2, FIRST, PS>(src, u0, vlo, g0, acc); break;
    case 3: rs_batch_shift<F32, CL, U, 3, FIRST, PS>(src, u0, vlo, g0, acc); break;
    case 4: rs_batch_shift<F32, CL, U, 4, FIRST, PS>(src, u0, vlo, g0, acc); break;
    case 5: rs_batch_shift<F32, CL, U, 5, FIRST, PS>(src, u0, vlo, g0, acc); break;
    case 6: rs_batch_shift<F32, CL, U, 6, FIRST, PS>(src, u0, vlo, g0, acc); break;
    case 7: rs_batch_shift<F32, CL, U, 7, FIRST, PS>(src, u0, vlo, g0, acc); break;
    default: rs_batch_shift<F32, CL, U, 8, FIRST, PS>(src, u0, vlo, g0, acc); break;
  }
}

// Realigned sum body for any W: full steps as in any_steps, then the groups
// left over element by element (so that no load is unaligned).
template <bool F32, bool CL, bool CS, int EPI, int PS>
__device__ __forceinline__ void shift_sum_body(const void* const* src, int32_t W, float* dst, int64_t vlo,
                                               int64_t vhi, float alpha) {
  constexpr int U = F32 ? 1 : kRsUnroll;
  const int64_t ng = (vhi - vlo) >> 2;
  const int64_t g = lane_id();
  const int32_t full = W >> 3, rest = W & 7;
  float* d = dst + vlo;
  int64_t base = 0;
  for (; base + 64 * U <= ng; base += 64 * U) {
    float acc[U][4];
    f32x4 o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) o[k] = old4<EPI, CL>(d + (base + g + 64 * k) * 4);
    if (full > 0) {
      rs_batch_shift<F32, CL, U, 8, true, PS>(src, 0, vlo, base + g, acc);
      for (int32_t b = 1; b < full; ++b) rs_batch_shift<F32, CL, U, 8, false, PS>(src, b * 8, vlo, base + g, acc);
      if (rest > 0) rs_batch_shift_n<F32, CL, U, false, PS>(rest, src, full * 8, vlo, base + g, acc);
    } else {
      rs_batch_shift_n<F32, CL, U, true, PS>(rest, src, 0, vlo, base + g, acc);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) put4<CS, EPI>(d + (base + g + 64 * k) * 4, acc[k], alpha, o[k]);
  }
  for (int64_t e = vlo + base * 4 + g; e < vhi; e += 64) put1<EPI>(dst + e, sum_one<F32>(src, W, e), alpha);
}

// Vector body of a sum chunk: groups of 4 elements in [vlo, vhi), every
// source and the destination group-aligned there.  Lane l handles groups
// l, l + 64, ...; kRsUnroll groups per step keep kRsUnroll*W independent loads
// in flight; the remainder of a partial chunk goes one group per step.
template <int WT, bool F32, bool CL, bool CS, int EPI>
__device__ __forceinline__ void sum_body(const void* const* src, int32_t W, float* dst, int64_t vlo, int64_t vhi,
                                         float alpha) {
  using S = Src<F32>;
  using T = typename S::T;
  using V = typename S::V;
  constexpr int kGroupBytes = 4 * int(sizeof(T));
  const int64_t ng = (vhi - vlo) >> 2;
  const int64_t g = lane_id();
  if constexpr (WT > 0) {
    constexpr int U = WT <= 4 ? 2 * kRsUnroll : kRsUnroll;  // bf16 only, see below
    const T* s[WT];
#pragma unroll
    for (int u = 0; u < WT; ++u) s[u] = static_cast<const T*>(src[u]) + vlo;
    float* d = dst + vlo;
    // Source loads address a scalar base (the chunk body's start) plus a
    // 32-bit lane offset: two scalar registers per source, so that the next
    // chunk's descriptor, fetched meanwhile, stays in scalar registers and no
    // wait for it is needed before this chunk's loads.
    // bf16 sources: U groups per lane per step (twice as many for W = 4, whose
    // groups have half the sources).  fp32 sources have twice the bytes per
    // group and take one group per lane per step, the loop after this one;
    // either way a wave of the W = 8 path has 8 KiB of source loads in flight
    // (measured on MI355X: twice that is 6-9% slower for fp32, as it is for
    // bf16).
    int64_t base = 0;
    if constexpr (!F32) {
      for (; base + 64 * U <= ng; base += 64 * U) {
        V v[U][WT];
        f32x4 o[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
#pragma unroll
          for (int u = 0; u < WT; ++u)
            v[k][u] = load<V, CL>(reinterpret_cast<const char*>(s[u]) + uint32_t((base + g + 64 * k) * kGroupBytes));
          o[k] = old4<EPI, CL>(d + (base + g + 64 * k) * 4);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
          float a[4];
          S::first(v[k][0], a);
#pragma unroll
          for (int u = 1; u < WT; ++u) S::add(v[k][u], a);
          put4<CS, EPI>(d + (base + g + 64 * k) * 4, a, alpha, o[k]);
        }
      }
    }
    for (int64_t gk = base + g; gk < ng; gk += 64) {
      V v[WT];
#pragma unroll
      for (int u = 0; u < WT; ++u) v[u] = load<V, CL>(s[u] + gk * 4);
      const f32x4 o = old4<EPI, CL>(d + gk * 4);
      float a[4];
      S::first(v[0], a);
#pragma unroll
      for (int u = 1; u < WT; ++u) S::add(v[u], a);
      put4<CS, EPI>(d + gk * 4, a, alpha, o);
    }
  } else {
    // Any W: sources in batches of 8 (the last one shorter), added in rank
    // order into accumulators that carry from batch to batch.  A step covers
    // twice the groups per lane of the templated W = 8 path (four times with
    // W <= 3), since a batch often holds fewer than 8 sources.
    constexpr int U = (WT == kAnyTinyW ? 4 : 2) * (F32 ? 1 : kRsUnroll);
    const int64_t base = any_steps<F32, CL, CS, EPI, U>(src, W, dst, vlo, ng, g, alpha);
    // the groups left over (fewer than one step's), one per lane
    for (int64_t gk = base + g; gk < ng; gk += 64) {
      const int64_t e = vlo + gk * 4;
      float acc[4];
      S::first(load<V, CL>(static_cast<const T*>(src[0]) + e), acc);
      for (int32_t u0 = 1; u0 < W; u0 += 8) {
        const int32_t nb = (W - u0) < 8 ? (W - u0) : 8;
        V v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nb) v[k] = load<V, CL>(static_cast<const T*>(src[u0 + k]) + e);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nb) S::add(v[k], acc);
      }
      put4<CS, EPI>(dst + e, acc, alpha, old4<EPI, CL>(dst + e));
    }
  }
}

// Padding rows: every rank contributes zeros there, so the sum is +0.
template <bool CL, bool CS, int EPI>
__device__ __forceinline__ void zero_rows(float* dst, const Chunk& c, float alpha) {
  const int lane = lane_id();
  const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t e = c.lo + lane; e < c.vlo; e += 64) put1<EPI>(dst + e, 0.0f, alpha);
  for (int64_t e = c.vhi + lane; e < c.hi; e += 64) put1<EPI>(dst + e, 0.0f, alpha);
  for (int64_t e = c.vlo + int64_t(lane) * 4; e < c.vhi; e += 256)
    put4<CS, EPI>(dst + e, z, alpha, old4<EPI, CL>(dst + e));
}

// Elements (0..3) by which a source is past a group boundary at element e.
template <bool F32>
__device__ __forceinline__ int src_phase(const void* src, int64_t e) {
  using T = typename Src<F32>::T;
  const uintptr_t sa = reinterpret_cast<uintptr_t>(static_cast<const T*>(src) + e);
  return sgpr(int32_t((sa & (4 * sizeof(T) - 1)) / sizeof(T)));
}

// One chunk of the reduce-scatter: the sum of a kSum segment's piece, or the
// zeros of a padding piece.
template <int WT, bool F32, bool CL, bool CS, int EPI>
__device__ __forceinline__ void rs_chunk(const Tables& a, const Desc<WT>& d, int32_t W, float alpha) {
  float* dst = static_cast<float*>(d.dst);
  const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 4);
  if (d.h.kind == tide::kZero) {
    zero_rows<CL, CS, EPI>(dst, r, alpha);
    return;
  }
  // any W: the sources are read from the call table as needed
  const void* const* src = WT > 0 ? d.src : a.ptrs + int64_t(d.seg) * (a.nsrc + 1);
  const int lane = lane_id();
  for (int64_t e = r.lo + lane; e < r.vlo; e += 64) put1<EPI>(dst + e, sum_one<F32>(src, W, e), alpha);
  for (int64_t e = r.vhi + lane; e < r.hi; e += 64) put1<EPI>(dst + e, sum_one<F32>(src, W, e), alpha);
  if (r.vhi <= r.vlo) return;
  // The destination is 16-byte aligned at vlo and all W sources share one
  // phase; sources off a group boundary there are realigned by the instance
  // launched for calls that have such segments (the others never meet one:
  // should they, the chunk goes element by element).
  const int ps = src_phase<F32>(src[0], r.vlo);
  if constexpr (WT == kAnyWShift) {
    switch (ps) {
      case 0: sum_body<kAnyW, F32, CL, CS, EPI>(src, W, dst, r.vlo, r.vhi, alpha); break;
      case 1: shift_sum_body<F32, CL, CS, EPI, 1>(src, W, dst, r.vlo, r.vhi, alpha); break;
      case 2: shift_sum_body<F32, CL, CS, EPI, 2>(src, W, dst, r.vlo, r.vhi, alpha); break;
      default: shift_sum_body<F32, CL, CS, EPI, 3>(src, W, dst, r.vlo, r.vhi, alpha); break;
    }
  } else if (ps == 0) {
    sum_body<WT, F32, CL, CS, EPI>(src, W, dst, r.vlo, r.vhi, alpha);
  } else {
    const void* const* row = a.ptrs + int64_t(d.seg) * (a.nsrc + 1);
    for (int64_t e = r.vlo + lane; e < r.vhi; e += 64) put1<EPI>(dst + e, sum_one<F32>(row, W, e), alpha);
  }
}

template <int WT, bool F32, bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void rs_local_kernel(const CallHdr* __restrict__ hdr,
                                                                  const void* const* __restrict__ ptrs,
                                                                  const int32_t* __restrict__ chunk_begin,
                                                                  int32_t nsrc, ChunkSpan span,
                                                                  int32_t chunk, float alpha, int32_t accumulate) {
  const Tables a{hdr, ptrs, nsrc, chunk, span};
  const int epi = accumulate != 0 ? kScaleAcc : !(alpha == 1.0f) ? kScale : kPlain;
  const int32_t W = WT > 0 ? WT : nsrc;
  for_each_chunk<WT, STAGED>(a, chunk_begin, [&](const Desc<WT>& d) {
    switch (epi) {
      case kPlain: rs_chunk<WT, F32, CL, CS, kPlain>(a, d, W, alpha); break;
      case kScale: rs_chunk<WT, F32, CL, CS, kScale>(a, d, W, alpha); break;
      default: rs_chunk<WT, F32, CL, CS, kScaleAcc>(a, d, W, alpha); break;
    }
  });
}

// ---------------------------------------------------------------------------
// Copies: all-gather copy-out and copy-in, stock gradient pack
// ---------------------------------------------------------------------------

// Full steps of U groups of 8 bf16 per lane (all loads issued before the
// stores); returns where the steps stopped.
template <int U, bool CL, bool CS>
__device__ __forceinline__ int64_t copy_steps(const uint16_t* sv, uint16_t* dv, int64_t base, int64_t ng, int lane) {
  for (; base + 64 * U <= ng; base += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = load<u32x4, CL>(sv + (base + lane + 64 * k) * 8);
#pragma unroll
    for (int k = 0; k < U; ++k) store<u32x4, CS>(dv + (base + lane + 64 * k) * 8, v[k]);
  }
  return base;
}

// Eight bf16 elements starting PS elements (1..7) into the 32 bytes a, b:
// a funnel shift of the two 16-byte blocks.
template <int PS>
__device__ __forceinline__ u32x4 shift8(u32x4 a, u32x4 b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  constexpr int q = PS >> 1;
  if constexpr ((PS & 1) != 0) {
    return u32x4{__builtin_amdgcn_alignbyte(w[q + 1], w[q], 2), __builtin_amdgcn_alignbyte(w[q + 2], w[q + 1], 2),
                 __builtin_amdgcn_alignbyte(w[q + 3], w[q + 2], 2), __builtin_amdgcn_alignbyte(w[q + 4], w[q + 3], 2)};
  } else {
    return u32x4{w[q], w[q + 1], w[q + 2], w[q + 3]};
  }
}

// Realigned steps of U groups of 8 per lane: the destination is 16-byte
// aligned, the source PS elements past a 16-byte boundary, so destination
// group k takes source blocks k and k + 1 of the aligned blocks sb[] (both
// hold elements of the group, so no load leaves the source's pages; the
// second is the neighbouring lane's first and comes from the cache).
template <int PS, int U, bool CL, bool CS>
__device__ __forceinline__ int64_t shift_steps(const u32x4* sb, uint16_t* dv, int64_t base, int64_t ng, int lane) {
  for (; base + 64 * U <= ng; base += 64 * U) {
    u32x4 a[U], b[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      a[k] = load<u32x4, CL>(sb + (base + lane + 64 * k));
      b[k] = load<u32x4, CL>(sb + (base + lane + 64 * k + 1));
    }
#pragma unroll
    for (int k = 0; k < U; ++k) store<u32x4, CS>(dv + (base + lane + 64 * k) * 8, shift8<PS>(a[k], b[k]));
  }
  return base;
}

template <int PS, bool CL, bool CS>
__device__ __forceinline__ void shift_body(const uint16_t* sv, uint16_t* dv, int64_t ng, int lane) {
  const u32x4* sb = reinterpret_cast<const u32x4*>(sv - PS);
  int64_t base = shift_steps<PS, kCoUnroll, CL, CS>(sb, dv, 0, ng, lane);
  base = shift_steps<PS, 1, CL, CS>(sb, dv, base, ng, lane);
  for (int64_t gk = base + lane; gk < ng; gk += 64)
    store<u32x4, CS>(dv + gk * 8, shift8<PS>(load<u32x4, CL>(sb + gk), load<u32x4, CL>(sb + gk + 1)));
}

// bf16 [lo, hi): groups of 8 in [vlo, vhi), where the destination is 16-byte
// aligned (kCoUnroll 16-byte loads in flight per lane, then two, then one;
// a source at another 16-byte phase takes the realigned body), the rest
// element by element.
template <bool CL, bool CS>
__device__ __forceinline__ void copy_chunk(const uint16_t* src, uint16_t* dst, const Chunk& r) {
  const int lane = lane_id();
  for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(dst + e, load2(src + e));
  for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(dst + e, load2(src + e));
  if (r.vhi <= r.vlo) return;
  const uint16_t* sv = src + r.vlo;
  uint16_t* dv = dst + r.vlo;
  const int64_t ng = (r.vhi - r.vlo) >> 3;
  const int ps = sgpr(int32_t((reinterpret_cast<uintptr_t>(sv) & 15) >> 1));
  switch (ps) {
    case 0: break;
    case 1: shift_body<1, CL, CS>(sv, dv, ng, lane); return;
    case 2: shift_body<2, CL, CS>(sv, dv, ng, lane); return;
    case 3: shift_body<3, CL, CS>(sv, dv, ng, lane); return;
    case 4: shift_body<4, CL, CS>(sv, dv, ng, lane); return;
    case 5: shift_body<5, CL, CS>(sv, dv, ng, lane); return;
    case 6: shift_body<6, CL, CS>(sv, dv, ng, lane); return;
    default: shift_body<7, CL, CS>(sv, dv, ng, lane); return;
  }
  int64_t base = 0;
  base = copy_steps<kCoUnroll, CL, CS>(sv, dv, base, ng, lane);
  base = copy_steps<2, CL, CS>(sv, dv, base, ng, lane);
  for (int64_t gk = base + lane; gk < ng; gk += 64) store<u32x4, CS>(dv + gk * 8, load<u32x4, CL>(sv + gk * 8));
}

template <bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void ag_copyout_kernel(const CallHdr* __restrict__ hdr,
                                                                    const void* const* __restrict__ ptrs,
                                                                    const int32_t* __restrict__ chunk_begin,
                                                                    ChunkSpan span, int32_t chunk) {
  const Tables a{hdr, ptrs, 1, chunk, span};
  for_each_chunk<1, STAGED>(a, chunk_begin, [&](const Desc<1>& d) {
    copy_chunk<CL, CS>(static_cast<const uint16_t*>(d.src[0]), static_cast<uint16_t*>(d.dst),
                       chunk_range(d.h, d.j, d.nch, a.chunk, 8));
  });
}

// fp32 -> bf16, round to nearest even, on the bit pattern; a NaN stays a NaN
// of the same sign with its top payload bits and the quiet bit set.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ u32x2 cast4(f32x4 v) {
  return u32x2{f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16), f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16)};
}

template <int U, bool CL, bool CS>
__device__ __forceinline__ int64_t cast_steps(const float* sv, uint16_t* dv, int64_t base, int64_t ng, int lane) {
  for (; base + 64 * U <= ng; base += 64 * U) {
    f32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = load<f32x4, CL>(sv + (base + lane + 64 * k) * 4);
#pragma unroll
    for (int k = 0; k < U; ++k) store<u32x2, CS>(dv + (base + lane + 64 * k) * 4, cast4(v[k]));
  }
  return base;
}


// Realigned cast body: the destination is 8-byte aligned, the source PS fp32
// elements past a 16-byte boundary; destination group k takes aligned source
// blocks k and k + 1 (both hold elements of the group).
template <int PS, bool CL, bool CS>
__device__ __forceinline__ void cast_shift_body(const float* sv, uint16_t* dv, int64_t ng, int lane) {
  const f32x4* sb = reinterpret_cast<const f32x4*>(sv - PS);
  constexpr int U = kCastUnroll;
  int64_t base = 0;
  for (; base + 64 * U <= ng; base += 64 * U) {
    f32x4 a[U], b[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      a[k] = load<f32x4, CL>(sb + (base + lane + 64 * k));
      b[k] = load<f32x4, CL>(sb + (base + lane + 64 * k + 1));
    }
#pragma unroll
    for (int k = 0; k < U; ++k) store<u32x2, CS>(dv + (base + lane + 64 * k) * 4, cast4(shift4<PS>(a[k], b[k])));
  }
  for (int64_t gk = base + lane; gk < ng; gk += 64)
    store<u32x2, CS>(dv + gk * 4, cast4(shift4<PS>(load<f32x4, CL>(sb + gk), load<f32x4, CL>(sb + gk + 1))));
}

// fp32 [lo, hi) -> bf16: groups of 4 in [vlo, vhi), where the destination is
// 8-byte aligned (16-byte loads, 8-byte stores, each contiguous across the
// wave; a source at another 16-byte phase takes the realigned body), the rest
// element by element.
template <bool CL, bool CS>
__device__ __forceinline__ void cast_chunk(const float* src, uint16_t* dst, const Chunk& r) {
  const int lane = lane_id();
  for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(dst + e, uint16_t(f32_to_bf16(load4(src + e))));
  for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(dst + e, uint16_t(f32_to_bf16(load4(src + e))));
  if (r.vhi <= r.vlo) return;
  const float* sv = src + r.vlo;
  uint16_t* dv = dst + r.vlo;
  const int64_t ng = (r.vhi - r.vlo) >> 2;
  const int ps = sgpr(int32_t((reinterpret_cast<uintptr_t>(sv) & 15) >> 2));
  switch (ps) {
    case 0: break;
    case 1: cast_shift_body<1, CL, CS>(sv, dv, ng, lane); return;
    case 2: cast_shift_body<2, CL, CS>(sv, dv, ng, lane); return;
    default: cast_shift_body<3, CL, CS>(sv, dv, ng, lane); return;
  }
  int64_t base = 0;
  base = cast_steps<kCastUnroll, CL, CS>(sv, dv, base, ng, lane);
  base = cast_steps<2, CL, CS>(sv, dv, base, ng, lane);
  for (int64_t gk = base + lane; gk < ng; gk += 64) store<u32x2, CS>(dv + gk * 4, cast4(load<f32x4, CL>(sv + gk * 4)));
}

template <bool F32, bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void ag_copyin_kernel(const CallHdr* __restrict__ hdr,
                                                                   const void* const* __restrict__ ptrs,
                                                                   const int32_t* __restrict__ chunk_begin,
                                                                   ChunkSpan span, int32_t chunk) {
  const Tables a{hdr, ptrs, 1, chunk, span};
  for_each_chunk<1, STAGED>(a, chunk_begin, [&](const Desc<1>& d) {
    uint16_t* dst = static_cast<uint16_t*>(d.dst);
    const int lane = lane_id();
    if (d.h.kind == tide::kZero) {
      // padding of the rank-major slot: bf16 +0
      const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 8);
      for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(dst + e, 0);
      for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(dst + e, 0);
      for (int64_t e = r.vlo + int64_t(lane) * 8; e < r.vhi; e += 512) store<u32x4, CS>(dst + e, u32x4{0, 0, 0, 0});
    } else if constexpr (F32) {
      cast_chunk<CL, CS>(static_cast<const float*>(d.src[0]), dst, chunk_range(d.h, d.j, d.nch, a.chunk, 4));
    } else {
      copy_chunk<CL, CS>(static_cast<const uint16_t*>(d.src[0]), dst, chunk_range(d.h, d.j, d.nch, a.chunk, 8));
    }
  });
}

template <bool CL, bool CS>
__device__ __forceinline__ void widen_group(const uint16_t* s, float* d) {
  float v[4];
  Src<false>::first(load<u32x2, CL>(s), v);
  store<f32x4, CS>(d, f32x4{v[0], v[1], v[2], v[3]});
}

// Full steps of U groups of 4 bf16 per lane widened to fp32 (all loads
// issued before the stores); returns where the steps stopped.
template <int U, bool CL, bool CS>
__device__ __forceinline__ int64_t widen_steps(const uint16_t* sv, float* dv, int64_t base, int64_t ng, int lane) {
  for (; base + 64 * U <= ng; base += 64 * U) {
    u32x2 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = load<u32x2, CL>(sv + (base + lane + 64 * k) * 4);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      float a[4];
      Src<false>::first(v[k], a);
      store<f32x4, CS>(dv + (base + lane + 64 * k) * 4, f32x4{a[0], a[1], a[2], a[3]});
    }
  }
  return base;
}

// Stock gradient pack of one rank: its bf16 rows widened to fp32 (groups of
// 4: 8-byte loads, 16-byte stores; kCastUnroll groups in flight per lane, then
// two, then one), padding rows +0.
template <bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void stock_pack_kernel(const CallHdr* __restrict__ hdr,
                                                                    const void* const* __restrict__ ptrs,
                                                                    const int32_t* __restrict__ chunk_begin,
                                                                    ChunkSpan span, int32_t chunk) {
  const Tables a{hdr, ptrs, 1, chunk, span};
  for_each_chunk<1, STAGED>(a, chunk_begin, [&](const Desc<1>& d) {
    float* dst = static_cast<float*>(d.dst);
    const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 4);
    const int lane = lane_id();
    if (d.h.kind == tide::kZero) {
      for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store4(dst + e, 0.0f);
      for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store4(dst + e, 0.0f);
      for (int64_t e = r.vlo + int64_t(lane) * 4; e < r.vhi; e += 256)
        store<f32x4, CS>(dst + e, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
      return;
    }
    const uint16_t* src = static_cast<const uint16_t*>(d.src[0]);
    for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store4(dst + e, bf16_to_f32(load2(src + e)));
    for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store4(dst + e, bf16_to_f32(load2(src + e)));
    if (r.vhi <= r.vlo) return;
    const uint16_t* sv = src + r.vlo;
    float* dv = dst + r.vlo;
    const int64_t ng = (r.vhi - r.vlo) >> 2;
    int64_t base = 0;
    base = widen_steps<kCastUnroll, CL, CS>(sv, dv, base, ng, lane);
    base = widen_steps<2, CL, CS>(sv, dv, base, ng, lane);
    for (int64_t gk = base + lane; gk < ng; gk += 64) widen_group<CL, CS>(sv + gk * 4, dv + gk * 4);
  });
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// LDS for the staged chunk table; large tables, and calls with
// TIDE_FLAG_NO_LDS, keep it in global memory.
size_t staged_bytes(const KernelArgs& a, bool* staged) {
  const int32_t n = a.span.seg_end - a.span.seg;  // entries n + 1
  *staged = n <= tide::kMaxStagedSegs && !(a.flags & TIDE_FLAG_NO_LDS);
  return *staged ? size_t(n + 1) * sizeof(int32_t) : 0;
}

// Calls f(CL, CS, STAGED, lds_bytes) with the kernel instance's flags as
// std::bool_constant values, chosen from the call's flags and table size.
template <typename F>
void by_instance(const KernelArgs& a, F f) {
  bool staged;
  const size_t lds = staged_bytes(a, &staged);
  const bool cl = a.flags & TIDE_FLAG_CACHED_LOADS, cs = a.flags & TIDE_FLAG_CACHED_STORES;
  auto go = [&](auto CL, auto CS) {
    if (staged) {
      f(CL, CS, std::true_type{}, lds);
    } else {
      f(CL, CS, std::false_type{}, size_t(0));
    }
  };
  if (cl && cs) {
    go(std::true_type{}, std::true_type{});
  } else if (cl) {
    go(std::true_type{}, std::false_type{});
  } else if (cs) {
    go(std::false_type{}, std::true_type{});
  } else {
    go(std::false_type{}, std::false_type{});
  }
}

#define TIDE_V(x) decltype(x)::value

template <int WT, bool F32>
int launch_rs_w(const KernelArgs& a, int64_t grid, hipStream_t s) {
  by_instance(a, [&](auto CL, auto CS, auto ST, size_t lds) {
    hipLaunchKernelGGL((rs_local_kernel<WT, F32, TIDE_V(CL), TIDE_V(CS), TIDE_V(ST)>), dim3(unsigned(grid)),
                       dim3(unsigned(tide::kThreads)), lds, s, a.hdr, a.ptrs, a.chunk_begin, a.nsrc,
                       a.span, a.chunk, a.alpha, a.accumulate);
  });
  return int(hipGetLastError());
}

// The realigning instances exist with the default (non-temporal) cache
// policy only; the cache flags are hints and never change results.
template <int WT, bool F32>
int launch_rs_realign(const KernelArgs& a, int64_t grid, hipStream_t s) {
  bool staged;
  const size_t lds = staged_bytes(a, &staged);
  if (staged) {
    hipLaunchKernelGGL((rs_local_kernel<WT, F32, false, false, true>), dim3(unsigned(grid)),
                       dim3(unsigned(tide::kThreads)), lds, s, a.hdr, a.ptrs, a.chunk_begin, a.nsrc, a.span, a.chunk,
                       a.alpha, a.accumulate);
  } else {
    hipLaunchKernelGGL((rs_local_kernel<WT, F32, false, false, false>), dim3(unsigned(grid)),
                       dim3(unsigned(tide::kThreads)), 0, s, a.hdr, a.ptrs, a.chunk_begin, a.nsrc, a.span, a.chunk,
                       a.alpha, a.accumulate);
  }
  return int(hipGetLastError());
}

template <bool F32>
int launch_rs_t(const KernelArgs& a, int64_t grid, hipStream_t s) {
  if (a.realign) return launch_rs_realign<kAnyWShift, F32>(a, grid, s);
  switch (a.nsrc) {
    case 8: return launch_rs_w<8, F32>(a, grid, s);
    case 4: return launch_rs_w<4, F32>(a, grid, s);
    default:
      if constexpr (!F32) {
        if (a.nsrc <= 3 && a.chunk >= 2048) return launch_rs_w<kAnyTinyW, F32>(a, grid, s);
      }
      return launch_rs_w<kAnyW, F32>(a, grid, s);
  }
}

}  // namespace

namespace tide {

int launch_rs_local(const KernelArgs& a, bool f32, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return f32 ? launch_rs_t<true>(a, grid, s) : launch_rs_t<false>(a, grid, s);
}

int launch_ag_copyout(const KernelArgs& a, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  by_instance(a, [&](auto CL, auto CS, auto ST, size_t lds) {
    hipLaunchKernelGGL((ag_copyout_kernel<TIDE_V(CL), TIDE_V(CS), TIDE_V(ST)>), dim3(unsigned(grid)),
                       dim3(unsigned(kThreads)), lds, s, a.hdr, a.ptrs, a.chunk_begin, a.span, a.chunk);
  });
  return int(hipGetLastError());
}

int launch_ag_copyin(const KernelArgs& a, bool f32, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  by_instance(a, [&](auto CL, auto CS, auto ST, size_t lds) {
    if (f32) {
      hipLaunchKernelGGL((ag_copyin_kernel<true, TIDE_V(CL), TIDE_V(CS), TIDE_V(ST)>), dim3(unsigned(grid)),
                         dim3(unsigned(kThreads)), lds, s, a.hdr, a.ptrs, a.chunk_begin, a.span, a.chunk);
    } else {
      hipLaunchKernelGGL((ag_copyin_kernel<false, TIDE_V(CL), TIDE_V(CS), TIDE_V(ST)>), dim3(unsigned(grid)),
                         dim3(unsigned(kThreads)), lds, s, a.hdr, a.ptrs, a.chunk_begin, a.span, a.chunk);
    }
  });
  return int(hipGetLastError());
}

int launch_stock_pack(const KernelArgs& a, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  by_instance(a, [&](auto CL, auto CS, auto ST, size_t lds) {
    hipLaunchKernelGGL((stock_pack_kernel<TIDE_V(CL), TIDE_V(CS), TIDE_V(ST)>), dim3(unsigned(grid)),
                       dim3(unsigned(kThreads)), lds, s, a.hdr, a.ptrs, a.chunk_begin, a.span, a.chunk);
  });
  return int(hipGetLastError());
}

}  // namespace tide
