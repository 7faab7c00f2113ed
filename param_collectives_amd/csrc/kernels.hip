// Device code of the layout-aware FSDP2 collective local stages for MI355X
// (gfx950, CDNA4), after "The Endgame of FSDP Communication: Layout-Aware
// Collectives on Copy Engines, RDMA, and NVSwitch" (Wang et al.).
//
//   rs_local_kernel    reduce-scatter local stage (Section 4, Equation 5;
//                      Section 4.1 "Level 1: Node-Local Reduction"): W ranks'
//                      bf16 gradients -> W packed fp32 shards, summed in rank
//                      order in fp32 (Section 4.3), padding rows written +0.
//   ag_copyout_kernel  all-gather copy-out (Section 2.1): rank-major bf16
//                      buffer -> per-parameter tensors.
//   ag_copyin_kernel   all-gather copy-in (Sections 2.1, 3.1): every rank's
//                      local shards (fp32 cast to bf16, or bf16) -> the
//                      rank-major bf16 buffer, padding +0.
//
// Both are HBM-bandwidth bound: no MFMA, no atomics, no communication between
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
//   * Vector bodies use non-temporal 8-byte (reduce-scatter) or 16-byte
//     (copy-out) loads and contiguous 16-byte stores; heads and tails of
//     misaligned tensors take a scalar path.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "tide_internal.h"

namespace {

using tide::CallHdr;
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
__device__ __forceinline__ void store4(float* p, float v) { *(TIDE_GLOBAL float*)(p) = v; }

// bf16 is the upper half of binary32, so widening is a shift (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Values all lanes hold identically are moved to scalar registers.
__device__ __forceinline__ int32_t sgpr(int32_t v) { return int32_t(__builtin_amdgcn_readfirstlane(uint32_t(v))); }

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ int lane_id() { return int(threadIdx.x & 63); }

// ---------------------------------------------------------------------------
// Chunk dealing and segment lookup
// ---------------------------------------------------------------------------

// The chunk -> segment search table: first-chunk indices of all segments,
// staged in LDS when it fits (it is read by every chunk of every wave).
extern __shared__ int32_t s_chunk_begin[];

template <bool STAGED>
__device__ __forceinline__ const int32_t* chunk_table(const int32_t* __restrict__ chunk_begin, int32_t nseg) {
  if constexpr (STAGED) {
    for (int i = threadIdx.x; i <= nseg; i += tide::kThreads) s_chunk_begin[i] = chunk_begin[i];
    __syncthreads();
    return s_chunk_begin;
  } else {
    return chunk_begin;
  }
}

// The plan's read-only tables, passed as separate restrict-qualified kernel
// arguments so that their (wave-uniform) loads go through the scalar cache.
struct Tables {
  const CallHdr* __restrict__ hdr;
  const void* const* __restrict__ ptrs;
  int32_t nseg, nsrc, nchunks, chunk;
};

// Advance `cur` (wave-uniform, non-decreasing) to the segment holding chunk
// c: the largest s with chunk_begin[s] <= c.  64 candidates per step.
__device__ __forceinline__ int32_t seek(const int32_t* cb, int32_t nseg, int32_t cur, int32_t c) {
  while (true) {
    const int32_t idx = cur + 1 + lane_id();
    const int32_t v = idx <= nseg ? cb[idx] : INT_MAX;  // cb[nseg] = nchunks > c
    const int32_t k = __popcll(__ballot(v <= c));
    cur += k;
    if (k < 64) return sgpr(cur);
  }
}

// A wave's view of one chunk.
struct Chunk {
  int64_t lo, vlo, vhi, hi;  // scalar [lo, vlo), vector groups [vlo, vhi), scalar [vhi, hi)
  int32_t kind;
};

// Chunk j of a segment of `len` elements, `nch` chunks: chunk boundaries after
// the first sit at j*chunk + h, h being the segment's aligned-body start, so
// every chunk but the first starts on the vector body; the last chunk runs to
// the end.  Which wave handles which chunk never changes any result.
__device__ __forceinline__ Chunk chunk_range(const CallHdr& h, int64_t j, int64_t nch, int64_t chunk, int group) {
  const int64_t head = h.head > 0 ? h.head : 0;
  Chunk r;
  r.kind = h.kind;
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

// ---------------------------------------------------------------------------
// Reduce-scatter local stage
// ---------------------------------------------------------------------------

// Sum of the W sources at element e (scalar path), rank order 0..W-1.
__device__ __forceinline__ float sum_one(const uint16_t* const* src, int32_t W, int64_t e) {
  float acc = bf16_to_f32(load2(src[0] + e));
  for (int32_t u = 1; u < W; ++u) acc = acc + bf16_to_f32(load2(src[u] + e));
  return acc;
}

// acc = widen(v) and acc = acc + widen(v): one binary32 addition per element.
__device__ __forceinline__ void widen4(u32x2 v, float a[4]) {
  a[0] = bf16_lo(v.x);
  a[1] = bf16_hi(v.x);
  a[2] = bf16_lo(v.y);
  a[3] = bf16_hi(v.y);
}
__device__ __forceinline__ void add4(u32x2 v, float a[4]) {
  a[0] = a[0] + bf16_lo(v.x);
  a[1] = a[1] + bf16_hi(v.x);
  a[2] = a[2] + bf16_lo(v.y);
  a[3] = a[3] + bf16_hi(v.y);
}

// Vector body of a sum chunk: groups of 4 elements in [vlo, vhi); sources
// 8-byte aligned and the destination 16-byte aligned there.  Lane l handles
// groups l, l + 64, ... (two per step: 2W independent loads in flight).
// Groups each lane has in flight per step (measured on MI355X: two groups of
// W 8-byte loads for the reduce-scatter, four 16-byte loads for the copy).
constexpr int kRsUnroll = 2;

// Buffer-resource word 3 for raw (untyped) byte-addressed buffers on gfx9-class
// GPUs, and the cache-policy operand bit that marks an access non-temporal.
constexpr int kRawBuffer = 0x00020000;
constexpr int kPolicyNT = 2;
constexpr int kCoUnroll = 4;

template <int WT, bool CL, bool CS>
__device__ __forceinline__ void sum_body(const uint16_t* const* src, int32_t W, float* dst, int64_t vlo, int64_t vhi) {
  const int64_t ng = (vhi - vlo) >> 2;
  int64_t g = lane_id();
  if constexpr (WT > 0) {
    constexpr int U = kRsUnroll;
    const uint16_t* s[WT];
#pragma unroll
    for (int u = 0; u < WT; ++u) s[u] = src[u] + vlo;
    float* d = dst + vlo;
    // U groups per lane per step, U*WT independent loads in flight; the
    // remainder of a partial chunk goes one group per lane per step.
    int64_t base = 0;
    // Source loads go through buffer resources covering exactly this chunk's
    // body (scalar base, 32-bit lane offsets, hardware range check).
    __amdgpu_buffer_rsrc_t rs[WT];
#pragma unroll
    for (int u = 0; u < WT; ++u)
      rs[u] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(s[u]), 0, int((vhi - vlo) * 2), kRawBuffer);
    for (; base + 64 * U <= ng; base += 64 * U) {
      u32x2 v[U][WT];
#pragma unroll
      for (int k = 0; k < U; ++k) {
#pragma unroll
        for (int u = 0; u < WT; ++u)
          v[k][u] = __builtin_amdgcn_raw_buffer_load_b64(rs[u], int((base + g + 64 * k) * 8), 0, CL ? 0 : kPolicyNT);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float a[4];
        widen4(v[k][0], a);
#pragma unroll
        for (int u = 1; u < WT; ++u) add4(v[k][u], a);
        store<f32x4, CS>(d + (base + g + 64 * k) * 4, f32x4{a[0], a[1], a[2], a[3]});
      }
    }
    for (int64_t gk = base + g; gk < ng; gk += 64) {
      u32x2 v[WT];
#pragma unroll
      for (int u = 0; u < WT; ++u) v[u] = load<u32x2, CL>(s[u] + gk * 4);
      float a[4];
      widen4(v[0], a);
#pragma unroll
      for (int u = 1; u < WT; ++u) add4(v[u], a);
      store<f32x4, CS>(d + gk * 4, f32x4{a[0], a[1], a[2], a[3]});
    }
  } else {
    // Any W: sources in batches of 8, still added in rank order.
    for (; g < ng; g += 64) {
      const int64_t e = vlo + g * 4;
      float acc[4];
      widen4(load<u32x2, CL>(src[0] + e), acc);
      for (int32_t u0 = 1; u0 < W; u0 += 8) {
        const int32_t nb = (W - u0) < 8 ? (W - u0) : 8;
        u32x2 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nb) v[k] = load<u32x2, CL>(src[u0 + k] + e);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nb) add4(v[k], acc);
      }
      store<f32x4, CS>(dst + e, f32x4{acc[0], acc[1], acc[2], acc[3]});
    }
  }
}

template <bool CS>
__device__ __forceinline__ void zero_chunk(float* dst, const Chunk& c) {
  const int lane = lane_id();
  for (int64_t e = c.lo + lane; e < c.vlo; e += 64) store4(dst + e, 0.0f);
  for (int64_t e = c.vhi + lane; e < c.hi; e += 64) store4(dst + e, 0.0f);
  for (int64_t e = c.vlo + int64_t(lane) * 4; e < c.vhi; e += 256) store<f32x4, CS>(dst + e, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
}

// Segment descriptor of the chunk a wave is about to process (wave-uniform).
template <int WT>
struct RsDesc {
  CallHdr h;
  int32_t seg, j, nch;
  const uint16_t* src[WT > 0 ? WT : 1];
  float* dst;
};

template <int WT>
__device__ __forceinline__ void rs_fetch(const Tables& a, const int32_t* cb, int32_t* cur, int32_t c, RsDesc<WT>* d) {
  *cur = seek(cb, a.nseg, *cur, c);
  const int32_t s = *cur;
  const int32_t first = sgpr(cb[s]);
  d->seg = s;
  d->j = c - first;
  d->nch = sgpr(cb[s + 1]) - first;
  d->h = a.hdr[s];
  const void* const* row = a.ptrs + int64_t(s) * (a.nsrc + 1);
  if constexpr (WT > 0) {
#pragma unroll
    for (int u = 0; u < WT; ++u) d->src[u] = static_cast<const uint16_t*>(row[u]);
  }
  d->dst = static_cast<float*>(const_cast<void*>(row[a.nsrc]));
}

template <int WT, bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void rs_local_kernel(const CallHdr* __restrict__ hdr,
                                                                  const void* const* __restrict__ ptrs,
                                                                  const int32_t* __restrict__ chunk_begin,
                                                                  int32_t nseg, int32_t nsrc, int32_t nchunks,
                                                                  int32_t chunk) {
  const Tables a{hdr, ptrs, nseg, nsrc, nchunks, chunk};
  const int32_t* cb = chunk_table<STAGED>(chunk_begin, nseg);
  int32_t w, nw;
  wave_slot(&w, &nw);
  const int32_t W = WT > 0 ? WT : a.nsrc;
  int32_t cur = 0;
  int32_t c = w;
  RsDesc<WT> next;
  if (c < a.nchunks) rs_fetch<WT>(a, cb, &cur, c, &next);
  while (c < a.nchunks) {
    const RsDesc<WT> d = next;
    const int32_t cn = c + nw;
    if (cn < a.nchunks) rs_fetch<WT>(a, cb, &cur, cn, &next);  // overlaps the loads below
    if (d.h.kind == tide::kZero) {
      zero_chunk<CS>(d.dst, chunk_range(d.h, d.j, d.nch, a.chunk, 4));
    } else {
      const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 4);
      const uint16_t* const* src;
      if constexpr (WT > 0) {
        src = d.src;
      } else {
        // any W: the sources are read from the call table as needed
        src = reinterpret_cast<const uint16_t* const*>(a.ptrs + int64_t(d.seg) * (a.nsrc + 1));
      }
      const int lane = lane_id();
      for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store4(d.dst + e, sum_one(src, W, e));
      for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store4(d.dst + e, sum_one(src, W, e));
      if (r.vhi > r.vlo) sum_body<WT, CL, CS>(src, W, d.dst, r.vlo, r.vhi);
    }
    c = cn;
  }
}

// ---------------------------------------------------------------------------
// All-gather copy-out
// ---------------------------------------------------------------------------

struct CoDesc {
  CallHdr h;
  int32_t j, nch;
  const void* src;
  uint16_t* dst;
};

__device__ __forceinline__ void co_fetch(const Tables& a, const int32_t* cb, int32_t* cur, int32_t c, CoDesc* d) {
  *cur = seek(cb, a.nseg, *cur, c);
  const int32_t s = *cur;
  const int32_t first = sgpr(cb[s]);
  d->j = c - first;
  d->nch = sgpr(cb[s + 1]) - first;
  d->h = a.hdr[s];
  d->src = a.ptrs[2 * int64_t(s)];
  d->dst = static_cast<uint16_t*>(const_cast<void*>(a.ptrs[2 * int64_t(s) + 1]));
}

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

// bf16 words of [vlo, vhi) (groups of 8, both sides 16-byte aligned).
template <bool CL, bool CS>
__device__ __forceinline__ void copy_body(const uint16_t* src, uint16_t* dst, int64_t vlo, int64_t vhi) {
  const int lane = lane_id();
  const uint16_t* sv = src + vlo;
  uint16_t* dv = dst + vlo;
  const int64_t ng = (vhi - vlo) >> 3;
  // kCoUnroll 16-byte loads in flight per lane, then two, then one.
  int64_t base = 0;
  base = copy_steps<kCoUnroll, CL, CS>(sv, dv, base, ng, lane);
  base = copy_steps<2, CL, CS>(sv, dv, base, ng, lane);
  for (int64_t gk = base + lane; gk < ng; gk += 64) store<u32x4, CS>(dv + gk * 8, load<u32x4, CL>(sv + gk * 8));
}

template <bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void ag_copyout_kernel(const CallHdr* __restrict__ hdr,
                                                                    const void* const* __restrict__ ptrs,
                                                                    const int32_t* __restrict__ chunk_begin,
                                                                    int32_t nseg, int32_t nchunks, int32_t chunk) {
  const Tables a{hdr, ptrs, nseg, 1, nchunks, chunk};
  const int32_t* cb = chunk_table<STAGED>(chunk_begin, nseg);
  int32_t w, nw;
  wave_slot(&w, &nw);
  int32_t cur = 0;
  int32_t c = w;
  CoDesc next;
  if (c < a.nchunks) co_fetch(a, cb, &cur, c, &next);
  const int lane = lane_id();
  while (c < a.nchunks) {
    const CoDesc d = next;
    const int32_t cn = c + nw;
    if (cn < a.nchunks) co_fetch(a, cb, &cur, cn, &next);
    const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 8);
    const uint16_t* src = static_cast<const uint16_t*>(d.src);
    for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(d.dst + e, load2(src + e));
    for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(d.dst + e, load2(src + e));
    if (r.vhi > r.vlo) copy_body<CL, CS>(src, d.dst, r.vlo, r.vhi);
    c = cn;
  }
}

// ---------------------------------------------------------------------------
// All-gather copy-in
// ---------------------------------------------------------------------------

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

// fp32 [vlo, vhi) -> bf16 (groups of 4: 16-byte loads, 8-byte stores, each
// contiguous across the wave).
template <bool CL, bool CS>
__device__ __forceinline__ void cast_body(const float* src, uint16_t* dst, int64_t vlo, int64_t vhi) {
  const int lane = lane_id();
  const float* sv = src + vlo;
  uint16_t* dv = dst + vlo;
  const int64_t ng = (vhi - vlo) >> 2;
  int64_t base = 0;
  base = cast_steps<kCoUnroll, CL, CS>(sv, dv, base, ng, lane);
  base = cast_steps<2, CL, CS>(sv, dv, base, ng, lane);
  for (int64_t gk = base + lane; gk < ng; gk += 64)
    store<u32x2, CS>(dv + gk * 4, cast4(load<f32x4, CL>(sv + gk * 4)));
}

template <bool F32, bool CL, bool CS, bool STAGED>
__global__ __launch_bounds__(tide::kThreads) void ag_copyin_kernel(const CallHdr* __restrict__ hdr,
                                                                   const void* const* __restrict__ ptrs,
                                                                   const int32_t* __restrict__ chunk_begin,
                                                                   int32_t nseg, int32_t nchunks, int32_t chunk) {
  const Tables a{hdr, ptrs, nseg, 1, nchunks, chunk};
  const int32_t* cb = chunk_table<STAGED>(chunk_begin, nseg);
  int32_t w, nw;
  wave_slot(&w, &nw);
  int32_t cur = 0;
  int32_t c = w;
  CoDesc next;
  if (c < a.nchunks) co_fetch(a, cb, &cur, c, &next);
  const int lane = lane_id();
  while (c < a.nchunks) {
    const CoDesc d = next;
    const int32_t cn = c + nw;
    if (cn < a.nchunks) co_fetch(a, cb, &cur, cn, &next);
    if (d.h.kind == tide::kZero) {
      // padding of the rank-major slot: bf16 +0
      const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 8);
      for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(d.dst + e, 0);
      for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(d.dst + e, 0);
      for (int64_t e = r.vlo + int64_t(lane) * 8; e < r.vhi; e += 512) store<u32x4, CS>(d.dst + e, u32x4{0, 0, 0, 0});
    } else if constexpr (F32) {
      const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 4);
      const float* src = static_cast<const float*>(d.src);
      for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(d.dst + e, uint16_t(f32_to_bf16(load<float, true>(src + e))));
      for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(d.dst + e, uint16_t(f32_to_bf16(load<float, true>(src + e))));
      if (r.vhi > r.vlo) cast_body<CL, CS>(src, d.dst, r.vlo, r.vhi);
    } else {
      const Chunk r = chunk_range(d.h, d.j, d.nch, a.chunk, 8);
      const uint16_t* src = static_cast<const uint16_t*>(d.src);
      for (int64_t e = r.lo + lane; e < r.vlo; e += 64) store2(d.dst + e, load2(src + e));
      for (int64_t e = r.vhi + lane; e < r.hi; e += 64) store2(d.dst + e, load2(src + e));
      if (r.vhi > r.vlo) copy_body<CL, CS>(src, d.dst, r.vlo, r.vhi);
    }
    c = cn;
  }
}

size_t staged_bytes(const KernelArgs& a, bool* staged) {
  *staged = a.nseg <= tide::kMaxStagedSegs;
  return *staged ? size_t(a.nseg + 1) * sizeof(int32_t) : 0;
}

template <int WT>
int launch_rs_w(const KernelArgs& a, int64_t grid, hipStream_t stream) {
  bool staged;
  const size_t lds = staged_bytes(a, &staged);
  const bool cl = a.flags & TIDE_FLAG_CACHED_LOADS, cs = a.flags & TIDE_FLAG_CACHED_STORES;
  const dim3 g{unsigned(grid), 1, 1}, b{unsigned(tide::kThreads), 1, 1};
#define TIDE_RS(CL, CS)                                                                   \
  do {                                                                                     \
    if (staged)                                                                            \
      hipLaunchKernelGGL((rs_local_kernel<WT, CL, CS, true>), g, b, lds, stream, a.hdr, a.ptrs, \
                         a.chunk_begin, a.nseg, a.nsrc, a.nchunks, a.chunk);                \
    else                                                                                   \
      hipLaunchKernelGGL((rs_local_kernel<WT, CL, CS, false>), g, b, 0, stream, a.hdr, a.ptrs, \
                         a.chunk_begin, a.nseg, a.nsrc, a.nchunks, a.chunk);                \
  } while (0)
  if (cl && cs) {
    TIDE_RS(true, true);
  } else if (cl) {
    TIDE_RS(true, false);
  } else if (cs) {
    TIDE_RS(false, true);
  } else {
    TIDE_RS(false, false);
  }
#undef TIDE_RS
  return int(hipGetLastError());
}

}  // namespace

namespace tide {

int launch_rs_local(const KernelArgs& a, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.nsrc) {
    case 8: return launch_rs_w<8>(a, grid, s);
    case 4: return launch_rs_w<4>(a, grid, s);
    case 2: return launch_rs_w<2>(a, grid, s);
    default: return launch_rs_w<0>(a, grid, s);
  }
}

int launch_ag_copyout(const KernelArgs& a, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool staged;
  const size_t lds = staged_bytes(a, &staged);
  const bool cl = a.flags & TIDE_FLAG_CACHED_LOADS, cs = a.flags & TIDE_FLAG_CACHED_STORES;
  const dim3 g{unsigned(grid), 1, 1}, b{unsigned(kThreads), 1, 1};
#define TIDE_CO(CL, CS)                                                                    \
  do {                                                                                      \
    if (staged)                                                                             \
      hipLaunchKernelGGL((ag_copyout_kernel<CL, CS, true>), g, b, lds, s, a.hdr, a.ptrs,     \
                         a.chunk_begin, a.nseg, a.nchunks, a.chunk);                        \
    else                                                                                    \
      hipLaunchKernelGGL((ag_copyout_kernel<CL, CS, false>), g, b, 0, s, a.hdr, a.ptrs,      \
                         a.chunk_begin, a.nseg, a.nchunks, a.chunk);                        \
  } while (0)
  if (cl && cs) {
    TIDE_CO(true, true);
  } else if (cl) {
    TIDE_CO(true, false);
  } else if (cs) {
    TIDE_CO(false, true);
  } else {
    TIDE_CO(false, false);
  }
#undef TIDE_CO
  return int(hipGetLastError());
}

int launch_ag_copyin(const KernelArgs& a, bool f32, int64_t grid, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool staged;
  const size_t lds = staged_bytes(a, &staged);
  const bool cl = a.flags & TIDE_FLAG_CACHED_LOADS, cs = a.flags & TIDE_FLAG_CACHED_STORES;
  const dim3 g{unsigned(grid), 1, 1}, b{unsigned(kThreads), 1, 1};
#define TIDE_CI(F, CL, CS)                                                                       \
  do {                                                                                            \
    if (staged)                                                                                   \
      hipLaunchKernelGGL((ag_copyin_kernel<F, CL, CS, true>), g, b, lds, s, a.hdr, a.ptrs,        \
                         a.chunk_begin, a.nseg, a.nchunks, a.chunk);                              \
    else                                                                                          \
      hipLaunchKernelGGL((ag_copyin_kernel<F, CL, CS, false>), g, b, 0, s, a.hdr, a.ptrs,         \
                         a.chunk_begin, a.nseg, a.nchunks, a.chunk);                              \
  } while (0)
#define TIDE_CI_F(F)              \
  do {                            \
    if (cl && cs) {               \
      TIDE_CI(F, true, true);     \
    } else if (cl) {              \
      TIDE_CI(F, true, false);    \
    } else if (cs) {              \
      TIDE_CI(F, false, true);    \
    } else {                      \
      TIDE_CI(F, false, false);   \
    }                             \
  } while (0)
  if (f32) {
    TIDE_CI_F(true);
  } else {
    TIDE_CI_F(false);
  }
#undef TIDE_CI_F
#undef TIDE_CI
  return int(hipGetLastError());
}

}  // namespace tide
