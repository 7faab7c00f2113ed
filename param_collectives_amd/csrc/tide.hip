// HIP kernels and C ABI for the layout-aware FSDP2 collective local stages on
// MI355X (gfx950, CDNA4), after "The Endgame of FSDP Communication:
// Layout-Aware Collectives on Copy Engines, RDMA, and NVSwitch" (Wang et al.).
//
//   rs_local_kernel    reduce-scatter local stage (Section 4, Equation 5;
//                      Section 4.1 "Level 1: Node-Local Reduction"): W ranks'
//                      bf16 gradients -> W packed fp32 shards, summed in rank
//                      order in fp32 (Section 4.3), padding rows written +0.
//   ag_copyout_kernel  all-gather copy-out (Section 2.1): rank-major bf16
//                      buffer -> per-parameter tensors.
//
// Both kernels are HBM-bandwidth bound (no MFMA, no atomics, no cross-
// workgroup communication).  Structure shared by both:
//   * a persistent grid of cu_budget * wg_per_cu workgroups; workgroup b owns
//     a contiguous, balanced range of fixed-size chunks of the plan's segment
//     table (each output element has exactly one writer);
//   * the segment descriptors of the range (and, for the reduce-scatter, the W
//     source pointers of each) are staged in LDS in batches, and the
//     per-segment alignment phase is resolved there once;
//   * 16-byte global loads and stores on the aligned body of each segment
//     (8 bf16 in, 8 fp32 or 8 bf16 out per lane and group), with scalar
//     heads and tails where a tensor does not start on a 16-byte boundary;
//   * optional non-temporal hints for streaming loads and stores.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "tide_internal.h"

namespace {

using tide::Seg;
using tide::kThreads;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStage = 16;      // segment descriptors staged per batch
constexpr int kPtrSlots = 256;  // LDS source-pointer slots per batch (>= TIDE_MAX_WORLD)
static_assert(kPtrSlots >= TIDE_MAX_WORLD, "one segment's sources must fit a batch");

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// All tensors live in global memory; saying so (address space 1) lets the
// compiler emit global_load/global_store instead of flat accesses.
#define TIDE_GLOBAL __attribute__((address_space(1)))

template <bool NT>
__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  const TIDE_GLOBAL u32x4* q = (const TIDE_GLOBAL u32x4*)(p);
  if constexpr (NT) {
    return __builtin_nontemporal_load(q);
  } else {
    return *q;
  }
}

template <bool NT>
__device__ __forceinline__ void store16(float* p, f32x4 v) {
  TIDE_GLOBAL f32x4* q = (TIDE_GLOBAL f32x4*)(p);
  if constexpr (NT) {
    __builtin_nontemporal_store(v, q);
  } else {
    *q = v;
  }
}

template <bool NT>
__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) {
  TIDE_GLOBAL u32x4* q = (TIDE_GLOBAL u32x4*)(p);
  if constexpr (NT) {
    __builtin_nontemporal_store(v, q);
  } else {
    *q = v;
  }
}

__device__ __forceinline__ uint16_t load2(const uint16_t* p) { return *(const TIDE_GLOBAL uint16_t*)(p); }
__device__ __forceinline__ void store2(uint16_t* p, uint16_t v) { *(TIDE_GLOBAL uint16_t*)(p) = v; }
__device__ __forceinline__ void store4(float* p, float v) { *(TIDE_GLOBAL float*)(p) = v; }

// bf16 is the upper half of binary32, so widening is a shift (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void widen8(u32x4 v, float a[8]) {
  a[0] = bf16_lo(v.x);
  a[1] = bf16_hi(v.x);
  a[2] = bf16_lo(v.y);
  a[3] = bf16_hi(v.y);
  a[4] = bf16_lo(v.z);
  a[5] = bf16_hi(v.z);
  a[6] = bf16_lo(v.w);
  a[7] = bf16_hi(v.w);
}

// acc[i] = acc[i] + widen(v)[i]: one binary32 addition per element.
__device__ __forceinline__ void add8(u32x4 v, float a[8]) {
  a[0] = a[0] + bf16_lo(v.x);
  a[1] = a[1] + bf16_hi(v.x);
  a[2] = a[2] + bf16_lo(v.y);
  a[3] = a[3] + bf16_hi(v.y);
  a[4] = a[4] + bf16_lo(v.z);
  a[5] = a[5] + bf16_hi(v.z);
  a[6] = a[6] + bf16_lo(v.w);
  a[7] = a[7] + bf16_hi(v.w);
}

// Values every lane of the wave holds identically (read from LDS) are moved
// to scalar registers, so loads use a scalar base plus a lane offset.
template <typename T>
__device__ __forceinline__ T* uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<T*>((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// A segment descriptor as staged in LDS.
struct Staged {
  int64_t len;          // elements
  int64_t chunk_begin;  // first chunk of the segment
  int64_t nchunks;      // ceil(len / chunk)
  void* dst;            // destination at the segment's element 0
  const uint16_t* src;  // copy-out: source at element 0 (reduce-scatter: unused)
  int32_t kind;
  int32_t head;         // elements before the first 16-byte-aligned group; -1 = no aligned body
};

// Chunk j of a segment covers [lo, hi).  Chunk boundaries after the first sit
// at j*chunk + h, so that every chunk but the first starts on the aligned
// body; the last chunk runs to the end of the segment.  The split depends on
// the launch knobs only through which workgroup does which element.
struct Range {
  int64_t lo, vlo, vhi, hi;  // scalar [lo, vlo), vector groups [vlo, vhi), scalar [vhi, hi)
};

__device__ __forceinline__ Range chunk_range(const Staged& s, int64_t j, int64_t chunk, int group) {
  const int64_t h = s.head > 0 ? s.head : 0;
  Range r;
  r.lo = (j == 0) ? 0 : min64(s.len, j * chunk + h);
  r.hi = (j == s.nchunks - 1) ? s.len : min64(s.len, (j + 1) * chunk + h);
  if (s.head < 0) {
    r.vlo = r.vhi = r.hi;
  } else {
    r.vlo = (j == 0) ? min64(h, r.hi) : r.lo;
    r.vhi = r.vlo + ((r.hi - r.vlo) / group) * group;
  }
  return r;
}

// Largest s with segs[s].chunk_begin <= c (segs[0].chunk_begin is 0).
__device__ __forceinline__ int32_t find_segment(const Seg* __restrict__ segs, int32_t nseg, int64_t c) {
  int32_t lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (segs[mid].chunk_begin <= c) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  return lo;
}

// Balanced contiguous split of nchunks over the grid (no 64-bit overflow).
__device__ __forceinline__ void block_range(int64_t nchunks, int64_t* c0, int64_t* c1) {
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t q = nchunks / G, rem = nchunks % G;
  *c0 = b * q + (b < rem ? b : rem);
  *c1 = *c0 + q + (b < rem ? 1 : 0);
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

template <bool NTS>
__device__ __forceinline__ void store8(float* d, const float a[8]) {
  store16<NTS>(d, f32x4{a[0], a[1], a[2], a[3]});
  store16<NTS>(d + 4, f32x4{a[4], a[5], a[6], a[7]});
}

// Groups of 8 elements in [a, b) (b - a a multiple of 8, all 16-byte aligned).
template <int WT, bool NTL, bool NTS>
__device__ __forceinline__ void sum_groups(const uint16_t* const* src, int32_t W, float* dst, int64_t a, int64_t b) {
  const int64_t ng = (b - a) >> 3;
  if constexpr (WT > 0) {
    const uint16_t* s[WT];
#pragma unroll
    for (int u = 0; u < WT; ++u) s[u] = uniform(src[u] + a);
    float* d = uniform(dst + a);
    int64_t g = threadIdx.x;
    // Two groups per lane per step: 2*WT independent 16-byte loads in flight.
    for (; g + kThreads < ng; g += 2 * kThreads) {
      u32x4 v0[WT], v1[WT];
#pragma unroll
      for (int u = 0; u < WT; ++u) v0[u] = load16<NTL>(s[u] + g * 8);
#pragma unroll
      for (int u = 0; u < WT; ++u) v1[u] = load16<NTL>(s[u] + (g + kThreads) * 8);
      float a0[8], a1[8];
      widen8(v0[0], a0);
      widen8(v1[0], a1);
#pragma unroll
      for (int u = 1; u < WT; ++u) {
        add8(v0[u], a0);
        add8(v1[u], a1);
      }
      store8<NTS>(d + g * 8, a0);
      store8<NTS>(d + (g + kThreads) * 8, a1);
    }
    if (g < ng) {
      u32x4 v0[WT];
#pragma unroll
      for (int u = 0; u < WT; ++u) v0[u] = load16<NTL>(s[u] + g * 8);
      float a0[8];
      widen8(v0[0], a0);
#pragma unroll
      for (int u = 1; u < WT; ++u) add8(v0[u], a0);
      store8<NTS>(d + g * 8, a0);
    }
  } else {
    // Any W: sources in batches of 8, still added in rank order.
    for (int64_t g = threadIdx.x; g < ng; g += kThreads) {
      const int64_t e = a + g * 8;
      float acc[8];
      widen8(load16<NTL>(src[0] + e), acc);
      for (int32_t u0 = 1; u0 < W; u0 += 8) {
        const int32_t nb = (W - u0) < 8 ? (W - u0) : 8;
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nb) v[k] = load16<NTL>(src[u0 + k] + e);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < nb) add8(v[k], acc);
      }
      store8<NTS>(dst + e, acc);
    }
  }
}

template <int WT, bool NTL, bool NTS>
__device__ __forceinline__ void rs_chunk(const Staged& s, const uint16_t* const* src, int32_t W, int64_t j,
                                         int64_t chunk) {
  float* dst = static_cast<float*>(s.dst);
  if (s.kind == tide::kZero) {
    // Padding rows: +0.0f (rows past D_p are zero).
    const Range r = chunk_range(s, j, chunk, 4);
    for (int64_t e = r.lo + threadIdx.x; e < r.vlo; e += kThreads) store4(dst + e, 0.0f);
    for (int64_t e = r.vhi + threadIdx.x; e < r.hi; e += kThreads) store4(dst + e, 0.0f);
    for (int64_t e = r.vlo + int64_t(threadIdx.x) * 4; e < r.vhi; e += int64_t(kThreads) * 4)
      store16<NTS>(dst + e, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    return;
  }
  const Range r = chunk_range(s, j, chunk, 8);
  for (int64_t e = r.lo + threadIdx.x; e < r.vlo; e += kThreads) store4(dst + e, sum_one(src, W, e));
  for (int64_t e = r.vhi + threadIdx.x; e < r.hi; e += kThreads) store4(dst + e, sum_one(src, W, e));
  if (r.vhi > r.vlo) sum_groups<WT, NTL, NTS>(src, W, dst, r.vlo, r.vhi);
}

template <int WT, bool NTL, bool NTS>
__global__ __launch_bounds__(kThreads) void rs_local_kernel(const Seg* __restrict__ segs, int32_t nseg,
                                                            int64_t nchunks, int64_t chunk,
                                                            const uint16_t* const* __restrict__ grads,
                                                            float* const* __restrict__ outs, int32_t world,
                                                            int32_t nparams) {
  const int32_t W = WT > 0 ? WT : world;
  __shared__ Staged st[kStage];
  __shared__ const uint16_t* sp[kPtrSlots];

  int64_t c, cend;
  block_range(nchunks, &c, &cend);
  if (c >= cend) return;
  const int32_t per_batch = (kPtrSlots / W) < kStage ? (kPtrSlots / W) : kStage;
  int32_t s = find_segment(segs, nseg, c);
  while (c < cend) {
    const int32_t nb = (nseg - s) < per_batch ? (nseg - s) : per_batch;
    __syncthreads();  // the previous batch is no longer read
    for (int t = threadIdx.x; t < nb * W; t += kThreads) {
      const int32_t k = t / W, u = t - k * W;
      const Seg& g = segs[s + k];
      sp[k * W + u] = (g.kind == tide::kSum) ? grads[int64_t(u) * nparams + g.src_idx] + g.src_off : nullptr;
    }
    for (int k = threadIdx.x; k < nb; k += kThreads) {
      const Seg g = segs[s + k];
      st[k].len = g.len;
      st[k].chunk_begin = g.chunk_begin;
      st[k].nchunks = (g.len + chunk - 1) / chunk;
      st[k].dst = outs[g.dst_idx] + g.dst_off;
      st[k].src = nullptr;
      st[k].kind = g.kind;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < nb; k += kThreads) {
      const uintptr_t pd = reinterpret_cast<uintptr_t>(st[k].dst) & 15;
      int32_t head;
      if (st[k].kind == tide::kZero) {
        head = int32_t(((16 - pd) & 15) / 4);
      } else {
        // A vector body needs every source and the destination 16-byte
        // aligned at the same element.
        const uintptr_t ps = reinterpret_cast<uintptr_t>(sp[k * W]) & 15;
        bool same = true;
        for (int32_t u = 1; u < W; ++u) same = same && ((reinterpret_cast<uintptr_t>(sp[k * W + u]) & 15) == ps);
        head = int32_t(((16 - ps) & 15) / 2);
        if (!same || ((pd + 4 * uintptr_t(head)) & 15) != 0) head = -1;
      }
      st[k].head = head;
    }
    __syncthreads();
    for (int32_t k = 0; k < nb && c < cend; ++k) {
      const int64_t cb = st[k].chunk_begin;
      const int64_t stop = min64(cend, cb + st[k].nchunks);
      for (; c < stop; ++c) rs_chunk<WT, NTL, NTS>(st[k], &sp[k * W], W, c - cb, chunk);
    }
    s += nb;
  }
}

// ---------------------------------------------------------------------------
// All-gather copy-out
// ---------------------------------------------------------------------------

template <bool NTL, bool NTS>
__device__ __forceinline__ void copy_chunk(const Staged& s, int64_t j, int64_t chunk) {
  const uint16_t* src = s.src;
  uint16_t* dst = static_cast<uint16_t*>(s.dst);
  const Range r = chunk_range(s, j, chunk, 8);
  for (int64_t e = r.lo + threadIdx.x; e < r.vlo; e += kThreads) store2(dst + e, load2(src + e));
  for (int64_t e = r.vhi + threadIdx.x; e < r.hi; e += kThreads) store2(dst + e, load2(src + e));
  if (r.vhi <= r.vlo) return;
  const uint16_t* sv = uniform(src + r.vlo);
  uint16_t* dv = uniform(dst + r.vlo);
  const int64_t ng = (r.vhi - r.vlo) >> 3;
  int64_t g = threadIdx.x;
  // Four 16-byte loads in flight per lane.
  for (; g + 3 * kThreads < ng; g += 4 * kThreads) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = load16<NTL>(sv + (g + k * kThreads) * 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) store16<NTS>(dv + (g + k * kThreads) * 8, v[k]);
  }
  for (; g < ng; g += kThreads) store16<NTS>(dv + g * 8, load16<NTL>(sv + g * 8));
}

template <bool NTL, bool NTS>
__global__ __launch_bounds__(kThreads) void ag_copyout_kernel(const Seg* __restrict__ segs, int32_t nseg,
                                                              int64_t nchunks, int64_t chunk,
                                                              const uint16_t* __restrict__ rank_major,
                                                              uint16_t* const* __restrict__ params) {
  __shared__ Staged st[kStage];
  int64_t c, cend;
  block_range(nchunks, &c, &cend);
  if (c >= cend) return;
  int32_t s = find_segment(segs, nseg, c);
  while (c < cend) {
    const int32_t nb = (nseg - s) < kStage ? (nseg - s) : kStage;
    __syncthreads();
    for (int k = threadIdx.x; k < nb; k += kThreads) {
      const Seg g = segs[s + k];
      const uint16_t* src = rank_major + g.src_off;
      uint16_t* dst = params[g.dst_idx] + g.dst_off;
      const uintptr_t ps = reinterpret_cast<uintptr_t>(src) & 15;
      const uintptr_t pd = reinterpret_cast<uintptr_t>(dst) & 15;
      st[k].len = g.len;
      st[k].chunk_begin = g.chunk_begin;
      st[k].nchunks = (g.len + chunk - 1) / chunk;
      st[k].dst = dst;
      st[k].src = src;
      st[k].kind = g.kind;
      st[k].head = (ps == pd) ? int32_t(((16 - ps) & 15) / 2) : -1;
    }
    __syncthreads();
    for (int32_t k = 0; k < nb && c < cend; ++k) {
      const int64_t cb = st[k].chunk_begin;
      const int64_t stop = min64(cend, cb + st[k].nchunks);
      for (; c < stop; ++c) copy_chunk<NTL, NTS>(st[k], c - cb, chunk);
    }
    s += nb;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

thread_local std::string g_last_error;

tide_status fail(tide_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

tide_status hip_fail(hipError_t e, const char* what) {
  return fail(TIDE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// One host->device upload channel: a pinned staging buffer whose previous
// copy must have finished before it is rewritten.
struct Upload {
  void* host = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};

}  // namespace

struct tide_plan {
  uint64_t magic = 0;
  tide::Geometry geo;
  tide_options opt{};
  std::vector<Seg> rs, co;
  int64_t rs_chunks = 0, co_chunks = 0;
  // device binding (made by the first reduce-scatter or copy-out call)
  int device = -1;
  int cu_count = 0;
  Seg* d_rs = nullptr;
  Seg* d_co = nullptr;
  void** d_rs_ptrs = nullptr;  // [W*P grads | W outs]
  void** d_co_ptrs = nullptr;  // [P params]
  bool rs_segs_stale = true, co_segs_stale = true;
  std::vector<void*> rs_ptrs, co_ptrs;  // last uploaded pointer tables
  bool rs_ptrs_valid = false, co_ptrs_valid = false;
  Upload up_rs_segs, up_co_segs, up_rs_ptrs, up_co_ptrs;
};

namespace {

constexpr uint64_t kMagic = 0x7469646570616e31ull;
std::mutex g_plans_mu;
std::unordered_set<const tide_plan*> g_plans;

bool live(const tide_plan* p) {
  if (p == nullptr) return false;
  std::lock_guard<std::mutex> lock(g_plans_mu);
  return g_plans.count(p) != 0 && p->magic == kMagic;
}

tide_status rebuild_chunks(tide_plan* p) {
  p->rs_chunks = tide::assign_chunks(&p->rs, p->opt.chunk_elems);
  p->co_chunks = tide::assign_chunks(&p->co, p->opt.chunk_elems);
  p->rs_segs_stale = p->co_segs_stale = true;
  return TIDE_OK;
}

tide_status make_upload(Upload* u, size_t bytes) {
  u->bytes = bytes;
  if (bytes == 0) return TIDE_OK;
  hipError_t e = hipHostMalloc(&u->host, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    u->host = nullptr;
    return fail(TIDE_ERR_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  }
  e = hipEventCreateWithFlags(&u->done, hipEventDisableTiming);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  return TIDE_OK;
}

void free_upload(Upload* u) {
  if (u->done) {
    if (u->pending) (void)hipEventSynchronize(u->done);
    (void)hipEventDestroy(u->done);
  }
  if (u->host) (void)hipHostFree(u->host);
  *u = Upload{};
}

tide_status upload(Upload* u, void* dev, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return TIDE_OK;
  if (u->pending) {
    hipError_t e = hipEventSynchronize(u->done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    u->pending = false;
  }
  std::memcpy(u->host, src, bytes);
  hipError_t e = hipMemcpyAsync(dev, u->host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipEventRecord(u->done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  u->pending = true;
  return TIDE_OK;
}

void release_device(tide_plan* p) {
  if (p->device < 0) return;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(p->device);
  free_upload(&p->up_rs_segs);
  free_upload(&p->up_co_segs);
  free_upload(&p->up_rs_ptrs);
  free_upload(&p->up_co_ptrs);
  if (p->d_rs) (void)hipFree(p->d_rs);
  if (p->d_co) (void)hipFree(p->d_co);
  if (p->d_rs_ptrs) (void)hipFree(p->d_rs_ptrs);
  if (p->d_co_ptrs) (void)hipFree(p->d_co_ptrs);
  p->d_rs = p->d_co = nullptr;
  p->d_rs_ptrs = p->d_co_ptrs = nullptr;
  p->device = -1;
  if (prev >= 0) (void)hipSetDevice(prev);
}

template <typename T>
tide_status dev_alloc(T** out, size_t bytes) {
  *out = nullptr;
  if (bytes == 0) return TIDE_OK;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(out), bytes);
  if (e != hipSuccess) {
    *out = nullptr;
    return fail(TIDE_ERR_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
  }
  return TIDE_OK;
}

// Bind the plan to the current device on first use.
tide_status bind_device(tide_plan* p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->device >= 0) {
    if (dev != p->device)
      return fail(TIDE_ERR_INVALID, "plan is bound to device " + std::to_string(p->device) +
                                        " but device " + std::to_string(dev) + " is current");
    return TIDE_OK;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  p->device = dev;
  p->cu_count = cus;
  const int64_t W = p->geo.world, P = p->geo.nparams;
  tide_status st;
  if ((st = dev_alloc(&p->d_rs, p->rs.size() * sizeof(Seg))) != TIDE_OK ||
      (st = dev_alloc(&p->d_co, p->co.size() * sizeof(Seg))) != TIDE_OK ||
      (st = dev_alloc(&p->d_rs_ptrs, size_t(W * P + W) * sizeof(void*))) != TIDE_OK ||
      (st = dev_alloc(&p->d_co_ptrs, size_t(P) * sizeof(void*))) != TIDE_OK ||
      (st = make_upload(&p->up_rs_segs, p->rs.size() * sizeof(Seg))) != TIDE_OK ||
      (st = make_upload(&p->up_co_segs, p->co.size() * sizeof(Seg))) != TIDE_OK ||
      (st = make_upload(&p->up_rs_ptrs, size_t(W * P + W) * sizeof(void*))) != TIDE_OK ||
      (st = make_upload(&p->up_co_ptrs, size_t(P) * sizeof(void*))) != TIDE_OK) {
    const std::string why = g_last_error;
    release_device(p);
    return fail(st, why);
  }
  p->rs_segs_stale = p->co_segs_stale = true;
  p->rs_ptrs_valid = p->co_ptrs_valid = false;
  return TIDE_OK;
}

int64_t grid_for(const tide_plan* p, int64_t nchunks) {
  const int64_t budget = p->opt.cu_budget > 0 ? p->opt.cu_budget : p->cu_count;
  int64_t grid = budget * p->opt.wg_per_cu;
  if (grid > nchunks) grid = nchunks;
  if (grid < 1) grid = 1;
  return grid;
}

template <int WT>
void launch_rs(const tide_plan* p, int64_t grid, hipStream_t stream, void* const* ptrs) {
  const uint16_t* const* grads = reinterpret_cast<const uint16_t* const*>(ptrs);
  float* const* outs = reinterpret_cast<float* const*>(ptrs + int64_t(p->geo.world) * p->geo.nparams);
  const int32_t nseg = int32_t(p->rs.size());
  const bool ntl = p->opt.flags & TIDE_FLAG_NT_LOADS, nts = p->opt.flags & TIDE_FLAG_NT_STORES;
#define TIDE_RS_LAUNCH(L, S)                                                                              \
  hipLaunchKernelGGL((rs_local_kernel<WT, L, S>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p->d_rs, \
                     nseg, p->rs_chunks, p->opt.chunk_elems, grads, outs, p->geo.world, p->geo.nparams)
  if (ntl && nts) {
    TIDE_RS_LAUNCH(true, true);
  } else if (ntl) {
    TIDE_RS_LAUNCH(true, false);
  } else if (nts) {
    TIDE_RS_LAUNCH(false, true);
  } else {
    TIDE_RS_LAUNCH(false, false);
  }
#undef TIDE_RS_LAUNCH
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

tide_status tide_plan_create(int32_t world, int32_t nparams, const int32_t* ndims, const int64_t* dims,
                             const tide_options* opt, tide_plan** out_plan) {
  g_last_error.clear();
  if (out_plan == nullptr) return fail(TIDE_ERR_INVALID, "out_plan must not be NULL");
  *out_plan = nullptr;
  std::string why;
  tide_options resolved;
  tide_status st = tide::resolve_options(opt, &resolved, &why);
  if (st != TIDE_OK) return fail(st, why);
  tide_plan* p = new (std::nothrow) tide_plan();
  if (p == nullptr) return fail(TIDE_ERR_NOMEM, "out of host memory");
  st = tide::build_geometry(world, nparams, ndims, dims, &p->geo, &why);
  if (st != TIDE_OK) {
    delete p;
    return fail(st, why);
  }
  try {
    p->rs = tide::rs_segments(p->geo);
    p->co = tide::copyout_segments(p->geo);
  } catch (...) {
    delete p;
    return fail(TIDE_ERR_NOMEM, "out of host memory");
  }
  if (p->rs.size() > size_t(INT32_MAX) || p->co.size() > size_t(INT32_MAX)) {
    delete p;
    return fail(TIDE_ERR_RANGE, "too many segments");
  }
  p->opt = resolved;
  rebuild_chunks(p);
  p->magic = kMagic;
  {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    g_plans.insert(p);
  }
  *out_plan = p;
  return TIDE_OK;
}

tide_status tide_plan_layout(const tide_plan* plan, int64_t* rows_per_rank, int64_t* shard_offset,
                             int64_t* shard_elems) {
  g_last_error.clear();
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  for (int32_t p = 0; p < plan->geo.nparams; ++p) {
    if (rows_per_rank) rows_per_rank[p] = plan->geo.R[p];
    if (shard_offset) shard_offset[p] = plan->geo.o[p];
  }
  if (shard_elems) *shard_elems = plan->geo.S;
  return TIDE_OK;
}

tide_status tide_plan_segments(const tide_plan* plan, int32_t op, int64_t* table, int64_t capacity,
                               int64_t* count) {
  g_last_error.clear();
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  if (op != 0 && op != 1) return fail(TIDE_ERR_INVALID, "op must be 0 (reduce-scatter) or 1 (copy-out)");
  if (count == nullptr || capacity < 0 || (capacity > 0 && table == nullptr))
    return fail(TIDE_ERR_INVALID, "bad table/capacity/count");
  const std::vector<Seg>& segs = op == 0 ? plan->rs : plan->co;
  *count = int64_t(segs.size());
  const int64_t n = capacity < *count ? capacity : *count;
  for (int64_t i = 0; i < n; ++i) {
    const Seg& s = segs[size_t(i)];
    int64_t* row = table + 6 * i;
    row[0] = s.kind;
    row[1] = s.src_idx;
    row[2] = s.dst_idx;
    row[3] = s.src_off;
    row[4] = s.dst_off;
    row[5] = s.len;
  }
  return TIDE_OK;
}

tide_status tide_plan_set_options(tide_plan* plan, const tide_options* opt) {
  g_last_error.clear();
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  std::string why;
  tide_options resolved;
  tide_status st = tide::resolve_options(opt, &resolved, &why);
  if (st != TIDE_OK) return fail(st, why);
  const bool rechunk = resolved.chunk_elems != plan->opt.chunk_elems;
  plan->opt = resolved;
  if (rechunk) rebuild_chunks(plan);
  return TIDE_OK;
}

tide_status tide_plan_get_options(const tide_plan* plan, tide_options* out) {
  g_last_error.clear();
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  if (out == nullptr) return fail(TIDE_ERR_INVALID, "out must not be NULL");
  *out = plan->opt;
  if (out->cu_budget == 0) out->cu_budget = plan->cu_count;
  return TIDE_OK;
}

tide_status tide_reduce_scatter_local(tide_plan* plan, const uint16_t* const* grads, float* const* out,
                                      float alpha, int32_t accumulate, void* stream_) {
  g_last_error.clear();
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  if (grads == nullptr || out == nullptr) return fail(TIDE_ERR_INVALID, "grads and out must not be NULL");
  if (!(alpha == 1.0f) || accumulate != 0)
    return fail(TIDE_ERR_UNSUPPORTED, "only alpha = 1 and accumulate = 0 are provided");
  const tide::Geometry& g = plan->geo;
  const int64_t W = g.world, P = g.nparams;
  for (int64_t u = 0; u < W; ++u) {
    for (int64_t p = 0; p < P; ++p) {
      const uint16_t* ptr = grads[u * P + p];
      if (g.D[p] * g.K[p] == 0) continue;
      if (ptr == nullptr)
        return fail(TIDE_ERR_INVALID, "grads[" + std::to_string(u * P + p) + "] is NULL");
      if (reinterpret_cast<uintptr_t>(ptr) & 1)
        return fail(TIDE_ERR_ALIGN, "grads[" + std::to_string(u * P + p) + "] is not 2-byte aligned");
    }
  }
  for (int64_t r = 0; r < W; ++r) {
    if (g.S == 0) continue;
    if (out[r] == nullptr) return fail(TIDE_ERR_INVALID, "out[" + std::to_string(r) + "] is NULL");
    if (reinterpret_cast<uintptr_t>(out[r]) & 3)
      return fail(TIDE_ERR_ALIGN, "out[" + std::to_string(r) + "] is not 4-byte aligned");
  }
  if (plan->rs_chunks == 0) return TIDE_OK;  // nothing to write
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  tide_status st = bind_device(plan);
  if (st != TIDE_OK) return st;
  if (plan->rs_segs_stale) {
    st = upload(&plan->up_rs_segs, plan->d_rs, plan->rs.data(), plan->rs.size() * sizeof(Seg), stream);
    if (st != TIDE_OK) return st;
    plan->rs_segs_stale = false;
  }
  std::vector<void*>& cache = plan->rs_ptrs;
  const size_t nptr = size_t(W * P + W);
  bool same = plan->rs_ptrs_valid && cache.size() == nptr;
  if (same) {
    for (size_t i = 0; i < size_t(W * P) && same; ++i) same = cache[i] == grads[i];
    for (size_t r = 0; r < size_t(W) && same; ++r) same = cache[size_t(W * P) + r] == out[r];
  }
  if (!same) {
    cache.resize(nptr);
    for (size_t i = 0; i < size_t(W * P); ++i) cache[i] = const_cast<uint16_t*>(grads[i]);
    for (size_t r = 0; r < size_t(W); ++r) cache[size_t(W * P) + r] = out[r];
    plan->rs_ptrs_valid = false;
    st = upload(&plan->up_rs_ptrs, plan->d_rs_ptrs, cache.data(), nptr * sizeof(void*), stream);
    if (st != TIDE_OK) return st;
    plan->rs_ptrs_valid = true;
  }
  const int64_t grid = grid_for(plan, plan->rs_chunks);
  void* const* ptrs = plan->d_rs_ptrs;
  switch (W) {
    case 8: launch_rs<8>(plan, grid, stream, ptrs); break;
    case 4: launch_rs<4>(plan, grid, stream, ptrs); break;
    case 2: launch_rs<2>(plan, grid, stream, ptrs); break;
    default: launch_rs<0>(plan, grid, stream, ptrs); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "rs_local_kernel launch");
  return TIDE_OK;
}

tide_status tide_allgather_copyout(tide_plan* plan, const uint16_t* rank_major, uint16_t* const* params,
                                   void* stream_) {
  g_last_error.clear();
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  if (params == nullptr) return fail(TIDE_ERR_INVALID, "params must not be NULL");
  const tide::Geometry& g = plan->geo;
  const int64_t P = g.nparams;
  for (int64_t p = 0; p < P; ++p) {
    if (g.D[p] * g.K[p] == 0) continue;
    if (params[p] == nullptr) return fail(TIDE_ERR_INVALID, "params[" + std::to_string(p) + "] is NULL");
    if (reinterpret_cast<uintptr_t>(params[p]) & 1)
      return fail(TIDE_ERR_ALIGN, "params[" + std::to_string(p) + "] is not 2-byte aligned");
  }
  if (plan->co_chunks == 0) return TIDE_OK;  // nothing to write
  if (rank_major == nullptr) return fail(TIDE_ERR_INVALID, "rank_major must not be NULL");
  if (reinterpret_cast<uintptr_t>(rank_major) & 1) return fail(TIDE_ERR_ALIGN, "rank_major is not 2-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  tide_status st = bind_device(plan);
  if (st != TIDE_OK) return st;
  if (plan->co_segs_stale) {
    st = upload(&plan->up_co_segs, plan->d_co, plan->co.data(), plan->co.size() * sizeof(Seg), stream);
    if (st != TIDE_OK) return st;
    plan->co_segs_stale = false;
  }
  std::vector<void*>& cache = plan->co_ptrs;
  bool same = plan->co_ptrs_valid && cache.size() == size_t(P);
  for (size_t p = 0; p < size_t(P) && same; ++p) same = cache[p] == params[p];
  if (!same) {
    cache.assign(params, params + P);
    plan->co_ptrs_valid = false;
    st = upload(&plan->up_co_ptrs, plan->d_co_ptrs, cache.data(), size_t(P) * sizeof(void*), stream);
    if (st != TIDE_OK) return st;
    plan->co_ptrs_valid = true;
  }
  const int64_t grid = grid_for(plan, plan->co_chunks);
  const int32_t nseg = int32_t(plan->co.size());
  uint16_t* const* dparams = reinterpret_cast<uint16_t* const*>(plan->d_co_ptrs);
  const bool ntl = plan->opt.flags & TIDE_FLAG_NT_LOADS, nts = plan->opt.flags & TIDE_FLAG_NT_STORES;
#define TIDE_CO_LAUNCH(L, S)                                                                             \
  hipLaunchKernelGGL((ag_copyout_kernel<L, S>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, plan->d_co, \
                     nseg, plan->co_chunks, plan->opt.chunk_elems, rank_major, dparams)
  if (ntl && nts) {
    TIDE_CO_LAUNCH(true, true);
  } else if (ntl) {
    TIDE_CO_LAUNCH(true, false);
  } else if (nts) {
    TIDE_CO_LAUNCH(false, true);
  } else {
    TIDE_CO_LAUNCH(false, false);
  }
#undef TIDE_CO_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "ag_copyout_kernel launch");
  return TIDE_OK;
}

void tide_plan_destroy(tide_plan* plan) {
  if (plan == nullptr) return;
  {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    if (g_plans.erase(plan) == 0) return;  // unknown or already destroyed
  }
  release_device(plan);
  plan->magic = 0;
  delete plan;
}

const char* tide_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
