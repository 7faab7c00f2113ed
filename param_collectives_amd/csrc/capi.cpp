// C ABI of libtide (include/tide.h): plan lifetime, argument checks, device
// tables and kernel launches for the layout-aware FSDP2 collective local
// stages ("The Endgame of FSDP Communication", Wang et al., Sections 2.1, 4
// and 6).  Host code only; the kernels are in kernels.hip.
//
// Device state of a plan (allocated on its first launch, on the device that
// is current then):
//   chunk table   per operation, the first-chunk index of every segment
//                 (fixed by the plan and its chunk size; re-uploaded when the
//                 chunk size changes);
//   call table    per operation, every segment's resolved source and
//                 destination pointers and vector-body start, rebuilt on the
//                 host and re-uploaded only when a call passes pointers that
//                 differ from the previous call's (Section 6: no per-call
//                 metadata copy in steady state).
// Uploads go through pinned staging buffers with hipMemcpyAsync on the
// caller's stream, so they are ordered before the launch that reads them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_set>
#include <utility>
#include <vector>

#include "tide_internal.h"

namespace {

thread_local std::string g_last_error;

tide_status fail(tide_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

tide_status hip_fail(hipError_t e, const char* what) {
  return fail(TIDE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

namespace tide {

tide_status set_error(tide_status st, const std::string& msg) { return fail(st, msg); }

void clear_error() { g_last_error.clear(); }

tide_status set_error_nothrow(tide_status st, const char* msg) noexcept {
  try {
    g_last_error = msg;
  } catch (...) {
    g_last_error.clear();  // never allocates
  }
  return st;
}

}  // namespace tide

namespace {

// One host->device upload channel: a pinned staging buffer whose previous
// copy must have finished before it is rewritten.
struct Upload {
  void* host = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};

// Device tables of one operation.
struct OpState {
  std::vector<tide::Seg> segs;
  std::vector<int32_t> chunk_begin;  // host copy, [nseg + 1]
  bool chunks_stale = true;
  int32_t* d_chunk_begin = nullptr;
  void* d_call = nullptr;            // [CallHdr x nseg | pointers x nseg*(nsrc+1)]
  size_t call_bytes = 0;
  std::vector<const void*> key;      // pointers of the last uploaded call table
  bool key_valid = false;
  bool has_shift = false;            // reduce-scatter: the call table needs the realigning instance
  std::vector<tide::CallHdr> hdr;    // host scratch for building the call table
  std::vector<const void*> ptrs;
  std::vector<unsigned char> call_host;
  Upload up_chunks, up_call;
};

}  // namespace

// Host side of the allocation-free reduce-scatter: the buffers its calls
// build their tables in, sized when the plan is created, so that a call
// allocates nothing.  The tables go to the device's scratch array as one
// image: the chunk table (int32, padded to 16 bytes), the segment headers,
// then the pointers.
struct NoAllocHost {
  std::vector<tide::CallHdr> hdr;
  std::vector<const void*> ptrs;
  std::vector<uint64_t> image;
  size_t bytes = 0;     // of the image
  size_t hdr_off = 0;   // byte offsets of the headers and the pointers in it
  size_t ptrs_off = 0;
};

struct tide_plan {
  uint64_t magic = 0;
  tide::Geometry geo;
  tide_options given{};  // as passed (0 = default)
  OpState rs, co, ci, pk, rsf;  // rsf: the reduce-scatter of fp32 gradients
  NoAllocHost na;                // the allocation-free reduce-scatter (bf16 gradients)
  int device = -1;
  int cu_count = 0;
};

namespace {

constexpr uint64_t kMagic = 0x7469646570616e32ull;
std::mutex g_plans_mu;
std::unordered_set<const tide_plan*> g_plans;

bool live(const tide_plan* p) {
  if (p == nullptr) return false;
  std::lock_guard<std::mutex> lock(g_plans_mu);
  return g_plans.count(p) != 0 && p->magic == kMagic;
}

int32_t nsrc_of(const tide_plan* p, tide::Op op) {
  return op == tide::kOpRs || op == tide::kOpRsF32 ? p->geo.world : 1;
}

OpState& op_state(tide_plan* p, tide::Op op) {
  switch (op) {
    case tide::kOpRs: return p->rs;
    case tide::kOpCo: return p->co;
    case tide::kOpCi: return p->ci;
    case tide::kOpPack: return p->pk;
    default: return p->rsf;
  }
}
const OpState& op_state(const tide_plan* p, tide::Op op) { return op_state(const_cast<tide_plan*>(p), op); }

const tide::Op kOps[tide::kNumOps] = {tide::kOpRs, tide::kOpCo, tide::kOpCi, tide::kOpPack, tide::kOpRsF32};

const char* const kOpNames =
    "0 (reduce-scatter), 1 (copy-out), 2 (copy-in), 3 (stock pack) or 4 (reduce-scatter of fp32 gradients)";

tide_status rebuild_chunks(tide_plan* p, const tide_options& given) {
  std::string why;
  std::vector<int32_t> cb[tide::kNumOps];
  for (int i = 0; i < tide::kNumOps; ++i) {
    const tide_options eff = tide::effective_options(given, kOps[i], 0, p->geo.world);
    tide_status st = tide::chunk_table(op_state(p, kOps[i]).segs, eff.chunk_elems, &cb[i], &why);
    if (st != TIDE_OK) return fail(st, why);
  }
  for (int i = 0; i < tide::kNumOps; ++i) {
    op_state(p, kOps[i]).chunk_begin.swap(cb[i]);
    op_state(p, kOps[i]).chunks_stale = true;
  }
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

// hipFree synchronizes the device first, so launches still reading the tables
// finish before they are freed.
void release_op(OpState* s) {
  free_upload(&s->up_chunks);
  free_upload(&s->up_call);
  if (s->d_chunk_begin) (void)hipFree(s->d_chunk_begin);
  if (s->d_call) (void)hipFree(s->d_call);
  s->d_chunk_begin = nullptr;
  s->d_call = nullptr;
  s->key_valid = false;
  s->chunks_stale = true;
}

void release_device(tide_plan* p) {
  if (p->device < 0) return;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(p->device);
  for (tide::Op op : kOps) release_op(&op_state(p, op));
  p->device = -1;
  if (prev >= 0) (void)hipSetDevice(prev);
}

tide_status alloc_op(OpState* s, int32_t nsrc) {
  const size_t nseg = s->segs.size();
  s->call_bytes = nseg * sizeof(tide::CallHdr) + nseg * size_t(nsrc + 1) * sizeof(void*);
  tide_status st;
  if ((st = dev_alloc(&s->d_chunk_begin, (nseg + 1) * sizeof(int32_t))) != TIDE_OK) return st;
  if ((st = dev_alloc(&s->d_call, s->call_bytes)) != TIDE_OK) return st;
  if ((st = make_upload(&s->up_chunks, (nseg + 1) * sizeof(int32_t))) != TIDE_OK) return st;
  return make_upload(&s->up_call, s->call_bytes);
}

// Bind the plan to the current device on first use.
tide_status bind_device(tide_plan* p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->device >= 0) {
    if (dev != p->device)
      return fail(TIDE_ERR_INVALID, "plan is bound to device " + std::to_string(p->device) + " but device " +
                                        std::to_string(dev) + " is current");
    return TIDE_OK;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  p->device = dev;
  p->cu_count = cus;
  tide_status st = TIDE_OK;
  for (tide::Op op : kOps)
    if (st == TIDE_OK) st = alloc_op(&op_state(p, op), nsrc_of(p, op));
  if (st != TIDE_OK) {
    const std::string why = g_last_error;
    release_device(p);
    return fail(st, why);
  }
  return TIDE_OK;
}

// How one call of an operation is split into kernel launches.  At most
// wave_chunks chunks per wave per launch: longer work runs as several
// launches of consecutive chunk ranges.  A round is one chunk for every wave;
// the launches get equal numbers of whole rounds (a short last launch would be
// all ramp-up and tail, a partial round leaves waves idle).
struct Launches {
  int64_t grid;                                     // workgroups of a full launch
  std::vector<std::pair<int64_t, int64_t>> ranges;  // [first, end) chunks of each launch
  int64_t nchunks;                                  // of the whole operation
};

// A reduce-scatter's chunks are first cut into groups, each split that way
// on its own: a group ends where the next rank's shard (a destination stream
// of at least one round) begins off the phase of the group's rounds (more
// than waves/64 chunks from a round boundary), once the group holds at least
// wave_chunks/2 rounds.  That rank's first chunk then opens a launch, and its
// rounds line up with the start of its shard as rank 0's do.  (Measured on
// MI355X, same-box A/B in the timed step: the reduce-scatter of the Qwen3 MoE
// layer, whose ranks own 292 mod 1024 chunks each, +0.75%; of the Wan2.2
// block, 915 mod 1024, +0.9%.  The Llama layers' ranks own 2 mod 1024 chunks
// and are not cut.  The same cut at a copy-out's parameters moved the Wan2.2
// copy-out by -0.7 to +0.4%, so the copies keep one group.)
Launches split_launches(const OpState& s, const tide_options& eff, bool by_destination) {
  Launches L;
  L.nchunks = s.chunk_begin.back();
  int64_t grid = int64_t(eff.cu_budget) * eff.wg_per_cu;
  const int64_t useful = (L.nchunks + tide::kWavesPerGroup - 1) / tide::kWavesPerGroup;
  if (grid > useful) grid = useful;
  if (grid > tide::kMaxGrid) grid = tide::kMaxGrid;
  if (grid < 1) grid = 1;
  L.grid = grid;
  const int64_t waves = grid * tide::kWavesPerGroup;
  // group boundaries (first chunks), then each group's launches
  std::vector<int64_t> cuts{0};
  const int64_t tol = std::max<int64_t>(1, waves / 64);
  const int64_t min_group = waves * std::max<int64_t>(1, eff.wave_chunks / 2);
  size_t i = by_destination ? 1 : s.segs.size();
  while (i < s.segs.size()) {
    if (s.segs[i].dst_idx == s.segs[i - 1].dst_idx) {
      ++i;
      continue;
    }
    size_t j = i + 1;  // [i, j): the run of segments with this destination
    while (j < s.segs.size() && s.segs[j].dst_idx == s.segs[i].dst_idx) ++j;
    const int64_t c = s.chunk_begin[i], run = s.chunk_begin[j] - c;
    const int64_t phase = (c - cuts.back()) % waves;
    if (phase > tol && phase < waves - tol && run >= waves && c - cuts.back() >= min_group) cuts.push_back(c);
    i = j;
  }
  cuts.push_back(L.nchunks);
  for (size_t k = 0; k + 1 < cuts.size(); ++k) {
    const int64_t g0 = cuts[k], n = cuts[k + 1] - g0;
    const int64_t rounds = (n + waves - 1) / waves;
    const int64_t launches = std::max<int64_t>(1, (rounds + eff.wave_chunks - 1) / eff.wave_chunks);
    const int64_t per = std::max<int64_t>(1, (rounds + launches - 1) / launches * waves);
    for (int64_t c0 = g0; c0 < g0 + n; c0 += per) L.ranges.emplace_back(c0, std::min(g0 + n, c0 + per));
  }
  return L;
}

// The launch of chunks [c0, c1): its span (chunks, and the segments they
// fall in) and its workgroup count.
void launch_at(const OpState& s, const Launches& L, int64_t c0, int64_t c1, tide::ChunkSpan* span, int64_t* grid) {
  // the segment of chunk c0, and one past the segment of chunk c1 - 1
  const auto it = std::upper_bound(s.chunk_begin.begin(), s.chunk_begin.end(), int32_t(c0));
  const auto it_end = std::upper_bound(it, s.chunk_begin.end(), int32_t(c1 - 1));
  *span = tide::ChunkSpan{int32_t(c0), int32_t(c1), int32_t(it - s.chunk_begin.begin()) - 1,
                          int32_t(it_end - s.chunk_begin.begin())};
  *grid = std::min<int64_t>(L.grid, (c1 - c0 + tide::kWavesPerGroup - 1) / tide::kWavesPerGroup);
}

// Whether a reduce-scatter call should run the kernel instance that realigns
// sum segments whose sources (all at one phase) are off a 4-element group
// boundary where the destination is 16-byte aligned: when such segments hold
// more than 1/50 of the call's elements.  (That instance is a few percent
// slower on aligned segments; the plain ones sum a few off-phase segments,
// say the norms of a layer, element by element.)
bool needs_shift(const std::vector<tide::CallHdr>& hdr, const std::vector<const void*>& ptrs, int32_t nsrc,
                 bool f32) {
  const uintptr_t esize = f32 ? 4 : 2;
  int64_t off = 0, total = 0;
  for (size_t i = 0; i < hdr.size(); ++i) {
    const tide::CallHdr& h = hdr[i];
    if (h.kind != tide::kSum) continue;
    total += h.len;
    if (h.head < 0 || h.len <= h.head) continue;
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptrs[i * size_t(nsrc + 1)]) + uintptr_t(h.head) * esize;
    if ((a & (4 * esize - 1)) != 0) off += h.len;
  }
  return off > total / 50;
}

tide_status launch_op(const OpState& s, tide::Op op, const tide_options& eff, tide::KernelArgs a, hipStream_t stream,
                      bool f32);

// Upload what is stale, then launch.  `f32`: the reduce-scatter's gradients
// or the copy-in's shards are fp32.  `alpha`, `accumulate`: the
// reduce-scatter's Equation 5 terms.
template <typename BuildCall>
tide_status run_op(tide_plan* p, tide::Op op, const std::vector<const void*>& key, BuildCall build,
                   hipStream_t stream, bool f32 = false, float alpha = 1.0f, int32_t accumulate = 0) {
  OpState& s = op_state(p, op);
  const int32_t nchunks = s.chunk_begin.back();
  if (nchunks == 0) return TIDE_OK;  // nothing to write
  // Under graph capture a call may only enqueue kernel launches: the plan's
  // first call (device set-up) and table uploads (new pointers or options)
  // would allocate, copy or synchronize, so they are refused before any of it.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t ce = hipStreamIsCapturing(stream, &cap);
  if (ce != hipSuccess) return hip_fail(ce, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone && (p->device < 0 || s.chunks_stale || !s.key_valid || s.key != key))
    return fail(TIDE_ERR_INVALID,
                "the stream is capturing a graph, but this call would set up or upload the plan's device tables "
                "(first call, new pointers or new options): make the same call once before capturing");
  tide_status st = bind_device(p);
  if (st != TIDE_OK) return st;
  if (s.chunks_stale) {
    st = upload(&s.up_chunks, s.d_chunk_begin, s.chunk_begin.data(), s.chunk_begin.size() * sizeof(int32_t),
                stream);
    if (st != TIDE_OK) return st;
    s.chunks_stale = false;
  }
  if (!s.key_valid || s.key != key) {
    s.key_valid = false;
    build(&s.hdr, &s.ptrs);
    s.has_shift = (op == tide::kOpRs || op == tide::kOpRsF32) && needs_shift(s.hdr, s.ptrs, nsrc_of(p, op), f32);
    const size_t hb = s.hdr.size() * sizeof(tide::CallHdr), pb = s.ptrs.size() * sizeof(void*);
    s.call_host.resize(hb + pb);
    std::memcpy(s.call_host.data(), s.hdr.data(), hb);
    std::memcpy(s.call_host.data() + hb, s.ptrs.data(), pb);
    st = upload(&s.up_call, s.d_call, s.call_host.data(), hb + pb, stream);
    if (st != TIDE_OK) return st;
    s.key = key;
    s.key_valid = true;
  }
  tide::KernelArgs a;
  a.hdr = static_cast<const tide::CallHdr*>(s.d_call);
  a.ptrs = reinterpret_cast<const void* const*>(static_cast<unsigned char*>(s.d_call) +
                                                s.segs.size() * sizeof(tide::CallHdr));
  a.chunk_begin = s.d_chunk_begin;
  a.nsrc = nsrc_of(p, op);
  a.alpha = alpha;
  a.accumulate = accumulate;
  a.realign = s.has_shift;
  return launch_op(s, op, tide::effective_options(p->given, op, p->cu_count, p->geo.world), a, stream, f32);
}

// Launch every kernel of one call of `op` whose tables `a` points to (its
// hdr, ptrs, chunk_begin, nsrc and Equation 5 fields set; the rest is filled
// in here from the options).
tide_status launch_op(const OpState& s, tide::Op op, const tide_options& eff, tide::KernelArgs a, hipStream_t stream,
                      bool f32) {
  const int32_t nchunks = s.chunk_begin.back();
  const Launches L = split_launches(s, eff, op == tide::kOpRs || op == tide::kOpRsF32);
  a.nchunks = nchunks;
  a.chunk = int32_t(eff.chunk_elems);
  a.flags = eff.flags;
  for (const auto& rg : L.ranges) {
    int64_t g = 0;
    launch_at(s, L, rg.first, rg.second, &a.span, &g);
    int rc = 0;
    const char* what = "";
    switch (op) {
      case tide::kOpRs:
      case tide::kOpRsF32:
        rc = tide::launch_rs_local(a, f32, g, stream);
        what = "rs_local_kernel launch";
        break;
      case tide::kOpCo:
        rc = tide::launch_ag_copyout(a, g, stream);
        what = "ag_copyout_kernel launch";
        break;
      case tide::kOpCi:
        rc = tide::launch_ag_copyin(a, f32, g, stream);
        what = "ag_copyin_kernel launch";
        break;
      case tide::kOpPack:
        rc = tide::launch_stock_pack(a, g, stream);
        what = "stock_pack_kernel launch";
        break;
    }
    if (rc != 0) return hip_fail(hipError_t(rc), what);
  }
  return TIDE_OK;
}

// Argument checks of every reduce-scatter entry point: `grads` holds uint16_t
// (bf16) or float pointers, as `f32` says.
tide_status check_rs(const tide_plan* plan, const void* const* grads, bool f32, float* const* out,
                     int32_t accumulate) {
  if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
  if (grads == nullptr || out == nullptr) return fail(TIDE_ERR_INVALID, "grads and out must not be NULL");
  if (accumulate != 0 && accumulate != 1) return fail(TIDE_ERR_INVALID, "accumulate must be 0 or 1");
  const tide::Geometry& g = plan->geo;
  const int64_t W = g.world, P = g.nparams;
  const uintptr_t align = f32 ? 4 : 2;
  for (int64_t u = 0; u < W; ++u) {
    for (int64_t p = 0; p < P; ++p) {
      const void* ptr = grads[u * P + p];
      if (g.D[p] * g.K[p] == 0) continue;
      if (ptr == nullptr) return fail(TIDE_ERR_INVALID, "grads[" + std::to_string(u * P + p) + "] is NULL");
      if (reinterpret_cast<uintptr_t>(ptr) & (align - 1))
        return fail(TIDE_ERR_ALIGN, "grads[" + std::to_string(u * P + p) + "] is not aligned to its element size");
    }
  }
  for (int64_t r = 0; r < W; ++r) {
    if (g.S == 0) continue;
    if (out[r] == nullptr) return fail(TIDE_ERR_INVALID, "out[" + std::to_string(r) + "] is NULL");
    if (reinterpret_cast<uintptr_t>(out[r]) & 3)
      return fail(TIDE_ERR_ALIGN, "out[" + std::to_string(r) + "] is not 4-byte aligned");
  }
  return TIDE_OK;
}

// Both reduce-scatter entry points with plan-owned device tables.
tide_status reduce_scatter(tide_plan* plan, const void* const* grads, bool f32, float* const* out, float alpha,
                           int32_t accumulate, void* stream) {
  g_last_error.clear();
  tide_status st = check_rs(plan, grads, f32, out, accumulate);
  if (st != TIDE_OK) return st;
  const tide::Geometry& g = plan->geo;
  const int64_t W = g.world, P = g.nparams;
  std::vector<const void*> key(grads, grads + W * P);
  key.insert(key.end(), out, out + W);
  const tide::Op op = f32 ? tide::kOpRsF32 : tide::kOpRs;
  return run_op(
      plan, op, key,
      [&](std::vector<tide::CallHdr>* hdr, std::vector<const void*>* ptrs) {
        tide::rs_call_table(g, op_state(plan, op).segs, grads, f32, out, hdr, ptrs);
      },
      static_cast<hipStream_t>(stream), f32, alpha, accumulate);
}

// Sizes the allocation-free reduce-scatter's host buffers (when its image
// fits the device scratch; its calls are refused otherwise).
void size_noalloc(tide_plan* p) {
  NoAllocHost& na = p->na;
  const size_t nseg = p->rs.segs.size(), W = size_t(p->geo.world);
  na.hdr_off = ((nseg + 1) * sizeof(int32_t) + 15) / 16 * 16;
  na.ptrs_off = na.hdr_off + nseg * sizeof(tide::CallHdr);
  na.bytes = na.ptrs_off + nseg * (W + 1) * sizeof(void*);
  if (na.bytes > tide::kScratchBytes) return;
  na.hdr.reserve(nseg);
  na.ptrs.reserve(nseg * (W + 1));
  na.image.assign((na.bytes + 7) / 8, 0);
}

// The allocation-free reduce-scatter: the tables of this call are built in the
// plan's preallocated host buffers, written to the current device's scratch
// array by put launches (their words travel as kernel arguments) and read
// there by the same kernels as tide_reduce_scatter_local's.
tide_status reduce_scatter_noalloc(tide_plan* plan, const uint16_t* const* grads, float* const* out, float alpha,
                                   int32_t accumulate, void* stream_v) {
  g_last_error.clear();
  tide_status st = check_rs(plan, reinterpret_cast<const void* const*>(grads), false, out, accumulate);
  if (st != TIDE_OK) return st;
  const OpState& s = plan->rs;
  NoAllocHost& na = plan->na;
  if (na.bytes > tide::kScratchBytes)
    return fail(TIDE_ERR_RANGE, "the reduce-scatter's tables take " + std::to_string(na.bytes) +
                                    " bytes; the allocation-free entry point holds at most " +
                                    std::to_string(tide::kScratchBytes));
  if (s.chunk_begin.back() == 0) return TIDE_OK;  // nothing to write
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  void* base = nullptr;
  int rc = tide::scratch_address(&base);
  if (rc != 0) return hip_fail(hipError_t(rc), "hipGetSymbolAddress of the scratch array");
  int dev = -1, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");

  const tide::Geometry& g = plan->geo;
  tide::rs_call_table(g, s.segs, reinterpret_cast<const void* const*>(grads), false, out, &na.hdr, &na.ptrs);
  unsigned char* img = reinterpret_cast<unsigned char*>(na.image.data());
  std::memcpy(img, s.chunk_begin.data(), s.chunk_begin.size() * sizeof(int32_t));
  std::memcpy(img + na.hdr_off, na.hdr.data(), na.hdr.size() * sizeof(tide::CallHdr));
  std::memcpy(img + na.ptrs_off, na.ptrs.data(), na.ptrs.size() * sizeof(void*));
  const size_t words = (na.bytes + 7) / 8;
  for (size_t w0 = 0; w0 < words; w0 += tide::kPutWords) {
    const uint32_t n = uint32_t(std::min<size_t>(tide::kPutWords, words - w0));
    rc = tide::launch_scratch_put(static_cast<uint64_t*>(base) + w0, na.image.data() + w0, n, stream);
    if (rc != 0) return hip_fail(hipError_t(rc), "scratch_put_kernel launch");
  }
  tide::KernelArgs a;
  unsigned char* b = static_cast<unsigned char*>(base);
  a.chunk_begin = reinterpret_cast<const int32_t*>(b);
  a.hdr = reinterpret_cast<const tide::CallHdr*>(b + na.hdr_off);
  a.ptrs = reinterpret_cast<const void* const*>(b + na.ptrs_off);
  a.nsrc = g.world;
  a.alpha = alpha;
  a.accumulate = accumulate;
  a.realign = needs_shift(na.hdr, na.ptrs, g.world, false);
  return launch_op(s, tide::kOpRs, tide::effective_options(plan->given, tide::kOpRs, cus, g.world), a, stream, false);
}

}  // namespace

extern "C" {

tide_status tide_plan_create(int32_t world, int32_t nparams, const int32_t* ndims, const int64_t* dims,
                             const tide_options* opt, tide_plan** out_plan) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (out_plan == nullptr) return fail(TIDE_ERR_INVALID, "out_plan must not be NULL");
    *out_plan = nullptr;
    std::string why;
    tide_options given;
    tide_status st = tide::check_options(opt, &given, &why);
    if (st != TIDE_OK) return fail(st, why);
    // Owned here until it is registered: any early return frees it (no device
    // state exists before the first launch).
    std::unique_ptr<tide_plan> p(new tide_plan());
    st = tide::build_geometry(world, nparams, ndims, dims, &p->geo, &why);
    if (st != TIDE_OK) return fail(st, why);
    p->rs.segs = tide::rs_segments(p->geo);
    p->co.segs = tide::copyout_segments(p->geo);
    p->ci.segs = tide::copyin_segments(p->geo);
    p->pk.segs = tide::pack_segments(p->geo);
    p->rsf.segs = p->rs.segs;
    for (tide::Op op : kOps)
      if (op_state(p.get(), op).segs.size() >= size_t(INT32_MAX)) return fail(TIDE_ERR_RANGE, "too many segments");
    p->given = given;
    st = rebuild_chunks(p.get(), given);
    if (st != TIDE_OK) return st;
    size_noalloc(p.get());
    p->magic = kMagic;
    {
      std::lock_guard<std::mutex> lock(g_plans_mu);
      g_plans.insert(p.get());
    }
    *out_plan = p.release();
    return TIDE_OK;
  });
}

tide_status tide_plan_layout(const tide_plan* plan, int64_t* rows_per_rank, int64_t* shard_offset,
                             int64_t* shard_elems) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    for (int32_t p = 0; p < plan->geo.nparams; ++p) {
      if (rows_per_rank) rows_per_rank[p] = plan->geo.R[p];
      if (shard_offset) shard_offset[p] = plan->geo.o[p];
    }
    if (shard_elems) *shard_elems = plan->geo.S;
    return TIDE_OK;
  });
}

tide_status tide_plan_sizes(const tide_plan* plan, int64_t* param_elems, int64_t* real_elems) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    const tide::Geometry& g = plan->geo;
    for (int32_t p = 0; p < g.nparams; ++p) {
      if (param_elems) param_elems[p] = g.D[p] * g.K[p];
      if (real_elems)
        for (int32_t r = 0; r < g.world; ++r) real_elems[int64_t(r) * g.nparams + p] = tide::real_elems(g, p, r);
    }
    return TIDE_OK;
  });
}

tide_status tide_plan_segments(const tide_plan* plan, int32_t op, int64_t* table, int64_t capacity,
                               int64_t* count) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    if (op < 0 || op >= tide::kNumOps) return fail(TIDE_ERR_INVALID, std::string("op must be ") + kOpNames);
    if (count == nullptr || capacity < 0 || (capacity > 0 && table == nullptr))
      return fail(TIDE_ERR_INVALID, "bad table/capacity/count");
    const std::vector<tide::Seg>& segs = op_state(plan, tide::Op(op)).segs;
    *count = int64_t(segs.size());
    const int64_t n = capacity < *count ? capacity : *count;
    for (int64_t i = 0; i < n; ++i) {
      const tide::Seg& s = segs[size_t(i)];
      int64_t* row = table + 6 * i;
      row[0] = s.kind;
      row[1] = s.src_idx;
      row[2] = s.dst_idx;
      row[3] = s.src_off;
      row[4] = s.dst_off;
      row[5] = s.len;
    }
    return TIDE_OK;
  });
}

tide_status tide_plan_launches(const tide_plan* plan, int32_t op, int32_t cu_count, int64_t* table,
                               int64_t capacity, int64_t* count) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    if (op < 0 || op >= tide::kNumOps) return fail(TIDE_ERR_INVALID, std::string("op must be ") + kOpNames);
    if (count == nullptr || capacity < 0 || (capacity > 0 && table == nullptr))
      return fail(TIDE_ERR_INVALID, "bad table/capacity/count");
    if (cu_count < 0) return fail(TIDE_ERR_INVALID, "cu_count must be >= 0");
    const tide_options eff =
        tide::effective_options(plan->given, tide::Op(op), cu_count > 0 ? cu_count : plan->cu_count, plan->geo.world);
    if (eff.cu_budget <= 0)
      return fail(TIDE_ERR_INVALID, "the plan is not bound to a device and has no cu_budget: pass cu_count");
    const OpState& s = op_state(plan, tide::Op(op));
    *count = 0;
    if (s.chunk_begin.back() == 0) return TIDE_OK;
    const Launches L = split_launches(s, eff, op == tide::kOpRs || op == tide::kOpRsF32);
    int64_t n = 0;
    for (const auto& rg : L.ranges) {
      if (n++ >= capacity) continue;
      tide::ChunkSpan sp;
      int64_t g = 0;
      launch_at(s, L, rg.first, rg.second, &sp, &g);
      int64_t* row = table + 5 * (n - 1);
      row[0] = sp.first;
      row[1] = sp.end;
      row[2] = sp.seg;
      row[3] = sp.seg_end;
      row[4] = g;
    }
    *count = n;
    return TIDE_OK;
  });
}

tide_status tide_plan_paths(const tide_plan* plan, int32_t op, int64_t* out) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    if (op < 0 || op >= tide::kNumOps) return fail(TIDE_ERR_INVALID, std::string("op must be ") + kOpNames);
    if (out == nullptr) return fail(TIDE_ERR_INVALID, "out must not be NULL");
    const OpState& s = op_state(plan, tide::Op(op));
    if (!s.key_valid)
      return fail(TIDE_ERR_INVALID, "no call of this operation has been made with the plan yet");
    const bool rs = op == tide::kOpRs || op == tide::kOpRsF32;
    const int32_t nsrc = nsrc_of(plan, tide::Op(op));
    int64_t vec = 0, shifted = 0, elem = 0;
    for (size_t i = 0; i < s.hdr.size(); ++i) {
      const tide::CallHdr& h = s.hdr[i];
      const void* src = s.ptrs[i * size_t(nsrc + 1)];
      // the kernels' vector group (elements) and source element size for this segment
      int64_t group = 4, esize = 0, salign = 16;
      switch (op) {
        case tide::kOpRs: esize = 2; salign = 8; break;
        case tide::kOpRsF32: esize = 4; break;
        case tide::kOpCo: group = 8; esize = 2; break;
        case tide::kOpCi:
          if (h.kind == tide::kCast) {
            esize = 4;
          } else {
            group = 8;
            esize = 2;
          }
          break;
        default: break;  // stock pack: the body starts where source and destination are both aligned
      }
      if (h.kind == tide::kZero || src == nullptr) esize = 0;
      if (h.head < 0 || h.len <= h.head) {
        elem += h.len;
        continue;
      }
      const int64_t body = (h.len - h.head) / group * group;
      elem += h.len - body;
      const bool off = esize > 0 && ((reinterpret_cast<uintptr_t>(src) + uintptr_t(h.head * esize)) &
                                     uintptr_t(salign - 1)) != 0;
      if (!off) {
        vec += body;
      } else if (!rs || s.has_shift) {
        shifted += body;
      } else {
        elem += body;  // the plain reduce-scatter instances take an off-phase body element by element
      }
    }
    out[0] = vec;
    out[1] = shifted;
    out[2] = elem;
    out[3] = rs && s.has_shift ? 1 : 0;
    return TIDE_OK;
  });
}

tide_status tide_plan_set_options(tide_plan* plan, const tide_options* opt) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    std::string why;
    tide_options given;
    tide_status st = tide::check_options(opt, &given, &why);
    if (st != TIDE_OK) return fail(st, why);
    st = rebuild_chunks(plan, given);
    if (st != TIDE_OK) return st;
    plan->given = given;
    return TIDE_OK;
  });
}

tide_status tide_plan_get_options(const tide_plan* plan, int32_t op, tide_options* out) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    if (op < 0 || op >= tide::kNumOps) return fail(TIDE_ERR_INVALID, std::string("op must be ") + kOpNames);
    if (out == nullptr) return fail(TIDE_ERR_INVALID, "out must not be NULL");
    *out = tide::effective_options(plan->given, tide::Op(op), plan->cu_count, plan->geo.world);
    return TIDE_OK;
  });
}

tide_status tide_reduce_scatter_local(tide_plan* plan, const uint16_t* const* grads, float* const* out,
                                      float alpha, int32_t accumulate, void* stream) {
  return tide::guarded([&]() -> tide_status {
    return reduce_scatter(plan, reinterpret_cast<const void* const*>(grads), false, out, alpha, accumulate, stream);
  });
}

tide_status tide_reduce_scatter_local_noalloc(tide_plan* plan, const uint16_t* const* grads, float* const* out,
                                              float alpha, int32_t accumulate, void* stream) {
  return tide::guarded(
      [&]() -> tide_status { return reduce_scatter_noalloc(plan, grads, out, alpha, accumulate, stream); });
}

tide_status tide_reduce_scatter_local_f32(tide_plan* plan, const float* const* grads, float* const* out,
                                          float alpha, int32_t accumulate, void* stream) {
  return tide::guarded([&]() -> tide_status {
    return reduce_scatter(plan, reinterpret_cast<const void* const*>(grads), true, out, alpha, accumulate, stream);
  });
}

tide_status tide_allgather_copyout(tide_plan* plan, const uint16_t* rank_major, uint16_t* const* params,
                                   void* stream) {
  return tide::guarded([&]() -> tide_status {
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
    if (plan->co.chunk_begin.back() == 0) return TIDE_OK;  // nothing to write
    if (rank_major == nullptr) return fail(TIDE_ERR_INVALID, "rank_major must not be NULL");
    if (reinterpret_cast<uintptr_t>(rank_major) & 1) return fail(TIDE_ERR_ALIGN, "rank_major is not 2-byte aligned");
    std::vector<const void*> key(params, params + P);
    key.push_back(rank_major);
    return run_op(
        plan, tide::kOpCo, key,
        [&](std::vector<tide::CallHdr>* hdr, std::vector<const void*>* ptrs) {
          tide::co_call_table(g, plan->co.segs, rank_major, params, hdr, ptrs);
        },
        static_cast<hipStream_t>(stream));
  });
}

tide_status tide_allgather_copyin(tide_plan* plan, const void* const* shards, int32_t shard_dtype,
                                  uint16_t* rank_major, void* stream) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    if (shards == nullptr) return fail(TIDE_ERR_INVALID, "shards must not be NULL");
    if (shard_dtype != TIDE_DTYPE_BF16 && shard_dtype != TIDE_DTYPE_F32)
      return fail(TIDE_ERR_INVALID, "shard_dtype must be TIDE_DTYPE_BF16 or TIDE_DTYPE_F32");
    const tide::Geometry& g = plan->geo;
    const int64_t W = g.world, P = g.nparams;
    const uintptr_t align = shard_dtype == TIDE_DTYPE_F32 ? 4 : 2;
    for (int64_t r = 0; r < W; ++r) {
      for (int64_t p = 0; p < P; ++p) {
        if (tide::real_elems(g, int32_t(p), int32_t(r)) == 0) continue;
        const void* s = shards[r * P + p];
        if (s == nullptr) return fail(TIDE_ERR_INVALID, "shards[" + std::to_string(r * P + p) + "] is NULL");
        if (reinterpret_cast<uintptr_t>(s) & (align - 1))
          return fail(TIDE_ERR_ALIGN, "shards[" + std::to_string(r * P + p) + "] is not aligned to its element size");
      }
    }
    if (plan->ci.chunk_begin.back() == 0) return TIDE_OK;  // nothing to write
    if (rank_major == nullptr) return fail(TIDE_ERR_INVALID, "rank_major must not be NULL");
    if (reinterpret_cast<uintptr_t>(rank_major) & 1) return fail(TIDE_ERR_ALIGN, "rank_major is not 2-byte aligned");
    const bool f32 = shard_dtype == TIDE_DTYPE_F32;
    std::vector<const void*> key(shards, shards + W * P);
    key.push_back(rank_major);
    key.push_back(reinterpret_cast<const void*>(uintptr_t(shard_dtype)));
    return run_op(
        plan, tide::kOpCi, key,
        [&](std::vector<tide::CallHdr>* hdr, std::vector<const void*>* ptrs) {
          tide::ci_call_table(g, plan->ci.segs, shards, f32, rank_major, hdr, ptrs);
        },
        static_cast<hipStream_t>(stream), f32);
  });
}

tide_status tide_stock_chunk_cat(tide_plan* plan, const uint16_t* const* grads, float* packed, void* stream) {
  return tide::guarded([&]() -> tide_status {
    g_last_error.clear();
    if (!live(plan)) return fail(TIDE_ERR_INVALID, "unknown or destroyed plan");
    if (grads == nullptr) return fail(TIDE_ERR_INVALID, "grads must not be NULL");
    const tide::Geometry& g = plan->geo;
    const int64_t P = g.nparams;
    for (int64_t p = 0; p < P; ++p) {
      if (g.D[p] * g.K[p] == 0) continue;
      if (grads[p] == nullptr) return fail(TIDE_ERR_INVALID, "grads[" + std::to_string(p) + "] is NULL");
      if (reinterpret_cast<uintptr_t>(grads[p]) & 1)
        return fail(TIDE_ERR_ALIGN, "grads[" + std::to_string(p) + "] is not 2-byte aligned");
    }
    if (plan->pk.chunk_begin.back() == 0) return TIDE_OK;  // nothing to write
    if (packed == nullptr) return fail(TIDE_ERR_INVALID, "packed must not be NULL");
    if (reinterpret_cast<uintptr_t>(packed) & 3) return fail(TIDE_ERR_ALIGN, "packed is not 4-byte aligned");
    std::vector<const void*> key(grads, grads + P);
    key.push_back(packed);
    return run_op(
        plan, tide::kOpPack, key,
        [&](std::vector<tide::CallHdr>* hdr, std::vector<const void*>* ptrs) {
          tide::pk_call_table(g, plan->pk.segs, grads, packed, hdr, ptrs);
        },
        static_cast<hipStream_t>(stream));
  });
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
