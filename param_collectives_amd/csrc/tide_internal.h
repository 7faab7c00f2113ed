// Private types shared by the host planner (plan.cpp), the C ABI (capi.cpp),
// the device code (kernels.hip) and the allocation-free scratch (scratch.hip)
// of the layout-aware FSDP2 collective local stages.
#pragma once

#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "tide.h"

namespace tide {

constexpr int kThreads = 256;  // threads per workgroup: four wave64s, each an independent worker
constexpr int kWavesPerGroup = kThreads / 64;
constexpr int64_t kMaxChunk = int64_t(1) << 28;  // keeps a chunk's byte offsets within 32 bits
// Chunk indices and wave counts are int32 on the device: with at most 2^30
// chunks and 2^27 workgroups (2^29 waves), chunk + waves never overflows.
constexpr int64_t kMaxChunks = int64_t(1) << 30;
constexpr int64_t kMaxGrid = int64_t(1) << 27;
constexpr int32_t kMaxStagedSegs = 16383;  // chunk-index table entries staged in LDS (64 KiB)

// Per-operation defaults, measured on MI355X over the four layer workloads:
// one workgroup (four waves) per CU keeps the HBM read/write mix most
// efficient for every kernel; the reduce-scatter prefers small chunks (the
// grid then sweeps a narrow window of every tensor), the copies larger ones.
// With fp32 gradients the reduce-scatter reads twice the bytes per element
// and takes one group per lane per step; its best chunk is a quarter as long.
constexpr int32_t kRsWgPerCu = 1;
constexpr int64_t kRsChunk = 1024;
constexpr int64_t kRsChunkFewRanks = 2048;  // W <= 3: fewer bytes per element, longer chunks for full steps
constexpr int32_t kRsF32WgPerCu = 1;
constexpr int64_t kRsF32Chunk = 256;
constexpr int32_t kCoWgPerCu = 1;
constexpr int64_t kCoChunk = 4096;
constexpr int32_t kCiWgPerCu = 1;
constexpr int64_t kCiChunk = 4096;
constexpr int32_t kPkWgPerCu = 1;    // the stock pack (bf16 -> fp32 widening copy)
constexpr int64_t kPkChunk = 2048;
constexpr int32_t kMaxWaveChunks = 1 << 30;  // chunks per wave per launch: no split
constexpr int32_t kWaveChunks = 64;  // measured on MI355X: 48-128 are equally good, 8 and no split 5-9% worse

enum SegKind : int32_t { kSum = 0, kZero = 1, kCopy = 2, kCast = 3 };
// Operations with their own chunk tables and launch knobs.  kOpRsF32 is the
// reduce-scatter of fp32 gradients: the same segments as kOpRs.
enum Op : int32_t { kOpRs = 0, kOpCo = 1, kOpCi = 2, kOpPack = 3, kOpRsF32 = 4 };
constexpr int kNumOps = 5;

// One contiguous run of work, fixed by the plan (host only).
struct Seg {
  int64_t src_off;  // element offset into each source tensor
  int64_t dst_off;  // element offset into the destination tensor
  int64_t len;      // elements, > 0
  int32_t src_idx;  // reduce-scatter, pack: parameter p; copy-out: 0; copy-in: shard r*P + p
  int32_t dst_idx;  // reduce-scatter: destination rank r; copy-out: parameter p; copy-in, pack: 0
  int32_t kind;     // SegKind
};

// Per-call segment header on the device (16 bytes).
struct CallHdr {
  int64_t len;   // elements
  int32_t kind;  // SegKind
  int32_t head;  // elements before the first aligned vector group; -1: no vector body
};
static_assert(sizeof(CallHdr) == 16, "CallHdr layout");

// Shard geometry of "The Endgame of FSDP Communication", Section 2.1, in
// elements: D_p rows of K_p, R_p = ceil(D_p / W) rows per rank, n_p = R_p K_p,
// o_p = sum_{i<p} n_i, S = sum_p n_p.
struct Geometry {
  int32_t world = 0;
  int32_t nparams = 0;
  std::vector<int64_t> D, K, R, n, o;
  int64_t S = 0;
};

tide_status build_geometry(int32_t world, int32_t nparams, const int32_t* ndims, const int64_t* dims,
                           Geometry* g, std::string* why);

// Real (non-padding) elements of parameter p in rank r's shard.
int64_t real_elems(const Geometry& g, int32_t p, int32_t r);

// Segment order decides which tensors the grid streams through at any moment
// (it works on a window of consecutive chunks).  Every operation is ordered so
// that its destination is written front to back: the reduce-scatter, copy-in
// and stock pack rank-major (r, then p: the slots of one destination rank are
// contiguous), the copy-out parameter-major (p, then r: the row blocks of one
// parameter are contiguous).  Measured on MI355X: one write stream per window
// beats one read stream per window by 3-5% on layers of many small tensors.
//  reduce-scatter: a kSum segment of the real elements and a kZero segment of
//    the padding elements of each (p, r) (each only when non-empty);
//  copy-out: a kCopy segment of the real elements of each (p, r).
//  copy-in: a kCopy segment of the real elements of each (p, r) (the kind
//    becomes kCast per call for fp32 shards) and a kZero segment of the
//    slot's padding.
//  stock pack (one rank's gradients into the rank-major fp32 buffer): a kCopy
//    (widening) segment of the rows of each (p, r) and a kZero segment of the
//    slot's padding.
std::vector<Seg> rs_segments(const Geometry& g);
std::vector<Seg> copyout_segments(const Geometry& g);
std::vector<Seg> copyin_segments(const Geometry& g);
std::vector<Seg> pack_segments(const Geometry& g);

// chunk_begin[s] = index of segment s's first chunk, chunk_begin[nseg] = total;
// segment s owns ceil(len / chunk) chunks.  Fails (TIDE_ERR_RANGE) when the
// total exceeds kMaxChunks.
tide_status chunk_table(const std::vector<Seg>& segs, int64_t chunk, std::vector<int32_t>* chunk_begin,
                        std::string* why);

// Options as given (0 = default) -> effective options for one operation.
tide_status check_options(const tide_options* in, tide_options* out, std::string* why);
tide_options effective_options(const tide_options& given, Op op, int32_t cu_count, int32_t world);

// Per-call tables.  Vector groups are 4 elements for the reduce-scatter
// (8-byte bf16 or 16-byte fp32 loads, 16-byte fp32 stores) and 8 elements for
// the copy-out (16-byte loads and stores).  A segment gets a vector body when
// every source and the destination reach their group alignment at the same
// element.
//  reduce-scatter: ptrs per segment = [W source pointers at the segment's
//    first element, destination pointer]; zero segments have null sources.
//    `grads` are uint16_t (bf16) or float pointers, as `f32` says.
//  copy-out: ptrs per segment = [source, destination].
void rs_call_table(const Geometry& g, const std::vector<Seg>& segs, const void* const* grads, bool f32,
                   float* const* out, std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs);
void co_call_table(const Geometry& g, const std::vector<Seg>& segs, const uint16_t* rank_major,
                   uint16_t* const* params, std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs);
//  copy-in: ptrs per segment = [shard (null for padding), destination];
//    groups are 4 elements for fp32 shards (16-byte loads, 8-byte stores), 8
//    for bf16 shards and for padding (16-byte accesses).
void ci_call_table(const Geometry& g, const std::vector<Seg>& segs, const void* const* shards, bool f32,
                   uint16_t* rank_major, std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs);
//  stock pack: ptrs per segment = [gradient (null for padding), destination];
//    groups of 4 elements (8-byte bf16 loads, 16-byte fp32 stores).
void pk_call_table(const Geometry& g, const std::vector<Seg>& segs, const uint16_t* const* grads, float* packed,
                   std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs);

// The chunks one launch covers, [first, end), and the segments they fall in,
// [seg, seg_end).  Long work is split into several launches: within one
// persistent launch the waves drift apart over time, widening the window of
// HBM they touch at once (measured on MI355X: one 17 GB reduce-scatter launch
// 5.85 TB/s, the same work in four launches 6.28 TB/s).
struct ChunkSpan {
  int32_t first, end, seg, seg_end;
};

// Device-side launch arguments (kernels.hip).
struct KernelArgs {
  const CallHdr* hdr;       // [nseg]
  const void* const* ptrs;  // [nseg * (nsrc + 1)]
  const int32_t* chunk_begin;  // [nseg + 1], nseg the operation's segment count
  int32_t nsrc;  // W (reduce-scatter) or 1 (the copies)
  int32_t nchunks;  // of the whole operation
  ChunkSpan span;   // of this launch
  int32_t chunk;    // elements per chunk
  uint32_t flags;
  float alpha;         // reduce-scatter only: Equation 5's scale
  int32_t accumulate;  // reduce-scatter only: add into the shards' old values
  bool realign = false;  // reduce-scatter only: some sum segment's sources are off the destination's phase
};

// The calling thread's error message (tide_last_error), shared by every
// source file of the C ABI.  set_error stores `msg` and returns `st`.
tide_status set_error(tide_status st, const std::string& msg);
void clear_error();

// Records a failure without allocating (for use where allocation failed).
tide_status set_error_nothrow(tide_status st, const char* msg) noexcept;

// Runs the body of a C-ABI entry point.  No C++ exception crosses the C ABI:
// a failed host allocation becomes TIDE_ERR_NOMEM, anything else thrown
// TIDE_ERR_INVALID, each with a message.
template <typename F>
tide_status guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return set_error_nothrow(TIDE_ERR_NOMEM, "out of host memory");
  } catch (...) {
    return set_error_nothrow(TIDE_ERR_INVALID, "unexpected host-side exception");
  }
}

// Device scratch of the allocation-free reduce-scatter: a file-scope device
// array of kScratchBytes (scratch.hip), one per device, holding the tables of
// the latest such call on that device.  Its tables are written by put
// launches, each carrying up to kPutWords 8-byte words as kernel arguments.
constexpr size_t kScratchBytes = TIDE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
constexpr uint32_t kPutWords = 500;
constexpr int kMaxDevices = 64;

// Address of the current device's scratch array (looked up once per device
// with hipGetSymbolAddress and kept); returns the hipError_t as int.
int scratch_address(void** out);
// Writes nwords (<= kPutWords) 8-byte words to dst (8-byte aligned) on
// `stream`; returns the launch status.
int launch_scratch_put(void* dst, const uint64_t* words, uint32_t nwords, void* stream);

// Launch with `grid` workgroups of kThreads on `stream`; returns the launch
// status (hipError_t as int).
int launch_rs_local(const KernelArgs& a, bool f32, int64_t grid, void* stream);
int launch_ag_copyout(const KernelArgs& a, int64_t grid, void* stream);
int launch_ag_copyin(const KernelArgs& a, bool f32, int64_t grid, void* stream);
int launch_stock_pack(const KernelArgs& a, int64_t grid, void* stream);

}  // namespace tide
