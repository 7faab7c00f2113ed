// Private types shared by the host planner (plan.cpp) and the device code
// (tide.hip) of the layout-aware FSDP2 collective local stages.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "tide.h"

namespace tide {

constexpr int kThreads = 256;              // threads per workgroup (four wave64s)
constexpr int32_t kDefaultWgPerCu = 8;      // 2048 threads per CU: full occupancy at <= 64 VGPRs
constexpr int64_t kDefaultChunk = 4096;     // elements per chunk
constexpr int64_t kMaxChunk = int64_t(1) << 30;

enum SegKind : int32_t { kSum = 0, kZero = 1, kCopy = 2 };

// One contiguous run of work.  Device layout: 48 bytes, naturally aligned.
struct Seg {
  int64_t src_off;      // element offset into each source tensor
  int64_t dst_off;      // element offset into the destination tensor
  int64_t len;          // elements, > 0
  int64_t chunk_begin;  // index of this segment's first chunk in the plan
  int32_t src_idx;      // reduce-scatter: parameter p; copy-out: 0
  int32_t dst_idx;      // reduce-scatter: destination rank r; copy-out: parameter p
  int32_t kind;         // SegKind
  int32_t reserved;     // 0
};
static_assert(sizeof(Seg) == 48, "Seg layout");

// Shard geometry of "The Endgame of FSDP Communication", Section 2.1, in
// elements: D_p rows of K_p, R_p = ceil(D_p / W) rows per rank, n_p = R_p K_p,
// o_p = sum_{i<p} n_i, S = sum_p n_p.
struct Geometry {
  int32_t world = 0;
  int32_t nparams = 0;
  std::vector<int64_t> D, K, R, n, o;
  int64_t S = 0;
};

// Builds the geometry; returns TIDE_OK or an error with `why` filled in.
tide_status build_geometry(int32_t world, int32_t nparams, const int32_t* ndims, const int64_t* dims,
                           Geometry* g, std::string* why);

// Real (non-padding) elements of parameter p in rank r's shard.
int64_t real_elems(const Geometry& g, int32_t p, int32_t r);

// Segment lists (chunk fields left 0; see assign_chunks).
//  reduce-scatter: for r, then p: a kSum segment of the real elements and a
//    kZero segment of the padding elements (each only when non-empty);
//  copy-out: for r, then p: a kCopy segment of the real elements.
std::vector<Seg> rs_segments(const Geometry& g);
std::vector<Seg> copyout_segments(const Geometry& g);

// Chunk split for a chunk size: segment s owns chunks [chunk_begin,
// chunk_begin + ceil(len / chunk)); returns the total number of chunks.
int64_t assign_chunks(std::vector<Seg>* segs, int64_t chunk);

// Resolve defaults and check ranges; returns TIDE_OK or an error with `why`.
tide_status resolve_options(const tide_options* in, tide_options* out, std::string* why);

}  // namespace tide
