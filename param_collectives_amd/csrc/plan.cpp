// Host shard-layout planner: the dimension-0 shard geometry of "The Endgame of
// FSDP Communication" (Wang et al.), Section 2.1, turned into the segment
// table the kernels walk.  The placement is decided here once per plan, so a
// call only passes tensor pointers (as in Section 6, where the kernels take
// the gradient pointers as arguments and the segment table is uploaded once,
// when the buffers are registered).
#include <string>
#include <vector>

#include "tide_internal.h"

namespace tide {

tide_status build_geometry(int32_t world, int32_t nparams, const int32_t* ndims, const int64_t* dims,
                           Geometry* g, std::string* why) {
  if (world < 1 || world > TIDE_MAX_WORLD) {
    *why = "world must be in [1, " + std::to_string(TIDE_MAX_WORLD) + "], got " + std::to_string(world);
    return TIDE_ERR_INVALID;
  }
  if (nparams < 1) {
    *why = "nparams must be >= 1, got " + std::to_string(nparams);
    return TIDE_ERR_INVALID;
  }
  if (ndims == nullptr || dims == nullptr) {
    *why = "ndims and dims must not be NULL";
    return TIDE_ERR_INVALID;
  }
  g->world = world;
  g->nparams = nparams;
  g->D.assign(nparams, 0);
  g->K.assign(nparams, 0);
  g->R.assign(nparams, 0);
  g->n.assign(nparams, 0);
  g->o.assign(nparams, 0);
  int64_t pos = 0, offset = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    if (ndims[p] < 1) {
      *why = "parameter " + std::to_string(p) + " has " + std::to_string(ndims[p]) +
             " dimensions; at least 1 is required";
      return TIDE_ERR_INVALID;
    }
    int64_t rows = dims[pos];
    int64_t row_len = 1;
    for (int32_t j = 0; j < ndims[p]; ++j) {
      if (dims[pos + j] < 0) {
        *why = "parameter " + std::to_string(p) + " has a negative dimension";
        return TIDE_ERR_INVALID;
      }
      if (j > 0 && __builtin_mul_overflow(row_len, dims[pos + j], &row_len)) {
        *why = "parameter " + std::to_string(p) + " is too large";
        return TIDE_ERR_RANGE;
      }
    }
    pos += ndims[p];
    int64_t numel, shard;
    const int64_t rows_per_rank = rows / world + (rows % world != 0);
    if (__builtin_mul_overflow(rows, row_len, &numel) ||
        __builtin_mul_overflow(rows_per_rank, row_len, &shard) ||
        __builtin_mul_overflow(shard, int64_t(world), &numel)) {
      *why = "parameter " + std::to_string(p) + " is too large";
      return TIDE_ERR_RANGE;
    }
    g->D[p] = rows;
    g->K[p] = row_len;
    g->R[p] = rows_per_rank;
    g->n[p] = shard;
    g->o[p] = offset;
    if (__builtin_add_overflow(offset, shard, &offset)) {
      *why = "the per-rank shard overflows int64";
      return TIDE_ERR_RANGE;
    }
  }
  int64_t whole;
  // Every element offset (at most W * S) is later scaled to bytes, by up to 4.
  if (__builtin_mul_overflow(offset, int64_t(world), &whole) || whole > INT64_MAX / 4) {
    *why = "W * S elements exceed 2^61";
    return TIDE_ERR_RANGE;
  }
  g->S = offset;
  return TIDE_OK;
}

int64_t real_elems(const Geometry& g, int32_t p, int32_t r) {
  const int64_t first_row = int64_t(r) * g.R[p];
  int64_t rows = g.D[p] - first_row;
  if (rows < 0) rows = 0;
  if (rows > g.R[p]) rows = g.R[p];
  return rows * g.K[p];
}

std::vector<Seg> rs_segments(const Geometry& g) {
  std::vector<Seg> segs;
  for (int32_t r = 0; r < g.world; ++r) {
    for (int32_t p = 0; p < g.nparams; ++p) {
      const int64_t real = real_elems(g, p, r);
      const int64_t src = int64_t(r) * g.n[p];  // first element of rows [r R_p, ...) in G_p
      if (real > 0) segs.push_back(Seg{src, g.o[p], real, p, r, kSum});
      if (g.n[p] > real) segs.push_back(Seg{0, g.o[p] + real, g.n[p] - real, p, r, kZero});
    }
  }
  return segs;
}

std::vector<Seg> copyout_segments(const Geometry& g) {
  std::vector<Seg> segs;
  for (int32_t p = 0; p < g.nparams; ++p) {
    for (int32_t r = 0; r < g.world; ++r) {
      const int64_t real = real_elems(g, p, r);
      if (real > 0) segs.push_back(Seg{int64_t(r) * g.S + g.o[p], int64_t(r) * g.n[p], real, 0, p, kCopy});
    }
  }
  return segs;
}

std::vector<Seg> copyin_segments(const Geometry& g) {
  std::vector<Seg> segs;
  for (int32_t r = 0; r < g.world; ++r) {
    for (int32_t p = 0; p < g.nparams; ++p) {
      const int64_t real = real_elems(g, p, r);
      const int64_t slot = int64_t(r) * g.S + g.o[p];
      const int32_t shard = r * g.nparams + p;
      if (real > 0) segs.push_back(Seg{0, slot, real, shard, 0, kCopy});
      if (g.n[p] > real) segs.push_back(Seg{0, slot + real, g.n[p] - real, shard, 0, kZero});
    }
  }
  return segs;
}

std::vector<Seg> pack_segments(const Geometry& g) {
  std::vector<Seg> segs;
  for (int32_t r = 0; r < g.world; ++r) {
    for (int32_t p = 0; p < g.nparams; ++p) {
      const int64_t real = real_elems(g, p, r);
      const int64_t slot = int64_t(r) * g.S + g.o[p];
      if (real > 0) segs.push_back(Seg{int64_t(r) * g.n[p], slot, real, p, 0, kCopy});
      if (g.n[p] > real) segs.push_back(Seg{0, slot + real, g.n[p] - real, p, 0, kZero});
    }
  }
  return segs;
}

tide_status chunk_table(const std::vector<Seg>& segs, int64_t chunk, std::vector<int32_t>* chunk_begin,
                        std::string* why) {
  chunk_begin->assign(segs.size() + 1, 0);
  int64_t total = 0;
  for (size_t s = 0; s < segs.size(); ++s) {
    (*chunk_begin)[s] = int32_t(total);
    total += segs[s].len / chunk + (segs[s].len % chunk != 0);
    if (total > kMaxChunks) {
      *why = "more than 2^30 chunks: use a larger chunk_elems";
      return TIDE_ERR_RANGE;
    }
  }
  (*chunk_begin)[segs.size()] = int32_t(total);
  return TIDE_OK;
}

tide_status check_options(const tide_options* in, tide_options* out, std::string* why) {
  tide_options o{0, 0, 0, 0, 0};
  if (in) o = *in;
  if (o.cu_budget < 0 || o.wg_per_cu < 0 || o.chunk_elems < 0 || o.wave_chunks < 0) {
    *why = "tide_options fields must be >= 0";
    return TIDE_ERR_INVALID;
  }
  if (o.wave_chunks > kMaxWaveChunks) {
    *why = "wave_chunks must be at most 2^30";
    return TIDE_ERR_INVALID;
  }
  if (o.chunk_elems % 8 != 0 || o.chunk_elems > kMaxChunk) {
    *why = "chunk_elems must be a multiple of 8 and at most 2^28";
    return TIDE_ERR_INVALID;
  }
  if (o.wg_per_cu > 64) {
    *why = "wg_per_cu must be at most 64";
    return TIDE_ERR_RANGE;
  }
  if (o.flags & ~(TIDE_FLAG_CACHED_LOADS | TIDE_FLAG_CACHED_STORES | TIDE_FLAG_NO_LDS)) {
    *why = "unknown bits in tide_options.flags";
    return TIDE_ERR_INVALID;
  }
  *out = o;
  return TIDE_OK;
}

tide_options effective_options(const tide_options& given, Op op, int32_t cu_count, int32_t world) {
  tide_options o = given;
  if (o.cu_budget == 0) o.cu_budget = cu_count;
  const int32_t wg[kNumOps] = {kRsWgPerCu, kCoWgPerCu, kCiWgPerCu, kPkWgPerCu, kRsF32WgPerCu};
  const int64_t chunk[kNumOps] = {world <= 3 ? kRsChunkFewRanks : kRsChunk, kCoChunk, kCiChunk, kPkChunk, kRsF32Chunk};
  if (o.wg_per_cu == 0) o.wg_per_cu = wg[op];
  if (o.chunk_elems == 0) o.chunk_elems = chunk[op];
  if (o.wave_chunks == 0) o.wave_chunks = kWaveChunks;
  return o;
}

namespace {

// Elements to skip from `addr` (an element address of `esize` bytes) until it
// is `align`-byte aligned.
int64_t skip_to(uintptr_t addr, int64_t esize, uintptr_t align) {
  return int64_t(((align - (addr & (align - 1))) & (align - 1)) / uintptr_t(esize));
}

}  // namespace

void rs_call_table(const Geometry& g, const std::vector<Seg>& segs, const void* const* grads, bool f32,
                   float* const* out, std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs) {
  const int32_t W = g.world, P = g.nparams;
  // a vector group of 4 elements: 8-byte bf16 or 16-byte fp32 source loads
  const int64_t esize = f32 ? 4 : 2;
  const uintptr_t salign = uintptr_t(4 * esize);
  hdr->resize(segs.size());
  ptrs->assign(segs.size() * size_t(W + 1), nullptr);
  for (size_t s = 0; s < segs.size(); ++s) {
    const Seg& sg = segs[s];
    const void** row = ptrs->data() + s * size_t(W + 1);
    float* dst = out[sg.dst_idx] + sg.dst_off;
    row[W] = dst;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
    int32_t head = -1;
    if (sg.kind == kZero) {
      head = int32_t(skip_to(d, 4, 16));  // 16-byte zero stores
    } else {
      // source loads of one group and 16-byte destination stores
      const uintptr_t s0 = reinterpret_cast<uintptr_t>(grads[sg.src_idx]) + uintptr_t(sg.src_off * esize);
      const uintptr_t phase = s0 & (salign - 1);
      bool same = true;
      for (int32_t u = 0; u < W; ++u) {
        const uintptr_t su = reinterpret_cast<uintptr_t>(grads[int64_t(u) * P + sg.src_idx]) +
                             uintptr_t(sg.src_off * esize);
        row[u] = reinterpret_cast<const void*>(su);
        same = same && (su & (salign - 1)) == phase;
      }
      // the vector body starts where the destination is 16-byte aligned; the
      // kernel realigns sources at another phase there, provided all W share
      // one phase (else the segment goes element by element)
      if (same) head = int32_t(skip_to(d, 4, 16));
    }
    (*hdr)[s] = CallHdr{sg.len, sg.kind, head};
  }
}

void co_call_table(const Geometry& g, const std::vector<Seg>& segs, const uint16_t* rank_major,
                   uint16_t* const* params, std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs) {
  (void)g;
  hdr->resize(segs.size());
  ptrs->assign(segs.size() * 2, nullptr);
  for (size_t s = 0; s < segs.size(); ++s) {
    const Seg& sg = segs[s];
    const uint16_t* src = rank_major + sg.src_off;
    uint16_t* dst = params[sg.dst_idx] + sg.dst_off;
    (*ptrs)[2 * s] = src;
    (*ptrs)[2 * s + 1] = dst;
    // the vector body starts where the destination is 16-byte aligned; a
    // source at another phase there takes the kernel's realigned body
    const int32_t head = int32_t(skip_to(reinterpret_cast<uintptr_t>(dst), 2, 16));
    (*hdr)[s] = CallHdr{sg.len, sg.kind, head};
  }
}

void ci_call_table(const Geometry& g, const std::vector<Seg>& segs, const void* const* shards, bool f32,
                   uint16_t* rank_major, std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs) {
  (void)g;
  hdr->resize(segs.size());
  ptrs->assign(segs.size() * 2, nullptr);
  for (size_t s = 0; s < segs.size(); ++s) {
    const Seg& sg = segs[s];
    uint16_t* dst = rank_major + sg.dst_off;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
    (*ptrs)[2 * s + 1] = dst;
    int32_t kind = sg.kind, head = -1;
    if (sg.kind == kZero) {
      head = int32_t(skip_to(d, 2, 16));  // 16-byte zero stores
    } else if (f32) {
      kind = kCast;
      const float* src = static_cast<const float*>(shards[sg.src_idx]) + sg.src_off;
      (*ptrs)[2 * s] = src;
      // 16-byte fp32 loads feeding 8-byte bf16 stores: 4 elements; the body
      // starts where the destination is 8-byte aligned (a source at another
      // 16-byte phase there takes the kernel's realigned body)
      head = int32_t(skip_to(d, 2, 8));
    } else {
      const uint16_t* src = static_cast<const uint16_t*>(shards[sg.src_idx]) + sg.src_off;
      (*ptrs)[2 * s] = src;
      head = int32_t(skip_to(d, 2, 16));  // as for the copy-out
    }
    (*hdr)[s] = CallHdr{sg.len, kind, head};
  }
}

void pk_call_table(const Geometry& g, const std::vector<Seg>& segs, const uint16_t* const* grads, float* packed,
                   std::vector<CallHdr>* hdr, std::vector<const void*>* ptrs) {
  (void)g;
  hdr->resize(segs.size());
  ptrs->assign(segs.size() * 2, nullptr);
  for (size_t s = 0; s < segs.size(); ++s) {
    const Seg& sg = segs[s];
    float* dst = packed + sg.dst_off;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
    (*ptrs)[2 * s + 1] = dst;
    int32_t head = -1;
    if (sg.kind == kZero) {
      head = int32_t(skip_to(d, 4, 16));  // 16-byte zero stores
    } else {
      const uint16_t* src = grads[sg.src_idx] + sg.src_off;
      (*ptrs)[2 * s] = src;
      // 8-byte bf16 loads feeding 16-byte fp32 stores: 4 elements
      const int64_t h = skip_to(reinterpret_cast<uintptr_t>(src), 2, 8);
      if (((d + uintptr_t(4 * h)) & 15) == 0) head = int32_t(h);
    }
    (*hdr)[s] = CallHdr{sg.len, sg.kind, head};
  }
}

}  // namespace tide
