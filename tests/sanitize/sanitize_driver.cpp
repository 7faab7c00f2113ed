// Host-only checks of the CPU oracle (oracle/tide_oracle.c) and the host
// shard-layout planner (param_collectives_amd/csrc/plan.cpp), built together
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py.  Test infrastructure: it links both sides only to
// compare them; neither side uses the other.
//
// On random layouts (world sizes 1..256, 1-3 dimensional parameters, empty
// and ragged ones, fewer rows than ranks) it checks that
//   - the planner's geometry equals the oracle's (Section 2.1 of "The Endgame
//     of FSDP Communication": R_p, n_p, o_p, S, n_real);
//   - every operation's segments tile its destination exactly once and read
//     only real rows of their sources;
//   - the chunk tables and per-call tables stay inside the tensors they
//     describe, for source pointers at every 2-byte phase;
//   - the reduce-scatter computed by walking the planner's segments equals
//     the oracle's, bit for bit, and the oracle's threaded runs equal its
//     single-threaded ones;
//   - the oracle's other operations (copy-out, pack, copy-in, Equation 5,
//     stock pack, cast, victim) run clean and satisfy their round trips;
//   - invalid arguments are rejected without touching memory.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "tide_internal.h"

extern "C" {
int oracle_plan(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, int64_t* D, int64_t* K, int64_t* R,
                int64_t* n, int64_t* o, int64_t* S, int64_t* n_real, int64_t* rank_major_offset,
                int64_t* landing_offset);
int oracle_rs_local(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* const* grads,
                    float* const* out, int32_t nthreads);
int oracle_copyout(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* rank_major,
                   uint16_t* const* params, int32_t nthreads);
int oracle_pack(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* const* params,
                uint16_t* rank_major, int32_t nthreads);
int oracle_copyin(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const void* const* shards,
                  int32_t shard_dtype, uint16_t* rank_major, int32_t nthreads);
int oracle_cast_bf16(const float* x, int64_t n, uint16_t* out);
int oracle_rs_local_ex(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const void* const* grads,
                       int32_t grad_dtype, float alpha, int32_t accumulate, float* const* out, int32_t nthreads);
int oracle_chunk_cat(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* const* grads,
                     float* packed, int32_t nthreads);
int oracle_axpb(int64_t n, const float* x, float a, float b, float* y);
}

namespace {

int g_failures = 0;

void expect(bool ok, const std::string& what) {
  if (!ok) {
    if (g_failures < 20) std::fprintf(stderr, "FAIL: %s\n", what.c_str());
    ++g_failures;
  }
}

// splitmix64: the cases' seeded random source
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  int64_t below(int64_t n) { return int64_t(next() % uint64_t(n)); }
};

float widen(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint32_t bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// finite bf16 values of moderate size (no NaN, so that bitwise equality is the test)
uint16_t rand_bf16(Rng& r) {
  const uint16_t sign = uint16_t(r.below(2) << 15);
  const uint16_t exp = uint16_t(100 + r.below(50));
  return uint16_t(sign | (exp << 7) | uint16_t(r.below(128)));
}

struct Case {
  int32_t W = 1;
  std::vector<int32_t> ndims;
  std::vector<int64_t> dims;
  int32_t P() const { return int32_t(ndims.size()); }
};

Case make_case(Rng& r, int idx) {
  static const int32_t worlds[] = {1, 2, 3, 4, 5, 7, 8, 9, 16, 33, 256};
  Case c;
  c.W = worlds[idx % int(sizeof(worlds) / sizeof(worlds[0]))];
  const bool wide = c.W > 16;  // keep the large world sizes small in elements
  const int32_t P = int32_t(1 + r.below(wide ? 3 : 7));
  for (int32_t p = 0; p < P; ++p) {
    const int32_t nd = int32_t(1 + r.below(3));
    c.ndims.push_back(nd);
    int64_t rows;
    switch (r.below(5)) {
      case 0: rows = 0; break;                                  // empty
      case 1: rows = 1 + r.below(c.W);                          // fewer rows than ranks (or equal)
      default: rows = r.below(wide ? c.W + 9 : 3 * c.W + 40);   // ragged
    }
    c.dims.push_back(rows);
    for (int32_t j = 1; j < nd; ++j) c.dims.push_back(r.below(6) == 0 ? 0 : 1 + r.below(5));
  }
  return c;
}

void check_case(const Case& c, Rng& r, int idx) {
  const int32_t W = c.W, P = c.P();
  const std::string tag = "case " + std::to_string(idx) + " (W=" + std::to_string(W) + ", P=" + std::to_string(P) + ")";
  // geometry: planner against oracle
  tide::Geometry g;
  std::string why;
  expect(tide::build_geometry(W, P, c.ndims.data(), c.dims.data(), &g, &why) == TIDE_OK, tag + ": planner " + why);
  std::vector<int64_t> D(P), K(P), R(P), n(P), o(P), nr(size_t(P) * W), rmo(size_t(P) * W), land(size_t(P) * W);
  int64_t S = -1;
  expect(oracle_plan(W, P, c.ndims.data(), c.dims.data(), D.data(), K.data(), R.data(), n.data(), o.data(), &S,
                     nr.data(), rmo.data(), land.data()) == 0, tag + ": oracle_plan");
  expect(S == g.S, tag + ": S");
  for (int32_t p = 0; p < P; ++p) {
    expect(D[p] == g.D[p] && K[p] == g.K[p] && R[p] == g.R[p] && n[p] == g.n[p] && o[p] == g.o[p],
           tag + ": geometry of parameter " + std::to_string(p));
    for (int32_t q = 0; q < W; ++q)
      expect(nr[size_t(p) * W + q] == tide::real_elems(g, p, q), tag + ": n_real");
  }

  // segments tile their destinations once and read only real rows
  const auto rs = tide::rs_segments(g);
  std::vector<std::vector<int>> cover(W, std::vector<int>(size_t(S), 0));
  for (const auto& s : rs) {
    expect(s.len > 0 && s.dst_off >= 0 && s.dst_off + s.len <= S, tag + ": rs segment range");
    if (s.dst_off < 0 || s.dst_off + s.len > S) continue;
    for (int64_t e = 0; e < s.len; ++e) ++cover[s.dst_idx][size_t(s.dst_off + e)];
    if (s.kind == tide::kSum)
      expect(s.src_off >= 0 && s.src_off + s.len <= g.D[s.src_idx] * g.K[s.src_idx], tag + ": rs source range");
  }
  for (int32_t q = 0; q < W; ++q)
    for (int64_t e = 0; e < S; ++e) expect(cover[q][size_t(e)] == 1, tag + ": rs output written once");
  const auto co = tide::copyout_segments(g);
  for (int32_t p = 0; p < P; ++p) {
    std::vector<int> pc(size_t(g.D[p] * g.K[p]), 0);
    for (const auto& s : co) {
      if (s.dst_idx != p) continue;
      expect(s.dst_off >= 0 && s.dst_off + s.len <= int64_t(pc.size()), tag + ": copy-out range");
      if (s.dst_off < 0 || s.dst_off + s.len > int64_t(pc.size())) continue;
      for (int64_t e = 0; e < s.len; ++e) ++pc[size_t(s.dst_off + e)];
      const int64_t q = s.dst_off / (g.n[p] > 0 ? g.n[p] : 1);
      expect(s.src_off == q * g.S + g.o[p] && s.len == tide::real_elems(g, p, int32_t(q)),
             tag + ": copy-out reads only the real part of slot (r, p)");
    }
    for (int v : pc) expect(v == 1, tag + ": copy-out parameter written once");
  }
  const std::vector<tide::Seg> rank_major_ops[2] = {tide::copyin_segments(g), tide::pack_segments(g)};
  for (const auto& segs : rank_major_ops) {
    std::vector<int> rc(size_t(W * S), 0);
    for (const auto& s : segs) {
      expect(s.dst_off >= 0 && s.dst_off + s.len <= W * S, tag + ": rank-major range");
      if (s.dst_off < 0 || s.dst_off + s.len > W * S) continue;
      for (int64_t e = 0; e < s.len; ++e) ++rc[size_t(s.dst_off + e)];
    }
    for (int v : rc) expect(v == 1, tag + ": rank-major buffer written once");
  }

  // chunk tables
  for (int64_t chunk : {8, 24, 1024}) {
    std::vector<int32_t> cb;
    expect(tide::chunk_table(rs, chunk, &cb, &why) == TIDE_OK, tag + ": chunk table");
    int64_t want = 0;
    for (size_t s = 0; s < rs.size(); ++s) {
      expect(cb[s] == want, tag + ": chunk_begin");
      want += (rs[s].len + chunk - 1) / chunk;
    }
    expect(cb.back() == want, tag + ": chunk total");
  }

  // per-call tables over stand-in addresses (never dereferenced): every
  // pointer with its segment's length stays inside its tensor
  const uintptr_t base = uintptr_t(1) << 40;
  std::vector<uintptr_t> gstart(size_t(W) * P), gend(size_t(W) * P);
  std::vector<const void*> gp(size_t(W) * P);
  const uintptr_t phase = uintptr_t(2 * r.below(8));  // all ranks at one 2-byte phase
  uintptr_t at = base;
  for (int32_t u = 0; u < W; ++u)
    for (int32_t p = 0; p < P; ++p) {
      const size_t i = size_t(u) * P + p;
      gstart[i] = at + phase;
      gend[i] = gstart[i] + uintptr_t(g.D[p] * g.K[p]) * 2;
      gp[i] = reinterpret_cast<const void*>(gstart[i]);
      at += (uintptr_t(g.D[p] * g.K[p]) * 4 + 256) & ~uintptr_t(255);
    }
  std::vector<float*> outp(W);
  for (int32_t q = 0; q < W; ++q) {
    outp[q] = reinterpret_cast<float*>(at + 4 * uintptr_t(r.below(4)));
    at += (uintptr_t(S) * 4 + 512) & ~uintptr_t(255);
  }
  std::vector<tide::CallHdr> hdr;
  std::vector<const void*> ptrs;
  tide::rs_call_table(g, rs, gp.data(), false, outp.data(), &hdr, &ptrs);
  expect(hdr.size() == rs.size() && ptrs.size() == rs.size() * size_t(W + 1), tag + ": call table size");
  for (size_t s = 0; s < rs.size() && s < hdr.size(); ++s) {
    const auto& sg = rs[s];
    expect(hdr[s].len == sg.len && hdr[s].kind == sg.kind && hdr[s].head < 4, tag + ": call header");
    if (hdr[s].head >= 0 && hdr[s].head < sg.len)  // the vector body starts where the destination is 16-byte aligned
      expect(((reinterpret_cast<uintptr_t>(ptrs[s * (W + 1) + W]) + uintptr_t(hdr[s].head) * 4) & 15) == 0,
             tag + ": vector body on a 16-byte destination boundary");
    const uintptr_t d = reinterpret_cast<uintptr_t>(ptrs[s * (W + 1) + W]);
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(outp[sg.dst_idx]);
    expect(d >= d0 && d + uintptr_t(sg.len) * 4 <= d0 + uintptr_t(S) * 4, tag + ": destination pointer range");
    if (sg.kind != tide::kSum) continue;
    for (int32_t u = 0; u < W; ++u) {
      const size_t i = size_t(u) * P + sg.src_idx;
      const uintptr_t a = reinterpret_cast<uintptr_t>(ptrs[s * (W + 1) + u]);
      expect(a >= gstart[i] && a + uintptr_t(sg.len) * 2 <= gend[i], tag + ": source pointer range");
    }
  }

  // values: the reduce-scatter by walking the planner's segments equals the oracle's
  std::vector<std::vector<uint16_t>> G(size_t(W) * P);
  std::vector<const uint16_t*> gptr(size_t(W) * P);
  for (size_t i = 0; i < G.size(); ++i) {
    const int32_t p = int32_t(i % size_t(P));
    G[i].resize(size_t(g.D[p] * g.K[p]) + 1);
    for (auto& v : G[i]) v = rand_bf16(r);
    gptr[i] = G[i].data();
  }
  std::vector<std::vector<float>> want(W, std::vector<float>(size_t(S) + 1)), one(W, std::vector<float>(size_t(S) + 1));
  std::vector<float*> wp(W), op(W);
  for (int32_t q = 0; q < W; ++q) {
    wp[q] = want[q].data();
    op[q] = one[q].data();
  }
  expect(oracle_rs_local(W, P, c.ndims.data(), c.dims.data(), gptr.data(), wp.data(), 3) == 0, tag + ": oracle rs");
  expect(oracle_rs_local(W, P, c.ndims.data(), c.dims.data(), gptr.data(), op.data(), 1) == 0, tag + ": oracle rs 1");
  std::vector<std::vector<float>> walk(W, std::vector<float>(size_t(S), NAN));
  for (const auto& s : rs)
    for (int64_t e = 0; e < s.len; ++e) {
      float acc = 0.0f;
      if (s.kind == tide::kSum) {
        acc = widen(G[size_t(s.src_idx)][size_t(s.src_off + e)]);
        for (int32_t u = 1; u < W; ++u) acc = acc + widen(G[size_t(u) * P + s.src_idx][size_t(s.src_off + e)]);
      }
      walk[s.dst_idx][size_t(s.dst_off + e)] = acc;
    }
  for (int32_t q = 0; q < W; ++q)
    for (int64_t e = 0; e < S; ++e) {
      expect(bits(walk[q][size_t(e)]) == bits(want[q][size_t(e)]), tag + ": segment walk equals the oracle");
      expect(bits(one[q][size_t(e)]) == bits(want[q][size_t(e)]), tag + ": thread-count invariance");
    }

  // the oracle's other operations, with their round trips
  std::vector<std::vector<uint16_t>> X(P);
  std::vector<const uint16_t*> xp(P);
  std::vector<uint16_t*> xo(P);
  std::vector<std::vector<uint16_t>> back(P);
  for (int32_t p = 0; p < P; ++p) {
    X[p].resize(size_t(g.D[p] * g.K[p]) + 1);
    for (auto& v : X[p]) v = rand_bf16(r);
    back[p].assign(X[p].size(), 0xFFFF);
    xp[p] = X[p].data();
    xo[p] = back[p].data();
  }
  std::vector<uint16_t> rm(size_t(W * S) + 1, 0xFFFF), rm2(size_t(W * S) + 1, 0xFFFF);
  expect(oracle_pack(W, P, c.ndims.data(), c.dims.data(), xp.data(), rm.data(), 2) == 0, tag + ": pack");
  expect(oracle_copyout(W, P, c.ndims.data(), c.dims.data(), rm.data(), xo.data(), 2) == 0, tag + ": copy-out");
  for (int32_t p = 0; p < P; ++p)
    for (int64_t e = 0; e < g.D[p] * g.K[p]; ++e) expect(back[p][size_t(e)] == X[p][size_t(e)], tag + ": round trip");
  std::vector<std::vector<uint16_t>> shards(size_t(W) * P);
  std::vector<const void*> sp(size_t(W) * P);
  for (int32_t q = 0; q < W; ++q)
    for (int32_t p = 0; p < P; ++p) {
      const int64_t real = tide::real_elems(g, p, q), first = int64_t(q) * g.R[p] * g.K[p];
      auto& sh = shards[size_t(q) * P + p];
      sh.assign(X[p].begin() + (real > 0 ? first : 0), X[p].begin() + (real > 0 ? first + real : 0));
      sh.push_back(0);
      sp[size_t(q) * P + p] = sh.data();
    }
  expect(oracle_copyin(W, P, c.ndims.data(), c.dims.data(), sp.data(), 0, rm2.data(), 2) == 0, tag + ": copy-in");
  for (int64_t e = 0; e < W * S; ++e) expect(rm2[size_t(e)] == rm[size_t(e)], tag + ": copy-in equals pack");
  std::vector<std::vector<float>> acc(W, std::vector<float>(size_t(S) + 1, 1.5f));
  std::vector<float*> ap(W);
  for (int32_t q = 0; q < W; ++q) ap[q] = acc[q].data();
  std::vector<const void*> gv(gptr.begin(), gptr.end());
  expect(oracle_rs_local_ex(W, P, c.ndims.data(), c.dims.data(), gv.data(), 0, 0.5f, 1, ap.data(), 2) == 0,
         tag + ": Equation 5");
  std::vector<float> packed(size_t(W * S) + 1);
  std::vector<const uint16_t*> g0(gptr.begin(), gptr.begin() + P);
  expect(oracle_chunk_cat(W, P, c.ndims.data(), c.dims.data(), g0.data(), packed.data(), 2) == 0, tag + ": chunk_cat");
}

void check_errors() {
  const int32_t nd[2] = {1, 0};
  const int64_t dims[2] = {-3, 4};
  tide::Geometry g;
  std::string why;
  expect(tide::build_geometry(0, 1, nd, dims, &g, &why) == TIDE_ERR_INVALID, "W = 0 rejected");
  expect(tide::build_geometry(2, 1, nd, dims, &g, &why) == TIDE_ERR_INVALID, "negative dimension rejected");
  expect(tide::build_geometry(2, 2, nd, dims, &g, &why) != TIDE_OK, "0-d parameter rejected");
  const int64_t huge[1] = {int64_t(1) << 62};
  expect(tide::build_geometry(4, 1, nd, huge, &g, &why) == TIDE_ERR_RANGE, "overflow rejected");
  int64_t out[16] = {0};
  expect(oracle_plan(0, 1, nd, dims, out, out, out, out, out, out, out, out, out) != 0, "oracle W = 0 rejected");
  expect(oracle_axpb(-1, nullptr, 1.0f, 0.0f, nullptr) != 0, "oracle negative length rejected");
  expect(oracle_cast_bf16(nullptr, 4, nullptr) != 0, "oracle null cast rejected");
  tide_options in{0, 0, 12, 0, 0}, o;
  expect(tide::check_options(&in, &o, &why) == TIDE_ERR_INVALID, "chunk not a multiple of 8 rejected");
}

void check_cast_and_victim() {
  std::vector<float> x = {1.0f, -0.0f, 3.4e38f, 1e-40f, NAN, -INFINITY, 1.00390625f, 1.01171875f};
  std::vector<uint16_t> b(x.size());
  expect(oracle_cast_bf16(x.data(), int64_t(x.size()), b.data()) == 0, "cast");
  expect(b[0] == 0x3F80 && b[1] == 0x8000 && b[5] == 0xFF80, "cast values");
  expect(b[6] == 0x3F80 && b[7] == 0x3F82, "cast ties to even");
  std::vector<float> y(x.size());
  expect(oracle_axpb(int64_t(x.size()), x.data(), 2.0f, 1.0f, y.data()) == 0, "victim");
  expect(y[0] == 3.0f, "victim value");
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 300;
  Rng r{20261203};
  for (int i = 0; i < cases; ++i) check_case(make_case(r, i), r, i);
  check_errors();
  check_cast_and_victim();
  if (g_failures) {
    std::fprintf(stderr, "%d failures\n", g_failures);
    return 1;
  }
  std::printf("sanitize driver: %d cases clean\n", cases);
  return 0;
}
