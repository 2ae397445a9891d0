// CPU check of the stage-3 gather's indexing, built with g++ from the same
// gather_plan.h the kernel compiles: every launch of a gather is planned as the
// library plans it, every workgroup of every launch recovers its piece as the
// kernel does, and the test checks, against the definition of the gather (flat
// index i lives in row i / S at column i mod S):
//  - the pieces of the launches tile [lo, lo + n) in order, one per rank shard;
//  - every piece's workgroups are hit exactly once, no workgroup beyond them;
//  - every vector access is aligned to its width on both sides and lies inside
//    its piece; the loose head and tail lie inside it too;
//  - on small cases, every output element is written exactly once, from its
//    owner's element (element by element).
// Addresses are never dereferenced: buffers are stand-in base addresses.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "gather_plan.h"

using zero::GatherArgs;
using zero::GatherLaunch;
using zero::GatherPiece;

static int g_fail = 0;
#define EXPECT(c, ...)                                                          \
  do {                                                                          \
    if (!(c)) {                                                                 \
      if (g_fail < 20) {                                                        \
        fprintf(stderr, "%s:%d: %s: ", __FILE__, __LINE__, #c);                 \
        fprintf(stderr, __VA_ARGS__);                                           \
        fprintf(stderr, "\n");                                                  \
      }                                                                         \
      ++g_fail;                                                                 \
    }                                                                           \
  } while (0)

struct Case {
  uint64_t psi, nd, pad, lo, n;
  uintptr_t shards_base, out_base;
};

static void check(const Case& c, bool elementwise) {
  const uint64_t s = c.psi / c.nd + (c.psi % c.nd != 0);
  const uint64_t stride = s + c.pad;
  GatherLaunch g;
  g.shards = reinterpret_cast<const uint16_t*>(c.shards_base);
  g.stride = stride;
  g.s = s;
  g.lo = c.lo;
  g.n = c.n;
  g.out = reinterpret_cast<uint16_t*>(c.out_base);
  std::vector<uint8_t> hits(elementwise ? c.n : 0, 0);
  const uint64_t end = c.lo + c.n, k_last = (end - 1) / s;
  uint64_t k = c.lo / s, expect_lo = c.lo, launches = 0;
  while (k <= k_last) {
    GatherArgs a;
    uint64_t blocks = 0;
    const uint64_t next = zero::gather_launch(g, k, &a, &blocks);
    EXPECT(blocks > 0 && next > k, "launch at row %llu", (unsigned long long)k);
    if (blocks == 0 || next <= k) return;
    ++launches;
    const uint64_t pieces = next - k;
    EXPECT(pieces <= zero::kMaxGatherPieces, "pieces %llu", (unsigned long long)pieces);
    std::vector<std::vector<uint8_t>> seen(pieces);
    for (uint64_t b = 0; b < blocks; ++b) {
      const GatherPiece pc = zero::gather_piece(a, static_cast<uint32_t>(b));
      const uintptr_t src = reinterpret_cast<uintptr_t>(pc.src);
      const uintptr_t dst = reinterpret_cast<uintptr_t>(pc.dst);
      // which piece: from the destination, against the definition
      const uint64_t p_lo = c.lo + (dst - c.out_base) / 2;
      const uint64_t row = p_lo / s;
      const uint64_t q = row - k;
      EXPECT(q < pieces, "block %llu maps to row %llu", (unsigned long long)b,
             (unsigned long long)row);
      if (q >= pieces) return;
      const uint64_t want_hi = (row + 1) * s < end ? (row + 1) * s : end;
      EXPECT(p_lo == (row * s > c.lo ? row * s : c.lo) && p_lo + pc.n == want_hi,
             "piece of row %llu", (unsigned long long)row);
      EXPECT(src == c.shards_base + 2 * (row * stride + (p_lo - row * s)),
             "source of row %llu", (unsigned long long)row);
      const zero::GatherPlan& pl = pc.pl;
      if (seen[q].empty()) seen[q].assign(pl.wgs, 0);
      EXPECT(pc.wg < pl.wgs, "block %llu: wg %llu of %llu", (unsigned long long)b,
             (unsigned long long)pc.wg, (unsigned long long)pl.wgs);
      if (pc.wg >= pl.wgs) return;
      ++seen[q][pc.wg];
      const uint64_t per = pl.width / 2;
      const uint64_t v0 = pc.wg * zero::kGatherThreads;
      const uint64_t v1 = v0 + zero::kGatherThreads < pl.nvec ? v0 + zero::kGatherThreads : pl.nvec;
      if (v1 > v0) {
        const uint64_t e0 = pl.head + v0 * per, e1 = pl.head + v1 * per;
        EXPECT(e1 <= pc.n, "vectors end %llu beyond piece %llu", (unsigned long long)e1,
               (unsigned long long)pc.n);
        EXPECT((dst + 2 * e0) % pl.width == 0 && (src + 2 * e0) % pl.width == 0,
               "width %u misaligned", pl.width);
        if (pl.width > 2)
          EXPECT((dst + 2 * pl.head) % 128 == 0 || pl.head == pc.n,
                 "destination not on a line after the head");
        if (elementwise && e1 <= pc.n)
          for (uint64_t e = e0; e < e1; ++e) ++hits[p_lo - c.lo + e];
      }
      if (pc.wg + 1 == pl.wgs) {
        const uint64_t tail0 = pl.head + pl.nvec * per;
        EXPECT(tail0 <= pc.n && pc.n - tail0 < per + (per == 1), "tail");
        if (elementwise && tail0 <= pc.n && pl.head <= pc.n) {
          for (uint64_t e = 0; e < pl.head; ++e) ++hits[p_lo - c.lo + e];
          for (uint64_t e = tail0; e < pc.n; ++e) ++hits[p_lo - c.lo + e];
        }
      }
    }
    // every piece of the launch tiles the range in order, all workgroups once
    for (uint64_t q = 0; q < pieces; ++q) {
      const uint64_t row = k + q;
      const uint64_t p_lo = row * s > c.lo ? row * s : c.lo;
      EXPECT(p_lo == expect_lo, "piece %llu starts at %llu, want %llu", (unsigned long long)q,
             (unsigned long long)p_lo, (unsigned long long)expect_lo);
      expect_lo = (row + 1) * s < end ? (row + 1) * s : end;
      EXPECT(!seen[q].empty(), "piece %llu has no workgroup", (unsigned long long)q);
      for (size_t w = 0; w < seen[q].size(); ++w)
        EXPECT(seen[q][w] == 1, "piece %llu wg %zu hit %u times", (unsigned long long)q, w,
               seen[q][w]);
    }
    k = next;
  }
  EXPECT(expect_lo == end, "pieces end at %llu, want %llu", (unsigned long long)expect_lo,
         (unsigned long long)end);
  for (uint64_t j = 0; j < hits.size(); ++j)
    EXPECT(hits[j] == 1, "element %llu written %u times", (unsigned long long)j, hits[j]);
  (void)launches;
}

int main() {
  const uintptr_t A = 0x7f0000000000ull, B = 0x7f2000000000ull;
  // the device test cases, with the output's guard offset, and shifted bases
  const uint64_t dev[][6] = {
      {1000000, 4, 0, 0, 1000000, 0},    {1000000, 4, 0, 249990, 20, 0},
      {1000003, 7, 5, 123457, 700001, 3}, {1000003, 7, 1, 142858, 142857, 1},
      {1000003, 7, 2, 3, 500000, 2},     {1000003, 7, 4, 3, 500000, 0},
      {600, 200, 0, 5, 590, 0},          {1700, 100, 0, 0, 272, 0},
      {1700, 100, 0, 0, 273, 0},         {1700, 100, 3, 5, 267, 1},
      {1700, 100, 3, 5, 268, 1},         {3300000, 33, 11, 99990, 3000000, 5},
      {1000003, 7, 0, 1000, 20, 0},      {10, 3, 0, 9, 1, 1},
      {40000, 37, 3, 5, 39990, 0}};
  int cases = 0;
  for (const auto& d : dev)
    for (uintptr_t shift : {0ull, 2ull, 6ull, 96ull, 254ull}) {
      check({d[0], d[1], d[2], d[3], d[4], A + shift, B + 2 * (40 + d[5]) + shift}, true);
      ++cases;
    }
  // every layer of the 7.5B stage-3 schedule (hidden 4096) and of a 100B stack
  // at Nd = 400 (hidden 8192, 4-5 shards per layer), counted per workgroup
  for (uint64_t hidden : {4096ull, 8192ull}) {
    const uint64_t psi = hidden == 4096 ? 7500000000ull : 100000000000ull;
    const uint64_t nd = hidden == 4096 ? 64 : 400;
    const uint64_t per = 12 * hidden * hidden + 2 * hidden;
    for (uint64_t off = 0; off < psi; off += per) {
      check({psi, nd, 0, off, psi - off < per ? psi - off : per, A, B}, false);
      ++cases;
      if (hidden == 8192 && off > 40 * per) break;
    }
  }
  // the top of a 64-bit range
  check({1ull << 62, 3, 0, (1ull << 62) - 100, 100, A, B}, true);
  check({(1ull << 62) + 5, 7, 9, (1ull << 62) - 50, 55, A + 2, B + 6}, true);
  cases += 2;
  // random small gathers, element by element
  std::mt19937_64 rng(12345);
  for (int i = 0; i < 3000; ++i) {
    const uint64_t nd = 1 + rng() % 300;
    const uint64_t psi = 1 + rng() % 200000;
    const uint64_t lo = rng() % psi;
    const uint64_t n = 1 + rng() % (psi - lo);
    check({psi, nd, rng() % 40, lo, n, A + 2 * (rng() % 128), B + 2 * (rng() % 128)}, true);
    ++cases;
  }
  if (g_fail) {
    fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  printf("gather plan check ok: %d cases\n", cases);
  return 0;
}
