// CPU check of the owner's reduce's indexing, built with g++ from the same
// reduce_plan.h the kernel compiles.  For each case, the launch is planned as
// the library plans it (the bucket-intersect-shard columns are derived the way
// zero_reduce_shard derives them), and every thread's group is walked as the
// kernel walks it.  Checked against the definition of the reduce (column c of
// the bucket, flat index bucket_offset + c, is reduced into shard element
// bucket_offset + c - shard offset, only inside bucket-intersect-shard):
//  - every owned column is reduced by exactly one thread, and no other column;
//  - every output index lies in [0, shard length);
//  - full groups lie wholly inside the owned columns, their row loads are
//    aligned to the chosen width in every row and stay inside the row buffer,
//    and their stores are aligned to the chosen store widths.
// Addresses are never dereferenced: buffers are stand-in base addresses.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "reduce_plan.h"

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
  uint64_t psi, nd, rank, boff, blen, stride;
  uintptr_t rows, out32, out16;  // 0: no such output
};

static uint64_t g_groups = 0;

static void check(const Case& c, bool columnwise) {
  // the rank's shard and the owned part of the bucket, as zero_reduce_shard has them
  const uint64_t s = c.psi / c.nd + (c.psi % c.nd != 0);
  const uint64_t s_lo = c.rank * s < c.psi ? c.rank * s : c.psi;
  const uint64_t len = c.psi - s_lo < s ? c.psi - s_lo : s;
  const uint64_t a = c.boff > s_lo ? c.boff : s_lo;
  const uint64_t b = c.boff + c.blen < s_lo + len ? c.boff + c.blen : s_lo + len;
  if (a >= b) return;                                   // nothing owned: no launch
  zero::ReduceLaunch L;
  L.rows = reinterpret_cast<const uint16_t*>(c.rows);
  L.stride = c.stride;
  L.nd = static_cast<uint32_t>(c.nd);
  L.c_lo = a - c.boff;
  L.c_hi = b - c.boff;
  L.delta = static_cast<int64_t>(c.boff - s_lo);
  L.out32 = reinterpret_cast<float*>(c.out32);
  L.out16 = reinterpret_cast<uint16_t*>(c.out16);
  L.inv_nd = 1.0f;
  int width = 0;
  uint64_t groups = 0;
  const zero::ReduceArgs args = zero::reduce_plan(L, &width, &groups);
  EXPECT(width == 16 || width == 8 || width == 4 || width == 2, "width %d", width);
  g_groups += groups;
  std::vector<uint8_t> hits(columnwise ? L.c_hi : 0, 0);
  uint64_t covered = 0;
  const uint64_t row_end = (c.nd - 1) * c.stride + c.blen;  // elements in the row buffer
  for (uint64_t gi = 0; gi < groups; ++gi) {
    uint64_t col = 0;
    const bool full = zero::reduce_group(args, gi, &col);
    if (full) {
      EXPECT(col >= L.c_lo && col + zero::kReduceCols <= L.c_hi, "full group at %llu",
             (unsigned long long)col);
      for (uint64_t k : {uint64_t{0}, uint64_t{1}, c.nd - 1}) {
        if (k >= c.nd) continue;
        const uint64_t e = k * c.stride + col;
        EXPECT((c.rows + 2 * e) % width == 0, "row %llu load misaligned",
               (unsigned long long)k);
        EXPECT(e + zero::kReduceCols <= row_end, "row %llu load beyond the buffer",
               (unsigned long long)k);
      }
      const uint64_t o = col + static_cast<uint64_t>(L.delta);
      EXPECT(o + zero::kReduceCols <= len, "output %llu beyond the shard", (unsigned long long)o);
      if (c.out32)
        EXPECT((c.out32 + 4 * o) % (4 * args.st32) == 0, "fp32 store misaligned");
      if (c.out16)
        EXPECT((c.out16 + 2 * o) % (2 * args.st16) == 0, "fp16 store misaligned");
      covered += zero::kReduceCols;
      if (columnwise)
        for (uint64_t e = col; e < col + zero::kReduceCols; ++e) ++hits[e];
    } else {
      for (uint64_t e = col; e < col + zero::kReduceCols; ++e) {
        if (e < L.c_lo || e >= L.c_hi) continue;
        const uint64_t o = e + static_cast<uint64_t>(L.delta);
        EXPECT(o < len, "ragged output %llu beyond the shard", (unsigned long long)o);
        EXPECT((c.nd - 1) * c.stride + e < row_end, "ragged load beyond the buffer");
        ++covered;
        if (columnwise) ++hits[e];
      }
    }
  }
  EXPECT(covered == L.c_hi - L.c_lo, "covered %llu of %llu columns",
         (unsigned long long)covered, (unsigned long long)(L.c_hi - L.c_lo));
  for (uint64_t e = 0; e < hits.size(); ++e)
    EXPECT(hits[e] == (e >= L.c_lo ? 1 : 0), "column %llu reduced %u times",
           (unsigned long long)e, hits[e]);
}

int main() {
  const uintptr_t R = 0x7f0000000000ull, O = 0x7f2000000000ull, H = 0x7f3000000000ull;
  int cases = 0;
  // the benchmarked workloads' launches at the advised stride (64-element rows,
  // plus 1,024 when a whole number of MiB), fp32 and fp16 outputs
  auto advised = [](uint64_t n) {
    uint64_t st = (n + 63) / 64 * 64;
    if (st != 0 && st % (1u << 19) == 0) st += 1024;
    return st;
  };
  for (uint64_t rank : {uint64_t{0}, uint64_t{1}, uint64_t{63}}) {       // 7.5B, Nd = 64
    const uint64_t psi = 7500000000ull, bucket = 25000000;
    for (uint64_t hi = psi; hi > 0; hi -= hi < bucket ? hi : bucket) {
      const uint64_t lo = hi < bucket ? 0 : hi - bucket;
      check({psi, 64, rank, lo, hi - lo, advised(hi - lo), R, O, H}, false);
      ++cases;
    }
  }
  for (uint64_t hi = 13000000000ull; hi > 12000000000ull; hi -= 25000000) {  // 13B, Nd = 32
    check({13000000000ull, 32, 0, hi - 25000000, 25000000, advised(25000000), R, O, 0}, false);
    ++cases;
  }
  // the 100B rank-137 chunks of 2^22 columns inside its first bucket
  for (uint64_t c0 = 34250000000ull; c0 < 34250000000ull + 21138048; c0 += 1u << 22) {
    const uint64_t n = (1u << 22) < 34250000000ull + 21138048 - c0 ? (1u << 22)
                                                                   : 34250000000ull + 21138048 - c0;
    check({100000000000ull, 400, 137, c0, n, advised(n), R, O, 0}, false);
    ++cases;
  }
  // random small launches: any stride >= the bucket, any 2-byte row base, any
  // 4-byte fp32 and 2-byte fp16 output base, column by column
  std::mt19937_64 rng(777);
  for (int i = 0; i < 20000; ++i) {
    const uint64_t nd = 1 + rng() % 70;
    const uint64_t psi = 1 + rng() % 5000;
    const uint64_t rank = rng() % nd;
    const uint64_t boff = rng() % psi;
    const uint64_t blen = 1 + rng() % (psi - boff);
    const uint64_t stride = blen + rng() % 40;
    const int outs = 1 + static_cast<int>(rng() % 3);  // 1: fp32, 2: fp16, 3: both
    check({psi, nd, rank, boff, blen, stride, R + 2 * (rng() % 64),
           outs & 1 ? O + 4 * (rng() % 32) : 0, outs & 2 ? H + 2 * (rng() % 64) : 0},
          true);
    ++cases;
  }
  if (g_fail) {
    fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  printf("reduce plan check ok: %d cases, %llu thread groups\n", cases,
         (unsigned long long)g_groups);
  return 0;
}
