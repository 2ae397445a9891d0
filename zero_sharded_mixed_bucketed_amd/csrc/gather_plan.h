// Index plan of the stage-3 layer gather (internal to libzero): how a flat range
// splits into per-rank pieces, which launch and workgroup copies which part of
// which piece, and how.  The host launch code, the kernel and a CPU check
// (tests/native/gather_plan_check.cpp, built with g++) all compile these same
// functions, so the kernel's indexing can be verified without a GPU.
#ifndef ZERO_GATHER_PLAN_H_
#define ZERO_GATHER_PLAN_H_

#include <stdint.h>

#ifdef __HIPCC__
#define ZERO_HD __host__ __device__
#else
#define ZERO_HD
#endif

namespace zero {

// The parameters of flat [lo, lo + n) gathered from the rank shards: row k at
// shards + k * stride holds flat [k * s, (k + 1) * s).
struct GatherLaunch {
  const uint16_t* shards;
  uint64_t stride;
  uint64_t s;
  uint64_t lo, n;
  uint16_t* out;
};

// Pieces (rank shards crossed) per gather launch; a gather that crosses more
// shards takes several launches.
constexpr uint64_t kMaxGatherPieces = 16;
constexpr int kGatherThreads = 64;      // one wavefront per workgroup
constexpr uintptr_t kGatherLine = 128;  // bytes per cache line

// How one piece of n elements from src to dst is copied: `width` bytes per
// access (16 when src and dst are 16-byte aligned relative to each other, else
// 8, 4 or element by element), `head` loose elements until dst reaches a line,
// then `nvec` accesses, then the loose tail; `wgs` workgroups.
struct GatherPlan {
  uint32_t width;
  uint64_t head, nvec, wgs;
};

ZERO_HD inline GatherPlan plan_piece(uintptr_t src, uintptr_t dst, uint64_t n) {
  GatherPlan p;
  const uintptr_t rel = src - dst;
  p.width = (rel % 16 == 0) ? 16 : (rel % 8 == 0) ? 8 : (rel % 4 == 0) ? 4 : 2;
  if (p.width == 2) {
    p.head = 0;
    p.nvec = n;
  } else {
    uint64_t head = ((kGatherLine - dst % kGatherLine) % kGatherLine) / 2;
    if (head > n) head = n;
    p.head = head;
    p.nvec = (n - head) / (p.width / 2);
  }
  const uint64_t w = (p.nvec + kGatherThreads - 1) / kGatherThreads;
  p.wgs = w ? w : 1;
  return p;
}

// The kernel arguments of one launch.
struct GatherArgs {
  const uint16_t* shards;  // row k at shards + k * stride holds flat [k s, (k + 1) s)
  uint64_t stride, s;
  uint64_t lo, end;        // this launch's flat range
  uint16_t* out;           // out[j] receives flat out_origin + j
  uint64_t out_origin;
  uint64_t k_first;        // the row of the launch's first piece
  uint32_t block0[kMaxGatherPieces];  // first workgroup of each piece; unused: ~0u
};

// What workgroup `block` of a launch copies: its piece (source, destination,
// length, plan) and its index among the piece's workgroups.  The piece is
// recovered from the launch geometry and the table of first workgroups alone,
// with no load through the piece index.
struct GatherPiece {
  const uint16_t* src;
  uint16_t* dst;
  uint64_t n;
  GatherPlan pl;
  uint64_t wg;
};

ZERO_HD inline GatherPiece gather_piece(const GatherArgs& a, uint32_t block) {
  uint32_t q = 0;
#pragma unroll
  for (uint32_t i = 1; i < kMaxGatherPieces; ++i) q += block >= a.block0[i] ? 1u : 0u;
  const uint64_t k = a.k_first + q;
  const uint64_t base = k * a.s;
  const uint64_t p_lo = base > a.lo ? base : a.lo;
  const uint64_t p_hi = a.end - base > a.s ? base + a.s : a.end;
  GatherPiece pc;
  pc.src = a.shards + k * a.stride + (p_lo - base);
  pc.dst = a.out + (p_lo - a.out_origin);
  pc.n = p_hi - p_lo;
  pc.pl = plan_piece(reinterpret_cast<uintptr_t>(pc.src), reinterpret_cast<uintptr_t>(pc.dst),
                     pc.n);
  pc.wg = block - a.block0[q];
  return pc;
}

// The launch that starts at row k (k <= the row of the range's last element):
// fills *a and *blocks and returns the next launch's first row.  Returns k and
// leaves *blocks at 0 when the grid would exceed 2^31 - 1 workgroups.
inline uint64_t gather_launch(const GatherLaunch& g, uint64_t k, GatherArgs* a, uint64_t* blocks) {
  const uint64_t end = g.lo + g.n;                     // <= psi: checked by the caller
  const uint64_t k_last = (end - 1) / g.s;
  a->shards = g.shards;
  a->stride = g.stride;
  a->s = g.s;
  a->out = g.out;
  a->out_origin = g.lo;
  a->k_first = k;
  a->lo = k * g.s > g.lo ? k * g.s : g.lo;
  a->end = a->lo;
  uint64_t nb = 0, p_hi = a->lo;
  uint32_t q = 0;
  for (; q < kMaxGatherPieces && k + q <= k_last; ++q) {
    const uint64_t base = (k + q) * g.s;               // <= end - 1: no overflow
    const uint64_t p_lo = base > g.lo ? base : g.lo;
    p_hi = end - base > g.s ? base + g.s : end;
    const uint16_t* src = g.shards + (k + q) * g.stride + (p_lo - base);
    const uint16_t* dst = g.out + (p_lo - g.lo);
    a->block0[q] = static_cast<uint32_t>(nb);
    nb += plan_piece(reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(dst),
                     p_hi - p_lo).wgs;
    if (nb > 0x7FFFFFFFull) {
      *blocks = 0;
      return k;
    }
  }
  for (uint32_t i = q; i < kMaxGatherPieces; ++i) a->block0[i] = ~0u;
  a->end = p_hi;
  *blocks = nb;
  return k + q;
}

}  // namespace zero

#endif  // ZERO_GATHER_PLAN_H_
