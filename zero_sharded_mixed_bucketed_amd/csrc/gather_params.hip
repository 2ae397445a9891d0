// The receive side of a stage-3 layer parameter gather (guide "ZeRO:
// particionar estados do treino entre GPUs", section "Como funciona": in the
// third stage the parameters are partitioned too and a process that needs
// another's partition receives it; lastdictionary entry "ZeRO": each layer's
// parameters are gathered just in time and discarded afterwards; card
// "ZeRO-2", "Why all-gather is still needed": the rank partitions in rank
// order are the full vector).
//
// Flat index i lives in rank k = i / S's shard at position i - k S.  A layer's
// range crosses one shard or a few, so the host splits it into per-rank pieces,
// each a contiguous copy, and one launch copies them all: every workgroup
// belongs to one piece (a table of at most kMaxGatherPieces in the kernel
// arguments).  A piece is copied with the widest access its source and
// destination allow together (16, 8, 4 or 2 bytes, from their alignment
// relative to each other); the elements before the destination reaches that
// alignment and after the last full vector go element by element.  The width
// is uniform within a workgroup.  Pure data movement, bit-exact.  When a
// range crosses more shards than the table holds, an element-wise kernel does
// the whole range in one launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace zero {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Piece {
  const uint16_t* src;
  uint16_t* dst;
  uint64_t n;         // elements
  uint64_t head;      // elements before dst reaches the access width
  uint64_t nvec;      // full vectors after the head
  uint32_t block0;    // first workgroup of this piece
  uint32_t width;     // bytes per access: 16, 8, 4 or 2
};

struct Pieces {
  Piece p[kMaxGatherPieces];
  uint32_t count;
};

template <typename VT, int kV>
__device__ __forceinline__ void copy_piece(const Piece& pc, uint64_t t) {
  if (t < pc.nvec) {
    const uint64_t e = pc.head + t * kV;
    const VT x = __builtin_nontemporal_load(reinterpret_cast<const VT*>(pc.src + e));
    __builtin_nontemporal_store(x, reinterpret_cast<VT*>(pc.dst + e));
    return;
  }
  const uint64_t r = t - pc.nvec;                     // a head or tail element
  const uint64_t e = r < pc.head ? r : pc.head + pc.nvec * kV + (r - pc.head);
  if (e < pc.n) pc.dst[e] = pc.src[e];
}

__global__ void __launch_bounds__(kThreads) copy_kernel(Pieces ps) {
  uint32_t q = 0;                                     // this workgroup's piece
  while (q + 1 < ps.count && blockIdx.x >= ps.p[q + 1].block0) ++q;
  const Piece& pc = ps.p[q];
  const uint64_t t = static_cast<uint64_t>(blockIdx.x - pc.block0) * kThreads + threadIdx.x;
  switch (pc.width) {
    case 16: copy_piece<u32x4, 8>(pc, t); break;
    case 8: copy_piece<u32x2, 4>(pc, t); break;
    case 4: copy_piece<uint32_t, 2>(pc, t); break;
    default:
      if (t < pc.n) pc.dst[t] = pc.src[t];
      break;
  }
}

// The whole range at once: out[j] = row (lo + j) / S at column (lo + j) mod S.
__global__ void __launch_bounds__(kThreads) gather_elem_kernel(GatherLaunch a) {
  const uint64_t j = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= a.n) return;
  const uint64_t i = a.lo + j;
  const uint64_t k = i / a.s;
  a.out[j] = a.shards[k * a.stride + (i - k * a.s)];
}

// Fills one piece's access width, head, vector count and thread count.
uint64_t plan_piece(Piece& pc) {
  const uintptr_t rel = reinterpret_cast<uintptr_t>(pc.src) - reinterpret_cast<uintptr_t>(pc.dst);
  const uintptr_t d = reinterpret_cast<uintptr_t>(pc.dst);
  const uint32_t w = (rel % 16 == 0) ? 16 : (rel % 8 == 0) ? 8 : (rel % 4 == 0) ? 4 : 2;
  pc.width = w;
  pc.head = pc.nvec = 0;
  if (w == 2) return pc.n;
  pc.head = ((w - d % w) % w) / 2;                    // elements until dst is w-aligned
  if (pc.head > pc.n) pc.head = pc.n;
  pc.nvec = (pc.n - pc.head) / (w / 2);
  return pc.nvec + (pc.n - pc.nvec * (w / 2));        // vectors + loose elements
}

}  // namespace

hipError_t launch_gather(const GatherLaunch& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const uint64_t k_first = a.lo / a.s, k_last = (a.lo + a.n - 1) / a.s;
  if (k_last - k_first + 1 > kMaxGatherPieces) {
    const uint64_t blocks = (a.n + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_elem_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
  }
  Pieces ps;
  ps.count = 0;
  uint64_t blocks = 0;
  const uint64_t end = a.lo + a.n;                    // <= psi: checked by the caller
  for (uint64_t k = k_first; k <= k_last; ++k) {
    const uint64_t base = k * a.s;                     // <= lo + n - 1: no overflow
    const uint64_t p_lo = base > a.lo ? base : a.lo;
    const uint64_t p_hi = end - base > a.s ? base + a.s : end;
    Piece& pc = ps.p[ps.count++];
    pc.src = a.shards + k * a.stride + (p_lo - k * a.s);
    pc.dst = a.out + (p_lo - a.lo);
    pc.n = p_hi - p_lo;
    const uint64_t work = plan_piece(pc);
    pc.block0 = static_cast<uint32_t>(blocks);
    blocks += (work + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     ps);
  return hipGetLastError();
}

}  // namespace zero
