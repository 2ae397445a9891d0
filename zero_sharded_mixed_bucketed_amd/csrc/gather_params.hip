// The receive side of a stage-3 layer parameter gather (guide "ZeRO:
// particionar estados do treino entre GPUs", section "Como funciona": in the
// third stage the parameters are partitioned too and a process that needs
// another's partition receives it; lastdictionary entry "ZeRO": a layer's
// parameters are fetched right before it runs and dropped once it is done;
// card "ZeRO-2", "Why all-gather is still needed": the rank partitions in rank
// order are the full vector).
//
// Flat index i lives in rank k = i / S's shard at position i - k S, so a
// layer's range splits at shard edges into pieces, each a contiguous copy from
// one rank's row.  A launch copies up to kMaxGatherPieces consecutive pieces
// (a range crossing more shards takes several launches).  Pure data movement,
// bit-exact.
//
// Design (an HBM-bound copy; measured on MI355X over the 37 full layers of a
// 7.5B model at Nd = 64, 805 MB moved per layer):
//  - a workgroup is one wavefront and each thread moves one 16-byte vector
//    with a non-temporal load and store: short-lived wave-sized workgroups
//    keep the most bytes in flight, as for a plain copy;
//  - each piece's destination is brought to a 128-byte line before its
//    vectors start (the loose elements before the line and after the last
//    vector are copied one by one): with 64-thread workgroups, destinations
//    off the lines ran 11% slower;
//  - a workgroup finds its piece with no dependent memory access: the first
//    workgroup of every piece is a kernel argument, and the piece's row,
//    bounds and plan are recomputed from the launch's geometry.  Loading the
//    piece's fields from a table indexed by the piece cost 1.5%.
// The result: 6.54 TB/s per full layer, 0.97 of a plain copy of the same
// bytes (6.71 TB/s); the previous piece-table kernel with 256-thread
// workgroups and 16-byte destination alignment ran at 6.15.
//
// Vector width: 16 bytes when a piece's source and destination are 16-byte
// aligned relative to each other, else 8 or 4 bytes, else element by element.
// The index plan (pieces, launches, each workgroup's piece) is in
// gather_plan.h, shared with a CPU check of the kernel's indexing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace zero {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename VT>
__device__ __forceinline__ void copy_vec(const uint16_t* src, uint16_t* dst, uint64_t e) {
  __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const VT*>(src + e)),
                              reinterpret_cast<VT*>(dst + e));
}

__global__ void __launch_bounds__(kGatherThreads) copy_kernel(GatherArgs a) {
  const GatherPiece pc = gather_piece(a, blockIdx.x);
  const GatherPlan& pl = pc.pl;
  const uint64_t v = pc.wg * kGatherThreads + threadIdx.x;
  const uint32_t per = pl.width / 2;                   // elements per access
  if (v < pl.nvec) {
    const uint64_t e = pl.head + v * per;
    switch (pl.width) {
      case 16: copy_vec<u32x4>(pc.src, pc.dst, e); break;
      case 8: copy_vec<u32x2>(pc.src, pc.dst, e); break;
      case 4: copy_vec<uint32_t>(pc.src, pc.dst, e); break;
      default: pc.dst[e] = pc.src[e]; break;
    }
  }
  // the loose elements, by the piece's last workgroup: the head before the
  // line and the tail after the last full access
  if (pc.wg + 1 == pl.wgs) {
    const uint64_t tail0 = pl.head + pl.nvec * per;
    const uint64_t loose = pl.head + (pc.n - tail0);
    for (uint64_t r = threadIdx.x; r < loose; r += kGatherThreads) {
      const uint64_t e = r < pl.head ? r : tail0 + (r - pl.head);
      pc.dst[e] = pc.src[e];
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherLaunch& g, hipStream_t stream) {
  if (g.n == 0) return hipSuccess;
  const uint64_t k_last = (g.lo + g.n - 1) / g.s;
  uint64_t k = g.lo / g.s;
  while (k <= k_last) {
    GatherArgs a;
    uint64_t blocks = 0;
    k = gather_launch(g, k, &a, &blocks);
    if (blocks == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kGatherThreads), 0,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace zero
