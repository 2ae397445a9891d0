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
// each a contiguous copy, and launches one copy per piece.  A piece is copied
// with the widest access the source and destination allow together (16, 8, 4
// or 2 bytes, from their alignment relative to each other); the elements
// before the destination reaches that alignment and after the last full vector
// go element by element in the same launch.  Pure data movement, bit-exact.
// When a range crosses many small shards an element-wise kernel does the whole
// range in one launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace zero {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int kW>
struct Vec;
template <>
struct Vec<16> { typedef u32x4 T; };
template <>
struct Vec<8> { typedef u32x2 T; };
template <>
struct Vec<4> { typedef uint32_t T; };

// Elements [0, head) and [head + nvec * V, n) element by element, the vectors
// in between with kW-byte accesses (V = kW / 2 elements each).
template <int kW>
__global__ void __launch_bounds__(kThreads) copy_kernel(const uint16_t* src, uint16_t* dst,
                                                        uint64_t n, uint64_t head,
                                                        uint64_t nvec) {
  const uint64_t t = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if constexpr (kW > 2) {
    constexpr uint64_t V = kW / 2;
    typedef typename Vec<kW>::T VT;
    if (t < nvec) {
      const uint64_t e = head + t * V;
      const VT x = __builtin_nontemporal_load(reinterpret_cast<const VT*>(src + e));
      __builtin_nontemporal_store(x, reinterpret_cast<VT*>(dst + e));
      return;
    }
    const uint64_t r = t - nvec;                      // a head or tail element
    const uint64_t e = r < head ? r : head + nvec * V + (r - head);
    if (e < n) dst[e] = src[e];
  } else {
    if (t < n) dst[t] = src[t];
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

hipError_t copy_piece(const uint16_t* src, uint16_t* dst, uint64_t n, hipStream_t stream) {
  const uintptr_t rel = (reinterpret_cast<uintptr_t>(src) - reinterpret_cast<uintptr_t>(dst));
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
  int w = (rel % 16 == 0) ? 16 : (rel % 8 == 0) ? 8 : (rel % 4 == 0) ? 4 : 2;
  uint64_t head = 0, nvec = 0;
  if (w > 2) {
    head = ((w - d % w) % w) / 2;                    // elements until dst is w-aligned
    if (head > n) head = n;
    nvec = (n - head) / (w / 2);
  }
  const uint64_t work = w > 2 ? nvec + (n - nvec * (w / 2)) : n;   // vectors + loose elements
  const uint64_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (w) {
    case 16: hipLaunchKernelGGL(copy_kernel<16>, grid, dim3(kThreads), 0, stream, src, dst, n, head, nvec); break;
    case 8: hipLaunchKernelGGL(copy_kernel<8>, grid, dim3(kThreads), 0, stream, src, dst, n, head, nvec); break;
    case 4: hipLaunchKernelGGL(copy_kernel<4>, grid, dim3(kThreads), 0, stream, src, dst, n, head, nvec); break;
    default: hipLaunchKernelGGL(copy_kernel<2>, grid, dim3(kThreads), 0, stream, src, dst, n, head, nvec); break;
  }
  return hipGetLastError();
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
  for (uint64_t k = k_first; k <= k_last; ++k) {
    const uint64_t p_lo = k * a.s > a.lo ? k * a.s : a.lo;
    const uint64_t p_hi = (k + 1) * a.s < a.lo + a.n ? (k + 1) * a.s : a.lo + a.n;
    const hipError_t e = copy_piece(a.shards + k * a.stride + (p_lo - k * a.s),
                                    a.out + (p_lo - a.lo), p_hi - p_lo, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace zero
