// The owner's reduce of one gradient bucket (guide "ZeRO: particionar estados
// do treino entre GPUs", section "Como funciona": in stage 2 a gradient is
// reduced only at the process that owns its partition, then released; card
// "ZeRO-2", section "Gradient lifecycle").
//
// Nd fp16 rows, one per data-parallel rank, are summed element by element in
// fp32, in ascending rank order starting from +0, and scaled once by RN32(1/Nd).
// Vectorisation is across elements, never across ranks, so each element's
// additions keep the rank order and the result is bit-exact.
//
// The kernel is HBM-bound (2 Nd bytes read and 4 written per output element,
// no reuse) and built for streaming:
//  - each thread owns 8 consecutive columns and reads each row's 8 fp16 values
//    with one 16-byte non-temporal load (narrower only when the row stride or
//    base rules 16 bytes out), keeping the 8 running sums in registers;
//  - the rows go in batches of 16 (the rest in batches of 8, 4, 2 and 1), and
//    each batch's loads overlap the additions of the rows before it, so 6 or 7
//    loads per thread are in flight throughout;
//  - a workgroup is one wavefront and reads 1 KiB contiguous per row;
//  - at most 8 workgroups share a compute unit (a dynamic-LDS occupancy cap set
//    at launch): fewer concurrent row streams per CU move more bytes per second
//    on MI355X (6.4 against 6.1 TB/s at Nd = 64).
// On MI355X the same access pattern without the stores streams at about
// 7.0 TB/s under the cap; the 4 bytes per element written back cost the rest
// (writes that leave L2 while the read stream saturates HBM are expensive).
//
// A thread reads every row of its columns before it writes their outputs, and
// no other thread touches those columns, so an output may share memory with a
// row column for column (the reduced value replacing that row's element).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

#pragma clang fp contract(off)

namespace zero {
namespace {

constexpr int kThreads = kReduceThreads;  // one wavefront per workgroup
constexpr int kCols = kReduceCols;        // columns per thread (one 16-byte fp16 load per row)
constexpr int kBatch = 16;                // rows per batch

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ uint32_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ void add8(float (&acc)[kCols], u32x4 x) {
  acc[0] = acc[0] + h2f(x.x & 0xFFFFu);
  acc[1] = acc[1] + h2f(x.x >> 16);
  acc[2] = acc[2] + h2f(x.y & 0xFFFFu);
  acc[3] = acc[3] + h2f(x.y >> 16);
  acc[4] = acc[4] + h2f(x.z & 0xFFFFu);
  acc[5] = acc[5] + h2f(x.z >> 16);
  acc[6] = acc[6] + h2f(x.w & 0xFFFFu);
  acc[7] = acc[7] + h2f(x.w >> 16);
}

using Args = ReduceArgs;

__device__ __forceinline__ void store_full(const Args& a, uint64_t o, const float (&r)[kCols]) {
  if (a.out32) {
    float* p = a.out32 + o;
    if (a.st32 == 4) {
      __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, reinterpret_cast<f32x4*>(p));
      __builtin_nontemporal_store(f32x4{r[4], r[5], r[6], r[7]}, reinterpret_cast<f32x4*>(p + 4));
    } else if (a.st32 == 2) {
#pragma unroll
      for (int e = 0; e < kCols; e += 2)
        __builtin_nontemporal_store(f32x2{r[e], r[e + 1]}, reinterpret_cast<f32x2*>(p + e));
    } else {
#pragma unroll
      for (int e = 0; e < kCols; ++e) __builtin_nontemporal_store(r[e], p + e);
    }
  }
  if (a.out16) {
    uint16_t* q = a.out16 + o;
    uint32_t h[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) h[e] = f2h(r[e]);
    if (a.st16 == 8) {
      __builtin_nontemporal_store(
          u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)},
          reinterpret_cast<u32x4*>(q));
    } else if (a.st16 == 4) {
      __builtin_nontemporal_store(u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)},
                                  reinterpret_cast<u32x2*>(q));
      __builtin_nontemporal_store(u32x2{h[4] | (h[5] << 16), h[6] | (h[7] << 16)},
                                  reinterpret_cast<u32x2*>(q + 4));
    } else if (a.st16 == 2) {
#pragma unroll
      for (int e = 0; e < kCols; e += 2)
        __builtin_nontemporal_store(h[e] | (h[e + 1] << 16), reinterpret_cast<uint32_t*>(q + e));
    } else {
#pragma unroll
      for (int e = 0; e < kCols; ++e) q[e] = static_cast<uint16_t>(h[e]);
    }
  }
}

// Loads the 8 fp16 values of one row at columns [c, c + 8) with accesses of
// kW bytes (16, 8, 4 or 2), the widest the row alignment allows.
template <int kW>
__device__ __forceinline__ u32x4 load8(const uint16_t* p) {
  if constexpr (kW == 16) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else if constexpr (kW == 8) {
    const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    const u32x2 b = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + 4));
    return u32x4{a.x, a.y, b.x, b.y};
  } else if constexpr (kW == 4) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    return u32x4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                 __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3)};
  } else {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = __builtin_nontemporal_load(p + e);
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                 h[6] | (h[7] << 16)};
  }
}

// Adds rows [k, k + kB) at the thread's 8 columns, in ascending order (the
// loads are independent of each other; the compiler overlaps them with the
// additions).
template <int kW, int kB>
__device__ __forceinline__ void add_rows(float (&acc)[kCols], const uint16_t* p, uint32_t k,
                                         uint64_t stride) {
  u32x4 x[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u) x[u] = load8<kW>(p + (k + u) * stride);
#pragma unroll
  for (int u = 0; u < kB; ++u) add8(acc, x[u]);
}

template <int kW>
__global__ void __launch_bounds__(kThreads) reduce_kernel(Args a) {
  const uint64_t gi = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gi >= a.ngroups) return;
  uint64_t c;
  const bool full = reduce_group(a, gi, &c);
  float acc[kCols];
#pragma unroll
  for (int e = 0; e < kCols; ++e) acc[e] = 0.0f;  // +0

  if (full) {
    const uint16_t* p = a.rows + c;
    uint32_t k = 0;
    // The bound is computed once: with it the compiler knows the trip count and
    // overlaps each batch's loads with the previous rows' additions (6 or 7 loads
    // in flight throughout), which streams about 5% faster than issuing the 16
    // loads of a batch at once and draining them.
    const uint32_t nfull = a.nd - a.nd % kBatch;
    for (; k < nfull; k += kBatch) add_rows<kW, kBatch>(acc, p, k, a.stride);
    // the remaining nd % 16 rows, still in ascending order
    if (a.nd - k >= 8) { add_rows<kW, 8>(acc, p, k, a.stride); k += 8; }
    if (a.nd - k >= 4) { add_rows<kW, 4>(acc, p, k, a.stride); k += 4; }
    if (a.nd - k >= 2) { add_rows<kW, 2>(acc, p, k, a.stride); k += 2; }
    if (a.nd - k >= 1) add_rows<kW, 1>(acc, p, k, a.stride);
    float r[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) r[e] = acc[e] * a.inv;
    store_full(a, c + static_cast<uint64_t>(a.delta), r);
    return;
  }

  // A ragged edge group: element-wise, with the same per-element order of
  // additions.
  for (uint32_t k = 0; k < a.nd; ++k) {
    const uint16_t* row = a.rows + static_cast<uint64_t>(k) * a.stride;
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      const uint64_t col = c + e;
      if (col >= a.c_lo && col < a.c_hi) acc[e] = acc[e] + h2f(row[col]);
    }
  }
#pragma unroll
  for (int e = 0; e < kCols; ++e) {
    const uint64_t col = c + e;
    if (col >= a.c_lo && col < a.c_hi) {
      const float r = acc[e] * a.inv;
      const uint64_t o = col + static_cast<uint64_t>(a.delta);
      if (a.out32) a.out32[o] = r;
      if (a.out16) a.out16[o] = static_cast<uint16_t>(f2h(r));
    }
  }
}

}  // namespace

const void* reduce_kernel_fn(int width) {
  switch (width) {
    case 16: return reinterpret_cast<const void*>(&reduce_kernel<16>);
    case 8: return reinterpret_cast<const void*>(&reduce_kernel<8>);
    case 4: return reinterpret_cast<const void*>(&reduce_kernel<4>);
    default: return reinterpret_cast<const void*>(&reduce_kernel<2>);
  }
}

hipError_t launch_reduce(const ReduceLaunch& L, const DeviceCaps& d, hipStream_t stream) {
  int w = 0;
  uint64_t groups = 0;
  const Args a = reduce_plan(L, &w, &groups);
  const uint64_t blocks = (groups + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  // the dynamic LDS that caps each instantiation at kReduceWgsPerCu per CU
  switch (w) {
    case 16:
      hipLaunchKernelGGL(reduce_kernel<16>, grid, dim3(kThreads), d.reduce_lds[0], stream, a);
      break;
    case 8:
      hipLaunchKernelGGL(reduce_kernel<8>, grid, dim3(kThreads), d.reduce_lds[1], stream, a);
      break;
    case 4:
      hipLaunchKernelGGL(reduce_kernel<4>, grid, dim3(kThreads), d.reduce_lds[2], stream, a);
      break;
    default:
      hipLaunchKernelGGL(reduce_kernel<2>, grid, dim3(kThreads), d.reduce_lds[3], stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace zero
