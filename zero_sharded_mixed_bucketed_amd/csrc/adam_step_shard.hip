// The fused sharded mixed-precision Adam step and the fp16 slot write (guide
// "ZeRO: particionar estados do treino entre GPUs", section "Como funciona":
// each process updates only its partition of the fp32 master weights,
// momentum and variance; card "ZeRO-2", section "Why all-gather is still
// needed": the updated fp16 shard is the rank's piece of the all-gather).
//
// Adam as published by Kingma & Ba (Algorithm 1), per element in fp32 with
// every operation rounded once (the file is compiled without contraction):
//   m' = b1*m + c1*g;  v' = b2*v + c2*(g*g);  den = sqrt(v')*isb + e;
//   th' = th - step*(m'/den);  p16 = fp16_rne(th')
// with the per-step scalars derived on the host.
//
// One pass over HBM: each element's g, th, m, v are read once and th, m, v and
// the fp16 slot written once (30 bytes per element with an fp32 gradient, 28
// with fp16).  There is no reuse, so the kernel streams with non-temporal
// hints: each thread owns 4 consecutive elements, loads all four inputs with
// 16-byte accesses before any arithmetic, and stores the results with 16-byte
// (fp32) and 8-byte (fp16) accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

#pragma clang fp contract(off)

namespace zero {
namespace {

constexpr int kThreads = kAdamThreads;  // one wavefront per workgroup
constexpr int kVec = 4;                 // elements per thread (16-byte accesses of the fp32 arrays)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Scalars {
  float b1, b2, c1, c2, eps, step, isb;
};

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ uint32_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// One element of the update.  sqrtf and the division are correctly rounded
// (the library is built with -fhip-fp32-correctly-rounded-divide-sqrt).
__device__ __forceinline__ void adam_elem(float& th, float& m, float& v, float g,
                                          const Scalars& s) {
  const float mn = s.b1 * m + s.c1 * g;
  const float vn = s.b2 * v + s.c2 * (g * g);
  const float den = sqrtf(vn) * s.isb + s.eps;
  th = th - s.step * (mn / den);
  m = mn;
  v = vn;
}

struct Args {
  float* master;
  float* m;
  float* v;
  const void* grad;
  uint16_t* p16;
  uint64_t n;
  uint64_t ngroups;  // full groups of kVec elements handled by the vector path
  Scalars s;
  int vec;           // master/m/v/grad aligned for 16-byte (8-byte fp16) access
  int st16;          // p16 slot alignment: 4: 8-byte stores, 2: 4-byte, 1: 2-byte
};

template <bool kG16>
__device__ __forceinline__ f32x4 load_grad(const Args& a, uint64_t j) {
  if constexpr (kG16) {
    const u32x2 h = __builtin_nontemporal_load(
        reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.grad) + j));
    return f32x4{h2f(h.x & 0xFFFFu), h2f(h.x >> 16), h2f(h.y & 0xFFFFu), h2f(h.y >> 16)};
  } else {
    return __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(static_cast<const float*>(a.grad) + j));
  }
}

__device__ __forceinline__ void store_p16(const Args& a, uint64_t j, const f32x4& th) {
  if (!a.p16) return;
  const uint32_t h0 = f2h(th.x), h1 = f2h(th.y), h2 = f2h(th.z), h3 = f2h(th.w);
  uint16_t* q = a.p16 + j;
  if (a.st16 == 4) {
    __builtin_nontemporal_store(u32x2{h0 | (h1 << 16), h2 | (h3 << 16)},
                                reinterpret_cast<u32x2*>(q));
  } else if (a.st16 == 2) {
    __builtin_nontemporal_store(h0 | (h1 << 16), reinterpret_cast<uint32_t*>(q));
    __builtin_nontemporal_store(h2 | (h3 << 16), reinterpret_cast<uint32_t*>(q + 2));
  } else {
    q[0] = static_cast<uint16_t>(h0);
    q[1] = static_cast<uint16_t>(h1);
    q[2] = static_cast<uint16_t>(h2);
    q[3] = static_cast<uint16_t>(h3);
  }
}

// One group of 4 elements per thread and a grid that covers the shard: on
// MI355X this streams the 4-read/4-write mix faster than a grid-stride loop
// with fewer, larger workgroups (short-lived wave-sized workgroups keep every
// CU refilled and the live accesses in one moving window of memory).  The
// launch caps a CU at 10 such workgroups (dynamic LDS the kernel never
// touches): with fewer concurrent streams per CU the mix runs at 6.55 rather
// than 6.0 TB/s.
template <bool kG16>
__global__ void __launch_bounds__(kThreads) adam_vec_kernel(Args a) {
  const uint64_t gi = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gi >= a.ngroups) return;
  const uint64_t j = gi * kVec;
  const f32x4 g = load_grad<kG16>(a, j);
  const f32x4 th = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.master + j));
  const f32x4 m = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.m + j));
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.v + j));
  float t0 = th.x, t1 = th.y, t2 = th.z, t3 = th.w;
  float m0 = m.x, m1 = m.y, m2 = m.z, m3 = m.w;
  float v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
  adam_elem(t0, m0, v0, g.x, a.s);
  adam_elem(t1, m1, v1, g.y, a.s);
  adam_elem(t2, m2, v2, g.z, a.s);
  adam_elem(t3, m3, v3, g.w, a.s);
  const f32x4 tn{t0, t1, t2, t3};
  __builtin_nontemporal_store(tn, reinterpret_cast<f32x4*>(a.master + j));
  __builtin_nontemporal_store(f32x4{m0, m1, m2, m3}, reinterpret_cast<f32x4*>(a.m + j));
  __builtin_nontemporal_store(f32x4{v0, v1, v2, v3}, reinterpret_cast<f32x4*>(a.v + j));
  store_p16(a, j, tn);
}

// Element-wise path: the tail after the last full group, or arrays that
// cannot take vector accesses.  Elements [first, n).
template <bool kG16>
__global__ void __launch_bounds__(kThreads) adam_scalar_kernel(Args a, uint64_t first) {
  const uint64_t nthreads = static_cast<uint64_t>(gridDim.x) * kThreads;
  for (uint64_t j = first + static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; j < a.n;
       j += nthreads) {
    float g;
    if constexpr (kG16) {
      g = h2f(static_cast<const uint16_t*>(a.grad)[j]);
    } else {
      g = static_cast<const float*>(a.grad)[j];
    }
    float th = a.master[j], m = a.m[j], v = a.v[j];
    adam_elem(th, m, v, g, a.s);
    a.master[j] = th;
    a.m[j] = m;
    a.v[j] = v;
    if (a.p16) a.p16[j] = static_cast<uint16_t>(f2h(th));
  }
}

}  // namespace

const void* adam_kernel_fn(int grad_is_fp16) {
  return grad_is_fp16 ? reinterpret_cast<const void*>(&adam_vec_kernel<true>)
                      : reinterpret_cast<const void*>(&adam_vec_kernel<false>);
}

hipError_t launch_adam(const AdamLaunch& L, const DeviceCaps& d, hipStream_t stream) {
  Args a;
  a.master = L.master;
  a.m = L.m;
  a.v = L.v;
  a.grad = L.grad;
  a.p16 = L.p16;
  a.n = L.n;
  a.s = Scalars{L.b1, L.b2, L.c1, L.c2, L.eps, L.step, L.isb};
  const auto al = [](const void* p, uintptr_t b) {
    return reinterpret_cast<uintptr_t>(p) % b == 0;
  };
  a.vec = al(L.master, 16) && al(L.m, 16) && al(L.v, 16) &&
          al(L.grad, L.grad_is_fp16 ? 8 : 16);
  a.st16 = 1;
  if (L.p16) a.st16 = al(L.p16, 8) ? 4 : al(L.p16, 4) ? 2 : 1;
  a.ngroups = a.vec ? L.n / kVec : 0;
  if (a.ngroups) {
    const uint64_t want = (a.ngroups + kThreads - 1) / kThreads;
    if (want > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const unsigned blocks = static_cast<unsigned>(want);
    // the dynamic LDS that caps the kernel at kAdamWgsPerCu per CU
    if (L.grad_is_fp16)
      hipLaunchKernelGGL(adam_vec_kernel<true>, dim3(blocks), dim3(kThreads), d.adam_lds[1],
                         stream, a);
    else
      hipLaunchKernelGGL(adam_vec_kernel<false>, dim3(blocks), dim3(kThreads), d.adam_lds[0],
                         stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const uint64_t first = a.ngroups * kVec;
  if (first < L.n) {
    const uint64_t rest = L.n - first;
    // the tail (< 4 elements) or a whole misaligned shard: grid-stride over it
    const uint64_t want_s = (rest + kThreads - 1) / kThreads;
    const uint64_t cap = static_cast<uint64_t>(d.cus) * 32;
    const unsigned blocks = static_cast<unsigned>(want_s < cap ? want_s : cap);
    if (L.grad_is_fp16)
      hipLaunchKernelGGL(adam_scalar_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, a,
                         first);
    else
      hipLaunchKernelGGL(adam_scalar_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, a,
                         first);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace zero
