// Streaming probes: the practical HBM rates of plain access patterns on the
// device, measured beside the path's kernels as context for their rates.  They
// compute nothing of the ZeRO method.
//
//  - read_rows: the owner reduce's access pattern (Nd rows, each thread one
//    16-byte column group read in every row with non-temporal loads) without
//    its additions and without its output stores; the rows are double-buffered
//    four at a time (the next four issued before the current four are used),
//    which streamed as fast as or faster than batches of 8 or 16 at every Nd
//    tried (8 to 400; batches of 16 drain at small Nd);
//  - write: one 16-byte store per thread, in workgroups of 256 threads;
//  - copy: one 16-byte non-temporal load and store per thread, in workgroups of
//    one wavefront.
// These were the fastest shapes of each pattern on MI355X: 64-thread workgroups
// that only write 1 KiB each are held to about 4.8 TB/s by the rate at which
// workgroups are dispatched, and non-temporal stores write no faster here.
// Each launch can cap the workgroups per compute unit with dynamic LDS that the
// kernel never touches (the device the path's kernels use).
//
//  - residency: each one-wavefront workgroup sleeps for a fixed time and its
//    first lane records the compute unit it ran on and the wall-clock interval
//    it spanned; the most intervals that overlap on one compute unit is the
//    number of workgroups resident there at once, under a given dynamic LDS
//    size.  It checks that an LDS size really caps residency on the hardware.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 64;
constexpr int kWriteThreads = 256;
constexpr int kDepth = 4;   // rows per buffer of the read probe

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// XOR of every 16-byte group the thread reads; written (one 4-byte vector store)
// only if it equals `key`, which keeps the loads live at no write cost.
__global__ void __launch_bounds__(kThreads) read_rows_kernel(const uint16_t* rows, uint64_t stride,
                                                             uint32_t nd, uint64_t ngroups,
                                                             uint32_t key, uint32_t* sink) {
  const uint64_t gi = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gi >= ngroups) return;
  const uint16_t* p = rows + gi * 8;
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint32_t k = 0;
  if (nd >= kDepth) {
    u32x4 cur[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
      cur[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + u * stride));
    const uint32_t nfull = nd - nd % kDepth;
    for (k = kDepth; k < nfull; k += kDepth) {
      u32x4 nxt[kDepth];
#pragma unroll
      for (int u = 0; u < kDepth; ++u)
        nxt[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + (k + u) * stride));
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        acc ^= cur[u];
        cur[u] = nxt[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kDepth; ++u) acc ^= cur[u];
  }
  for (; k < nd; ++k)
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + k * stride));
  const uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (h == key) sink[0] = static_cast<uint32_t>(gi);
}

__global__ void __launch_bounds__(kWriteThreads) write_kernel(u32x4* dst, uint64_t n, u32x4 v) {
  const uint64_t gi = static_cast<uint64_t>(blockIdx.x) * kWriteThreads + threadIdx.x;
  if (gi < n) dst[gi] = v;
}

__global__ void __launch_bounds__(kThreads) copy_kernel(const u32x4* src, u32x4* dst, uint64_t n) {
  const uint64_t gi = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gi < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + gi), dst + gi);
}

// A compute unit's identity: XCC (hardware register XCC_ID, bits 3:0) above
// bits 8..14 of HW_ID (CU_ID 11:8, SH_ID 12, SE_ID 14:13 on gfx950).
__device__ __forceinline__ uint32_t cu_key() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID, 32 bits
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);   // XCC_ID, 4 bits
  return ((xcc & 0xFu) << 8) | ((hw >> 8) & 0x7Fu);
}

// rec[3 b .. 3 b + 2] = {start, end, cu_key} of workgroup b; `sleeps` rounds of
// s_sleep (a bounded loop: every wave exits).
__global__ void __launch_bounds__(kThreads) residency_kernel(unsigned long long* rec,
                                                            uint32_t sleeps) {
  const unsigned long long t0 = static_cast<unsigned long long>(wall_clock64());
  for (uint32_t i = 0; i < sleeps; ++i) __builtin_amdgcn_s_sleep(8);
  const unsigned long long t1 = static_cast<unsigned long long>(wall_clock64());
  if (threadIdx.x == 0) {
    unsigned long long* r = rec + 3ull * blockIdx.x;
    r[0] = t0;
    r[1] = t1;
    r[2] = cu_key();
  }
}

// Dynamic LDS per workgroup that limits a compute unit to `wgs` workgroups (0:
// no cap), or -1 if the device cannot be queried: the CU's LDS over `wgs`,
// rounded down to the 1,280-byte granule in which gfx950 allocates LDS (a size
// between granules is rounded up by the hardware and can hold one workgroup
// fewer).
long cap_bytes(int wgs) {
  if (wgs <= 0) return 0;
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
      hipSuccess)
    return -1;
  return static_cast<long>(lds / wgs) / 1280 * 1280;
}

bool grid_of(uint64_t items, unsigned* blocks, uint64_t threads = kThreads) {
  const uint64_t b = (items + threads - 1) / threads;
  if (b == 0 || b > 0x7FFFFFFFull) return false;
  *blocks = static_cast<unsigned>(b);
  return true;
}

}  // namespace

extern "C" {

// Reads Nd rows of `cols` fp16 values (row k at rows + k * stride elements).
// rows must be 16-byte aligned, stride and cols multiples of 8 with stride >=
// cols; sink is a device uint32_t.  Returns 0, -1 on bad arguments, -3 if the
// device query or the launch failed.
int zprobe_read_rows(const uint16_t* rows, uint64_t stride, uint32_t nd, uint64_t cols,
                     int wgs_per_cu, uint32_t key, uint32_t* sink, void* stream) {
  unsigned blocks = 0;
  if (!rows || !sink || nd == 0 || cols % 8 || stride % 8 || stride < cols ||
      reinterpret_cast<uintptr_t>(rows) % 16 || !grid_of(cols / 8, &blocks))
    return -1;
  const long cap = cap_bytes(wgs_per_cu);
  if (cap < 0) return -3;
  hipLaunchKernelGGL(read_rows_kernel, dim3(blocks), dim3(kThreads), static_cast<unsigned>(cap),
                     static_cast<hipStream_t>(stream), rows, stride, nd, cols / 8, key, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Writes `bytes` (a multiple of 16) at dst (16-byte aligned).
int zprobe_write(void* dst, uint64_t bytes, int wgs_per_cu, void* stream) {
  unsigned blocks = 0;
  if (!dst || bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16 ||
      !grid_of(bytes / 16, &blocks, kWriteThreads))
    return -1;
  const long cap = cap_bytes(wgs_per_cu);
  if (cap < 0) return -3;
  const u32x4 v = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  hipLaunchKernelGGL(write_kernel, dim3(blocks), dim3(kWriteThreads), static_cast<unsigned>(cap),
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst), bytes / 16, v);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Copies `bytes` (a multiple of 16) from src to dst (both 16-byte aligned, not
// overlapping).
int zprobe_copy(const void* src, void* dst, uint64_t bytes, int wgs_per_cu, void* stream) {
  unsigned blocks = 0;
  if (!src || !dst || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16 || !grid_of(bytes / 16, &blocks))
    return -1;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (s < d + bytes && d < s + bytes) return -1;
  const long cap = cap_bytes(wgs_per_cu);
  if (cap < 0) return -3;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kThreads), static_cast<unsigned>(cap),
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Runs `blocks` residency workgroups with `lds_bytes` of dynamic LDS each; rec
// (device, 8-byte aligned) receives 3 * blocks values.  sleeps <= 100000.
int zprobe_residency(unsigned long long* rec, uint32_t blocks, uint32_t lds_bytes, uint32_t sleeps,
                     void* stream) {
  if (!rec || blocks == 0 || blocks > 0x7FFFFFFFu || sleeps > 100000 ||
      reinterpret_cast<uintptr_t>(rec) % 8)
    return -1;
  hipLaunchKernelGGL(residency_kernel, dim3(blocks), dim3(kThreads), lds_bytes,
                     static_cast<hipStream_t>(stream), rec, sleeps);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
