// Device-side generator of the seeded synthetic inputs.
//
// A second implementation of the generator defined in synth/gen.py: the
// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014) applied to
// key + (i + 1) * 0x9E3779B97F4A7C15, with the top 16 bits indexing a quantile
// table built on the host.  It exists so that full-size inputs (up to 200 GB of
// fp16 gradient rows) can be made where they are consumed; it computes no part
// of the ZeRO method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr unsigned kTailZeroBelow = 655;
constexpr unsigned kTailOutlierBelow = 1311;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint32_t kind,
                                               uint32_t rank) {
  return mix64(seed ^ (static_cast<uint64_t>(kind) << 56) ^ rank);
}

__device__ inline uint16_t grad_value(uint64_t key, uint64_t i,
                                      const uint16_t* __restrict__ table,
                                      const uint16_t* __restrict__ tail,
                                      int heavy) {
  const uint64_t x = mix64(key + (i + 1) * kGamma);
  const unsigned j = static_cast<unsigned>(x >> 48);
  if (heavy) {
    const unsigned u = static_cast<unsigned>((x >> 32) & 0xFFFFu);
    if (u < kTailZeroBelow) return 0;
    if (u < kTailOutlierBelow) return tail[j];
  }
  return table[j];
}

// One thread makes 8 consecutive values of one row; blockIdx.y is the row.
__global__ void __launch_bounds__(256)
grad_rows_kernel(uint16_t* __restrict__ out, uint64_t stride, uint64_t seed,
                 uint32_t kind, uint32_t rank0, uint64_t lo, uint64_t len,
                 const uint16_t* __restrict__ table,
                 const uint16_t* __restrict__ tail, int heavy, int vec_ok) {
  const uint32_t row = blockIdx.y;
  const uint64_t key = stream_key(seed, kind, rank0 + row);
  const uint64_t j0 = (static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (j0 >= len) return;
  uint16_t* dst = out + static_cast<uint64_t>(row) * stride + j0;
  if (vec_ok && j0 + 8 <= len) {
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = grad_value(key, lo + j0 + e, table, tail, heavy);
    uint4 pk;
    pk.x = v[0] | (static_cast<uint32_t>(v[1]) << 16);
    pk.y = v[2] | (static_cast<uint32_t>(v[3]) << 16);
    pk.z = v[4] | (static_cast<uint32_t>(v[5]) << 16);
    pk.w = v[6] | (static_cast<uint32_t>(v[7]) << 16);
    *reinterpret_cast<uint4*>(dst) = pk;
  } else {
    const uint64_t n = (len - j0) < 8 ? (len - j0) : 8;
    for (uint64_t e = 0; e < n; ++e) dst[e] = grad_value(key, lo + j0 + e, table, tail, heavy);
  }
}

__global__ void __launch_bounds__(256)
state_kernel(float* __restrict__ out, uint64_t seed, uint32_t kind, uint64_t lo,
             uint64_t len, const float* __restrict__ table) {
  const uint64_t key = stream_key(seed, kind, 0);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t j = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < len;
       j += stride) {
    const uint64_t x = mix64(key + (lo + j + 1) * kGamma);
    out[j] = table[static_cast<unsigned>(x >> 48)];
  }
}

}  // namespace

extern "C" {

// Fills rows k = 0..nrows-1 of out (row k at out + k * stride, fp16 bit
// patterns) with the gradient stream (seed, kind, rank0 + k) over flat indices
// [lo, lo + len).  Tables are device pointers to 2^16 fp16 entries.  Returns 0,
// or -1 on bad arguments, or -3 if the launch failed.
int zsynth_grad_rows(uint16_t* out, uint64_t stride, uint32_t nrows, uint64_t seed,
                     uint32_t kind, uint32_t rank0, uint64_t lo, uint64_t len,
                     const uint16_t* table, const uint16_t* tail, int heavy,
                     void* stream) {
  if (len == 0 || nrows == 0) return 0;
  if (!out || !table || (heavy && !tail) || stride < len || nrows > 65535) return -1;
  const uint64_t groups = (len + 7) / 8;
  const uint64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffffull) return -1;
  const int vec_ok = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (stride % 8 == 0);
  hipLaunchKernelGGL(grad_rows_kernel, dim3(static_cast<unsigned>(blocks), nrows),
                     dim3(256), 0, static_cast<hipStream_t>(stream), out, stride, seed,
                     kind, rank0, lo, len, table, tail, heavy, vec_ok);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Fills out[0..len) with the fp32 state stream (seed, kind, rank 0) over flat
// indices [lo, lo + len), from a device table of 2^16 fp32 entries.
int zsynth_state(float* out, uint64_t seed, uint32_t kind, uint64_t lo, uint64_t len,
                 const float* table, void* stream) {
  if (len == 0) return 0;
  if (!out || !table) return -1;
  uint64_t blocks = (len + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(state_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, seed, kind, lo, len, table);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
