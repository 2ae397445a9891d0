// Launch interfaces of the two device kernels (internal to libzero).
#ifndef ZERO_KERNELS_H_
#define ZERO_KERNELS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zero {

// One bucket (or chunk) of the owner's reduce.  Slice columns c in
// [c_lo, c_hi) are reduced; output element of column c is out32[c + delta].
struct ReduceLaunch {
  const uint16_t* rows;  // row k at rows + k * stride
  uint64_t stride;
  uint32_t nd;
  uint64_t c_lo, c_hi;
  int64_t delta;
  float* out32;     // nullable (not both)
  uint16_t* out16;  // nullable
  float inv_nd;
};

// One Adam step over n elements.  p16 (nullable) points at the slot of
// element 0 in the fp16 parameter window.
struct AdamLaunch {
  float* master;
  float* m;
  float* v;
  const void* grad;
  int grad_is_fp16;
  uint16_t* p16;
  uint64_t n;
  float b1, b2, c1, c2, eps, step, isb;
};

// The parameters of flat [lo, lo + n) gathered from the rank shards: row k at
// shards + k * stride holds flat [k * s, (k + 1) * s).
struct GatherLaunch {
  const uint16_t* shards;
  uint64_t stride;
  uint64_t s;
  uint64_t lo, n;
  uint16_t* out;
};

// A gather crossing more rank shards than this runs as one element-wise launch
// instead of one copy per shard piece.
constexpr uint64_t kMaxGatherPieces = 16;

// All return hipSuccess or the launch error.  `cus` is the device's compute
// unit count, used to size grid-stride launches.
hipError_t launch_reduce(const ReduceLaunch& a, int cus, hipStream_t stream);
hipError_t launch_adam(const AdamLaunch& a, int cus, hipStream_t stream);
hipError_t launch_gather(const GatherLaunch& a, hipStream_t stream);

}  // namespace zero

#endif  // ZERO_KERNELS_H_
