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

// The device a launch runs on.
struct DeviceInfo {
  int cus;         // compute units
  int lds_per_cu;  // LDS bytes per compute unit
};

// Dynamic LDS bytes per workgroup that let at most `wgs` workgroups share a
// compute unit.  The kernels do not use this memory: it caps how many
// workgroups (and so how many concurrent access streams) each CU runs, which
// on MI355X raises the HBM rate of these streaming kernels (measured: the
// reduce 6.1 -> 6.5 TB/s at 8 per CU, Adam 6.0 -> 6.55 TB/s at 10).
inline unsigned occupancy_cap_bytes(const DeviceInfo& d, int wgs) {
  const unsigned b = static_cast<unsigned>(d.lds_per_cu) / static_cast<unsigned>(wgs);
  const unsigned granule = 512;
  const unsigned capped = b > 65536 ? 65536 : b;
  return (capped / granule) * granule;
}

// All return hipSuccess or the launch error.
hipError_t launch_reduce(const ReduceLaunch& a, const DeviceInfo& d, hipStream_t stream);
hipError_t launch_adam(const AdamLaunch& a, const DeviceInfo& d, hipStream_t stream);
hipError_t launch_gather(const GatherLaunch& a, hipStream_t stream);

}  // namespace zero

#endif  // ZERO_KERNELS_H_
