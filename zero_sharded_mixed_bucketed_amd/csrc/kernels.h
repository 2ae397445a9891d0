// Launch interfaces of the two device kernels (internal to libzero).
#ifndef ZERO_KERNELS_H_
#define ZERO_KERNELS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gather_plan.h"
#include "reduce_plan.h"

namespace zero {

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

// Workgroup size and the cap on resident workgroups per compute unit of the
// two streaming kernels.  The cap is set with dynamic LDS that the kernels do
// not use: fewer concurrent access streams per CU move more bytes per second
// on MI355X.  Measured in one process over true residencies 4 to 32 per CU:
// the reduce (Nd = 64, 25M columns) peaks at 8 (6.47-6.50 TB/s, against 6.06
// uncapped and 6.36-6.39 at 9); Adam (117M elements) peaks at 10 (6.63 TB/s
// with an fp32 gradient and 6.55 with fp16, against 6.12 uncapped and
// 6.54-6.56 / 6.40-6.42 at 9).
constexpr int kReduceThreads = 64;
constexpr int kReduceWgsPerCu = 8;
constexpr int kAdamThreads = 64;
constexpr int kAdamWgsPerCu = 10;

// The reduce instantiations, by the byte width of their row loads.
constexpr int kReduceWidths[4] = {16, 8, 4, 2};

// Entry points of the capped kernels, for the occupancy calculator.
const void* reduce_kernel_fn(int width);       // width: 16, 8, 4 or 2
const void* adam_kernel_fn(int grad_is_fp16);  // 0 or 1

// What the launches on one device use: its compute-unit count, and for each
// capped kernel the dynamic LDS bytes that leave exactly its cap of workgroups
// resident per CU (resolved with the runtime's occupancy calculator on the
// kernel itself, once per device).
struct DeviceCaps {
  int cus;
  unsigned reduce_lds[4];  // by kReduceWidths
  unsigned adam_lds[2];    // fp32 gradient, fp16 gradient
};

// All return hipSuccess or the launch error.
hipError_t launch_reduce(const ReduceLaunch& a, const DeviceCaps& d, hipStream_t stream);
hipError_t launch_adam(const AdamLaunch& a, const DeviceCaps& d, hipStream_t stream);
hipError_t launch_gather(const GatherLaunch& a, hipStream_t stream);

}  // namespace zero

#endif  // ZERO_KERNELS_H_
