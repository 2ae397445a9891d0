// Index plan of the owner's reduce (internal to libzero): which columns each
// thread reduces, with which load and store widths, and where its outputs go.
// The host launch code, the kernel and a CPU check
// (tests/native/reduce_plan_check.cpp, built with g++) all compile these same
// functions, so the kernel's indexing can be verified without a GPU.
#ifndef ZERO_REDUCE_PLAN_H_
#define ZERO_REDUCE_PLAN_H_

#include <stdint.h>

#ifdef __HIPCC__
#define ZERO_HD __host__ __device__
#else
#define ZERO_HD
#endif

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

constexpr int kReduceCols = 8;  // columns per thread (one 16-byte fp16 load per row)

// The kernel arguments.  Thread gi takes the group of 8 columns starting at
// col0 + 8 gi; a group wholly inside [c_lo, c_hi) is a full group (vector
// loads and stores), any other is a ragged edge group (element by element).
struct ReduceArgs {
  const uint16_t* rows;
  uint64_t stride;
  uint32_t nd;
  uint64_t col0;     // first column of group 0 (a multiple of 8)
  uint64_t ngroups;  // groups of 8 columns
  uint64_t c_lo, c_hi;
  int64_t delta;
  float* out32;
  uint16_t* out16;
  float inv;
  int st32;          // 4: 16-byte stores, 2: 8-byte, 1: 4-byte
  int st16;          // 8: 16-byte stores, 4: 8-byte, 2: 4-byte, 1: 2-byte
};

// The first column of thread gi's group; true for a full group.
ZERO_HD inline bool reduce_group(const ReduceArgs& a, uint64_t gi, uint64_t* c) {
  *c = a.col0 + gi * kReduceCols;
  return *c >= a.c_lo && *c + kReduceCols <= a.c_hi;
}

// Fills the kernel arguments of a launch; *width gets the byte width of the row
// loads of full groups (the widest that every row start allows: group columns
// start a multiple of 8 elements, 16 bytes, from the row start) and *groups
// the number of threads.
inline ReduceArgs reduce_plan(const ReduceLaunch& L, int* width, uint64_t* groups) {
  ReduceArgs a;
  a.rows = L.rows;
  a.stride = L.stride;
  a.nd = L.nd;
  a.c_lo = L.c_lo;
  a.c_hi = L.c_hi;
  a.col0 = L.c_lo & ~static_cast<uint64_t>(kReduceCols - 1);
  a.ngroups = (L.c_hi - a.col0 + kReduceCols - 1) / kReduceCols;
  a.delta = L.delta;
  a.out32 = L.out32;
  a.out16 = L.out16;
  a.inv = L.inv_nd;
  const uintptr_t ra = reinterpret_cast<uintptr_t>(L.rows) | (2 * L.stride) | 16;
  *width = static_cast<int>(ra & (~ra + 1));          // lowest set bit, at most 16
  // Alignment of the output addresses of full groups: column col0 + 8j maps to
  // out32 + col0 + delta + 8j, so the alignment class is the same for all.
  const uint64_t o0 = a.col0 + static_cast<uint64_t>(a.delta);
  a.st32 = 1;
  if (L.out32) {
    const uintptr_t b32 = reinterpret_cast<uintptr_t>(L.out32) + 4 * o0;
    a.st32 = (b32 % 16 == 0) ? 4 : (b32 % 8 == 0) ? 2 : 1;
  }
  a.st16 = 1;
  if (L.out16) {
    const uintptr_t b16 = reinterpret_cast<uintptr_t>(L.out16) + 2 * o0;
    a.st16 = (b16 % 16 == 0) ? 8 : (b16 % 8 == 0) ? 4 : (b16 % 4 == 0) ? 2 : 1;
  }
  *groups = a.ngroups;
  return a;
}

}  // namespace zero

#endif  // ZERO_REDUCE_PLAN_H_
