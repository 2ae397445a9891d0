// Exercises every host-side path of the C ABI (include/zero.h) that runs
// without a device: the memory and communication models, the geometry, the
// Adam scalars, and every argument error of the device entry points, which
// are rejected before any HIP call.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side by tests/test_host_sanitizers.py;
// prints "abi host check ok" and exits 0 when every expectation holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zero.h"

static int g_fail = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
              __LINE__, #c);                                        \
      g_fail = 1;                                                   \
    }                                                               \
  } while (0)

int main() {
  // memory model: the guide's printed figures and the general-K form
  EXPECT(zero_memory_model(7500000000ull, 64, 0) == 120e9);
  EXPECT(zero_memory_model(7500000000ull, 64, 1) == 31.40625e9);
  EXPECT(zero_memory_model(7500000000ull, 64, 2) == 16.640625e9);
  EXPECT(zero_memory_model(7500000000ull, 64, 3) == 1.875e9);
  EXPECT(zero_memory_model_k(1000, 4, 2, 12.0) == zero_memory_model(1000, 4, 2));
  EXPECT(zero_memory_model(10, 0, 0) < 0 && strlen(zero_last_error()) > 0);
  EXPECT(zero_memory_model(10, 4, 7) < 0);
  EXPECT(zero_memory_model_k(10, 4, 0, -1.0) < 0);
  EXPECT(zero_memory_model_k(10, 4, 0, NAN) < 0);

  zero_comm_t c;
  EXPECT(zero_comm_volume(1000, 4, 3, &c) == ZERO_OK && c.all_gathers == 2 &&
         c.reduce_scatters == 1 && c.elems == 3000.0 && c.elems_sent_per_rank == 2250.0);
  EXPECT(zero_comm_volume(1000, 1, 2, &c) == ZERO_OK && c.elems_sent_per_rank == 0.0);
  EXPECT(zero_comm_volume(1000, 4, 4, &c) == ZERO_E_INVAL);
  EXPECT(zero_comm_volume(1000, 4, 2, NULL) == ZERO_E_INVAL);

  // geometry, including trailing empty shards and the largest sizes
  zero_geom_t g;
  EXPECT(zero_shard_geometry(10, 4, 3, &g) == ZERO_OK && g.offset == 9 && g.len == 1);
  EXPECT(zero_shard_geometry(9, 4, 3, &g) == ZERO_OK && g.offset == 9 && g.len == 0);
  EXPECT(zero_shard_geometry(UINT64_MAX, 7, 6, &g) == ZERO_OK && g.offset + g.len == UINT64_MAX);
  EXPECT(zero_shard_geometry(0, 4, 0, &g) == ZERO_E_INVAL);
  EXPECT(zero_shard_geometry(10, 4, 4, &g) == ZERO_E_INVAL);
  EXPECT(zero_shard_geometry(10, 4, 0, NULL) == ZERO_E_INVAL);
  uint64_t lo = 0, hi = 0;
  EXPECT(zero_shard_geometry(100, 4, 1, &g) == ZERO_OK);
  EXPECT(zero_bucket_intersect(&g, 20, 10, &lo, &hi) == ZERO_OK && lo == 25 && hi == 30);
  EXPECT(zero_bucket_intersect(&g, 95, 10, &lo, &hi) == ZERO_E_RANGE);
  EXPECT(zero_bucket_intersect(&g, UINT64_MAX - 3, 10, &lo, &hi) == ZERO_E_RANGE);
  EXPECT(zero_bucket_intersect(NULL, 0, 1, &lo, &hi) == ZERO_E_INVAL);
  uint64_t st = 0;
  EXPECT(zero_row_stride(1ull << 22, &st) == ZERO_OK && st == (1ull << 22) + 1024);
  EXPECT(zero_row_stride(UINT64_MAX - 1087, &st) == ZERO_OK && st % 64 == 0);
  EXPECT(zero_row_stride(UINT64_MAX - 1086, &st) == ZERO_E_RANGE);
  EXPECT(zero_row_stride(UINT64_MAX, &st) == ZERO_E_RANGE);
  EXPECT(zero_row_stride(5, NULL) == ZERO_E_INVAL);

  // Adam scalars and their argument checks
  float sc[7];
  EXPECT(zero_adam_scalars(1e-3, 0.9, 0.999, 1e-8, 1, sc) == ZERO_OK);
  EXPECT(sc[0] == 0.9f && sc[1] == 0.999f && sc[4] == 1e-8f);
  EXPECT(zero_adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0, sc) == ZERO_E_INVAL);
  EXPECT(zero_adam_scalars(1e-3, 1.0, 0.999, 1e-8, 1, sc) == ZERO_E_INVAL);
  EXPECT(zero_adam_scalars(NAN, 0.9, 0.999, 1e-8, 1, sc) == ZERO_E_INVAL);
  EXPECT(zero_adam_scalars(1e-3, 0.9, 0.999, 1e-8, UINT64_MAX, sc) == ZERO_OK);

  // device entry points: every rejection happens before any HIP call
  uint16_t* fake16 = (uint16_t*)(uintptr_t)0x10000;
  float* fake32 = (float*)(uintptr_t)0x10000;
  EXPECT(zero_reduce_shard(NULL, 0, 1, fake16, 1, fake32, NULL, NULL) == ZERO_E_INVAL);
  EXPECT(zero_reduce_shard(&g, 90, 20, fake16, 20, fake32, NULL, NULL) == ZERO_E_RANGE);
  EXPECT(zero_reduce_shard(&g, 25, 25, NULL, 25, fake32, NULL, NULL) == ZERO_E_INVAL);
  EXPECT(zero_reduce_shard(&g, 25, 25, fake16, 25, NULL, NULL, NULL) == ZERO_E_INVAL);
  EXPECT(zero_reduce_shard(&g, 25, 25, fake16, 24, fake32, NULL, NULL) == ZERO_E_RANGE);
  EXPECT(zero_reduce_shard(&g, 25, 25, fake16, 1ull << 63, fake32, NULL, NULL) == ZERO_E_RANGE);
  EXPECT(zero_reduce_shard(&g, 25, 25, fake16 + 0, 25, (float*)((char*)fake32 + 2), NULL,
                           NULL) == ZERO_E_ALIGN);
  EXPECT(zero_reduce_shard(&g, 0, 10, NULL, 0, NULL, NULL, NULL) == ZERO_OK);   // misses the shard
  {
    zero_geom_t big;
    EXPECT(zero_shard_geometry(1ull << 30, (1u << 24) + 1, 0, &big) == ZERO_OK);
    EXPECT(zero_reduce_shard(&big, 0, 10, fake16, 10, fake32, NULL, NULL) == ZERO_E_RANGE);
  }
  zero_geom_t bad = g;
  bad.offset += 1;
  EXPECT(zero_reduce_shard(&bad, 25, 25, fake16, 25, fake32, NULL, NULL) == ZERO_E_INVAL);

  zero_shard_t s;
  memset(&s, 0, sizeof s);
  s.master = s.m = s.v = fake32;
  s.grad = fake32;
  s.param16 = fake16;
  s.param16_origin = 0;
  s.param16_len = 100;
  EXPECT(zero_adam_step_shard(&g, NULL, 1e-3, 0.9, 0.999, 1e-8, 1, NULL) == ZERO_E_INVAL);
  EXPECT(zero_adam_step_shard(&g, &s, 1e-3, 0.9, 0.999, 1e-8, 0, NULL) == ZERO_E_INVAL);
  s.param16_len = 49;
  EXPECT(zero_adam_step_shard(&g, &s, 1e-3, 0.9, 0.999, 1e-8, 1, NULL) == ZERO_E_RANGE);
  s.param16_len = 100;
  s.param16_origin = UINT64_MAX - 10;
  EXPECT(zero_adam_step_shard(&g, &s, 1e-3, 0.9, 0.999, 1e-8, 1, NULL) == ZERO_E_RANGE);
  s.param16_origin = 0;
  s.grad_is_fp16 = 2;
  EXPECT(zero_adam_step_shard(&g, &s, 1e-3, 0.9, 0.999, 1e-8, 1, NULL) == ZERO_E_INVAL);
  s.grad_is_fp16 = 0;
  s.master = (float*)((char*)fake32 + 2);
  EXPECT(zero_adam_step_shard(&g, &s, 1e-3, 0.9, 0.999, 1e-8, 1, NULL) == ZERO_E_ALIGN);

  EXPECT(zero_gather_params(100, 0, 0, 1, fake16, 25, fake16, NULL) == ZERO_E_INVAL);
  EXPECT(zero_gather_params(100, 4, 90, 11, fake16, 25, fake16, NULL) == ZERO_E_RANGE);
  EXPECT(zero_gather_params(100, 4, 10, 10, fake16, 24, fake16, NULL) == ZERO_E_RANGE);
  EXPECT(zero_gather_params(100, 4, 10, 10, fake16, 1ull << 62, fake16, NULL) == ZERO_E_RANGE);
  EXPECT(zero_gather_params(100, 4, 10, 0, NULL, 0, NULL, NULL) == ZERO_OK);

  int wgs = 0;
  uint32_t lds = 0;
  EXPECT(zero_launch_occupancy(6, &wgs, &lds) == ZERO_E_INVAL);
  EXPECT(zero_launch_occupancy(-1, &wgs, NULL) == ZERO_E_INVAL);
  EXPECT(zero_launch_occupancy(ZERO_KERNEL_ADAM_G32, NULL, &lds) == ZERO_E_INVAL);

  if (g_fail) return 1;
  printf("abi host check ok\n");
  return 0;
}
