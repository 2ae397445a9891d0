// Host paths of libzero called from several threads at once (built with
// ThreadSanitizer on the host side only; no device call is made): geometry,
// bucket intersection, row stride, Adam scalars, the memory and communication
// models, and failing calls whose per-thread error messages must be their own.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "zero.h"

static std::atomic<int> g_bad{0};

static void worker(int id) {
  char want[64];
  for (int it = 0; it < 5000; ++it) {
    zero_geom_t g;
    const uint32_t nd = 3 + (id + it) % 61, rank = (uint32_t)(it % nd);
    const uint64_t psi = 1000003ull + (uint64_t)id * 7919u;
    if (zero_shard_geometry(psi, nd, rank, &g) != ZERO_OK) ++g_bad;
    uint64_t lo = 0, hi = 0;
    if (zero_bucket_intersect(&g, 0, psi / 2, &lo, &hi) != ZERO_OK || hi < lo) ++g_bad;
    uint64_t st = 0;
    if (zero_row_stride((uint64_t)it * 977u + 1, &st) != ZERO_OK || st % 64) ++g_bad;
    float sc[7];
    if (zero_adam_scalars(1e-4, 0.9, 0.999, 1e-8, (uint64_t)it + 1, sc) != ZERO_OK) ++g_bad;
    if (zero_memory_model_k(psi, nd, it % 4, 12.0) <= 0.0) ++g_bad;
    zero_comm_t c;
    if (zero_comm_volume(psi, nd, it % 4, &c) != ZERO_OK) ++g_bad;
    // a failing call whose message names this thread's values
    const uint64_t stride = 24 - (uint64_t)(id % 20);
    zero_geom_t g2;
    zero_shard_geometry(100, 4, 1, &g2);
    const uint16_t* fake16 = (const uint16_t*)0x10000;
    float* fake32 = (float*)0x10000;
    if (zero_reduce_shard(&g2, 25, 25, fake16, stride, fake32, NULL, NULL) != ZERO_E_RANGE) ++g_bad;
    snprintf(want, sizeof want, "slice_stride %llu ", (unsigned long long)stride);
    if (!strstr(zero_last_error(), want)) ++g_bad;
  }
}

int main() {
  std::vector<std::thread> ts;
  for (int i = 0; i < 8; ++i) ts.emplace_back(worker, i);
  for (auto& t : ts) t.join();
  if (g_bad.load()) {
    printf("abi thread check: %d failures\n", g_bad.load());
    return 1;
  }
  printf("abi thread check ok\n");
  return 0;
}
