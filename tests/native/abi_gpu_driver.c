/*
 * A plain C consumer of libzero: one rank's reduce of one bucket and a few Adam
 * steps through the C ABI alone, on device memory from hipMalloc and a HIP
 * stream of its own (no Python, no torch).  Inputs come from a file, outputs go
 * to a file; the test that runs it compares them with the oracle.
 *
 * usage: abi_gpu_driver <in> <out>
 * in (little endian):
 *   u64 psi; u32 nd, rank; u64 bucket_offset, bucket_len, stride; u32 steps, pad;
 *   f64 lr, beta1, beta2, eps;
 *   u16 rows[nd * stride]             row k = rank k's fp16 gradient over the bucket
 *   f32 master[S], m[S], v[S]         S = the rank's shard length
 * out:
 *   f32 grad32[S] (zeros outside the bucket), master[S], m[S], v[S];
 *   u16 param16[psi] (zeros outside the rank's slot)
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero.h"

#define HIP_OK(x)                                                             \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
      exit(3);                                                                \
    }                                                                         \
  } while (0)

#define ZERO_OK_OR_DIE(x)                                                     \
  do {                                                                        \
    int rc_ = (x);                                                            \
    if (rc_ != ZERO_OK) {                                                     \
      fprintf(stderr, "%s failed (%d): %s\n", #x, rc_, zero_last_error());   \
      exit(4);                                                                \
    }                                                                         \
  } while (0)

static void read_exact(FILE* f, void* p, size_t n) {
  if (fread(p, 1, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
}

static void write_exact(FILE* f, const void* p, size_t n) {
  if (fwrite(p, 1, n, f) != n) {
    fprintf(stderr, "short write\n");
    exit(2);
  }
}

static void* host_alloc(size_t n) {
  void* p = calloc(n ? n : 1, 1);
  if (!p) {
    fprintf(stderr, "out of host memory\n");
    exit(2);
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <in> <out>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 2;
  }
  uint64_t psi, bucket_offset, bucket_len, stride;
  uint32_t nd, rank, steps, pad;
  double lr, beta1, beta2, eps;
  read_exact(in, &psi, 8);
  read_exact(in, &nd, 4);
  read_exact(in, &rank, 4);
  read_exact(in, &bucket_offset, 8);
  read_exact(in, &bucket_len, 8);
  read_exact(in, &stride, 8);
  read_exact(in, &steps, 4);
  read_exact(in, &pad, 4);
  read_exact(in, &lr, 8);
  read_exact(in, &beta1, 8);
  read_exact(in, &beta2, 8);
  read_exact(in, &eps, 8);
  if (nd == 0 || nd > 4096 || psi == 0 || psi > (1ull << 28) || stride > (1ull << 28) ||
      steps > 1000) {
    fprintf(stderr, "input out of the driver's range\n");
    return 2;
  }

  zero_geom_t g;
  ZERO_OK_OR_DIE(zero_shard_geometry(psi, nd, rank, &g));
  const size_t S = (size_t)g.len;
  const size_t nrows = (size_t)nd * (size_t)stride;
  uint16_t* h_rows = (uint16_t*)host_alloc(nrows * 2);
  float* h_state = (float*)host_alloc(3 * S * 4);
  read_exact(in, h_rows, nrows * 2);
  read_exact(in, h_state, 3 * S * 4);
  fclose(in);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  uint16_t *d_rows, *d_p16;
  float *d_grad, *d_state;
  HIP_OK(hipMalloc((void**)&d_rows, nrows * 2 + 2));
  HIP_OK(hipMalloc((void**)&d_grad, S * 4 + 4));
  HIP_OK(hipMalloc((void**)&d_state, 3 * S * 4 + 4));
  HIP_OK(hipMalloc((void**)&d_p16, (size_t)psi * 2));
  HIP_OK(hipMemcpy(d_rows, h_rows, nrows * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_state, h_state, 3 * S * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(d_grad, 0, S * 4 + 4));
  HIP_OK(hipMemset(d_p16, 0, (size_t)psi * 2));

  ZERO_OK_OR_DIE(zero_reduce_shard(&g, bucket_offset, bucket_len, d_rows, stride, d_grad, NULL,
                                   (void*)stream));
  zero_shard_t s;
  memset(&s, 0, sizeof(s));
  s.master = d_state;
  s.m = d_state + S;
  s.v = d_state + 2 * S;
  s.grad = d_grad;
  s.grad_is_fp16 = 0;
  s.param16 = d_p16;
  s.param16_origin = 0;
  s.param16_len = psi;
  for (uint32_t t = 1; t <= steps; ++t)
    ZERO_OK_OR_DIE(zero_adam_step_shard(&g, &s, lr, beta1, beta2, eps, t, (void*)stream));
  HIP_OK(hipStreamSynchronize(stream));

  float* h_grad = (float*)host_alloc(S * 4);
  uint16_t* h_p16 = (uint16_t*)host_alloc((size_t)psi * 2);
  HIP_OK(hipMemcpy(h_grad, d_grad, S * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_state, d_state, 3 * S * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_p16, d_p16, (size_t)psi * 2, hipMemcpyDeviceToHost));
  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 2;
  }
  write_exact(out, h_grad, S * 4);
  write_exact(out, h_state, 3 * S * 4);
  write_exact(out, h_p16, (size_t)psi * 2);
  fclose(out);

  HIP_OK(hipFree(d_rows));
  HIP_OK(hipFree(d_grad));
  HIP_OK(hipFree(d_state));
  HIP_OK(hipFree(d_p16));
  HIP_OK(hipStreamDestroy(stream));
  free(h_rows);
  free(h_state);
  free(h_grad);
  free(h_p16);
  printf("abi gpu driver ok: shard [%llu, +%llu), %u Adam steps\n",
         (unsigned long long)g.offset, (unsigned long long)g.len, steps);
  return 0;
}
