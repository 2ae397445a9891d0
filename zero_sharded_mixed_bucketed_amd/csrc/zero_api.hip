// Host side of libzero: argument validation, shard and bucket geometry, the
// memory model, fp64 derivation of the Adam scalars, and launches.  Every check
// runs before the first HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>

#include "kernels.h"
#include "zero.h"

namespace {

thread_local char g_err[512];

constexpr uint32_t kMaxReduceNd = 1u << 24;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return ZERO_OK;
}

// Resident workgroups per compute unit of `fn` with `lds` bytes of dynamic LDS,
// from the runtime's occupancy calculator.
int occupancy(const void* fn, int threads, unsigned lds, int* wgs) {
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs, fn, threads, lds);
  if (e != hipSuccess)
    return fail(ZERO_E_DEVICE, "hipOccupancyMaxActiveBlocksPerMultiprocessor: %s",
                hipGetErrorString(e));
  return ZERO_OK;
}

// gfx950 allocates LDS to a workgroup in granules of 1,280 bytes (128 per
// 160 KiB): measured with a probe that records which workgroups overlap on a
// compute unit, a request of L bytes holds floor(160 KiB / roundup(L, 1280))
// workgroups per CU at every L from 8 to 32 KiB in 512-byte steps.  The
// runtime's occupancy calculator rounds to 512 bytes only, and reports one
// workgroup more than the hardware holds at, e.g., 16,384 bytes (10 against
// 9).  Sizes that are multiples of both granules are rounded by neither, so
// the calculator and the hardware agree on them: the cap is searched among
// those.
constexpr unsigned kLdsStep = 2560;  // lcm(1280, 512)

// The dynamic LDS bytes that leave exactly `want` workgroups of `fn` resident
// per CU of device `dev`: the largest multiple of kLdsStep, up to the
// per-workgroup limit, at which the occupancy calculator still allows `want`
// (residency does not grow with LDS, so bisection finds it).  Fails loudly
// when no such size gives exactly `want` -- the kernels would then run at a
// residency they were not tuned for.
int resolve_cap(const void* fn, int threads, int want, int dev, const char* name,
                unsigned* out) {
  int max_lds = 0;
  hipError_t e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess)
    return fail(ZERO_E_DEVICE, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (max_lds < static_cast<int>(kLdsStep))
    return fail(ZERO_E_DEVICE, "device %d reports %d bytes of LDS per workgroup", dev, max_lds);
  int n = 0, rc;
  if ((rc = occupancy(fn, threads, 0, &n))) return rc;
  if (n < want)
    return fail(ZERO_E_DEVICE, "%s: only %d workgroups fit a compute unit of device %d, "
                "the launch is tuned for %d", name, n, dev, want);
  // in units of kLdsStep: occ(lo) >= want > occ(hi)
  unsigned lo = 0, hi = static_cast<unsigned>(max_lds) / kLdsStep + 1;
  while (hi - lo > 1) {
    const unsigned mid = lo + (hi - lo) / 2;
    if ((rc = occupancy(fn, threads, mid * kLdsStep, &n))) return rc;
    if (n >= want) lo = mid; else hi = mid;
  }
  if ((rc = occupancy(fn, threads, lo * kLdsStep, &n))) return rc;
  if (n != want)
    return fail(ZERO_E_DEVICE, "%s: no dynamic LDS size holds a compute unit of device %d to "
                "%d workgroups (%d at %u bytes)", name, dev, want, n, lo * kLdsStep);
  *out = lo * kLdsStep;
  return ZERO_OK;
}

// Launch parameters of each device, resolved on the first call that launches
// on it and kept for the life of the process.
std::mutex g_caps_mu;
std::map<int, zero::DeviceCaps> g_caps;

int device_caps(zero::DeviceCaps* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZERO_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_caps_mu);
  auto it = g_caps.find(dev);
  if (it != g_caps.end()) {
    *out = it->second;
    return ZERO_OK;
  }
  zero::DeviceCaps c;
  e = hipDeviceGetAttribute(&c.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess)
    return fail(ZERO_E_DEVICE, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (c.cus <= 0) return fail(ZERO_E_DEVICE, "device %d reports %d compute units", dev, c.cus);
  int rc;
  for (int i = 0; i < 4; ++i) {
    if ((rc = resolve_cap(zero::reduce_kernel_fn(zero::kReduceWidths[i]), zero::kReduceThreads,
                          zero::kReduceWgsPerCu, dev, "reduce_kernel", &c.reduce_lds[i])))
      return rc;
  }
  for (int i = 0; i < 2; ++i) {
    if ((rc = resolve_cap(zero::adam_kernel_fn(i), zero::kAdamThreads, zero::kAdamWgsPerCu, dev,
                          "adam_vec_kernel", &c.adam_lds[i])))
      return rc;
  }
  g_caps.emplace(dev, c);
  *out = c;
  return ZERO_OK;
}

void geometry(uint64_t psi, uint32_t nd, uint32_t rank, zero_geom_t* out) {
  const uint64_t s = psi / nd + (psi % nd != 0);
  // lo = min(rank * S, psi) and hi = lo + min(S, psi - lo), computed without
  // overflow: for psi near 2^64, rank * S and (rank + 1) * S can exceed it.
  uint64_t lo = psi;
  if (rank == 0 || s <= psi / rank) lo = static_cast<uint64_t>(rank) * s;
  if (lo > psi) lo = psi;
  const uint64_t len = (psi - lo < s) ? psi - lo : s;
  out->psi = psi;
  out->nd = nd;
  out->rank = rank;
  out->offset = lo;
  out->len = len;
}

int check_geom(const zero_geom_t* g) {
  if (!g) return fail(ZERO_E_INVAL, "geometry is NULL");
  if (g->nd == 0 || g->rank >= g->nd || g->psi == 0)
    return fail(ZERO_E_INVAL, "geometry: need psi > 0, nd > 0 and rank < nd");
  zero_geom_t want;
  geometry(g->psi, g->nd, g->rank, &want);
  if (want.offset != g->offset || want.len != g->len)
    return fail(ZERO_E_INVAL,
                "geometry: rank %u of %u over psi=%llu owns [%llu, +%llu), not [%llu, +%llu)",
                g->rank, g->nd, (unsigned long long)g->psi, (unsigned long long)want.offset,
                (unsigned long long)want.len, (unsigned long long)g->offset,
                (unsigned long long)g->len);
  return ZERO_OK;
}

int check_bucket(const zero_geom_t* g, uint64_t off, uint64_t len) {
  if (off > g->psi || len > g->psi - off)
    return fail(ZERO_E_RANGE, "bucket [%llu, +%llu) leaves the parameter vector (psi=%llu)",
                (unsigned long long)off, (unsigned long long)len,
                (unsigned long long)g->psi);
  return ZERO_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_hparams(double lr, double beta1, double beta2, double eps, uint64_t t) {
  if (t == 0) return fail(ZERO_E_INVAL, "step counts from 1");
  if (!isfinite(lr)) return fail(ZERO_E_INVAL, "lr must be finite");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
    return fail(ZERO_E_INVAL, "betas must lie in [0, 1)");
  if (!(eps > 0.0) || !isfinite(eps)) return fail(ZERO_E_INVAL, "eps must be finite and > 0");
  return ZERO_OK;
}

void derive_scalars(double lr, double beta1, double beta2, double eps, uint64_t t,
                    float out[7]) {
  const double bc1 = 1.0 - pow(beta1, static_cast<double>(t));
  const double bc2 = 1.0 - pow(beta2, static_cast<double>(t));
  out[0] = static_cast<float>(beta1);
  out[1] = static_cast<float>(beta2);
  out[2] = static_cast<float>(1.0 - beta1);
  out[3] = static_cast<float>(1.0 - beta2);
  out[4] = static_cast<float>(eps);
  out[5] = static_cast<float>(lr / bc1);
  out[6] = static_cast<float>(1.0 / sqrt(bc2));
}

}  // namespace

extern "C" {

double zero_memory_model_k(uint64_t psi, uint32_t nd, int stage, double k) {
  if (nd == 0) {
    fail(ZERO_E_INVAL, "nd must be >= 1");
    return -1.0;
  }
  if (!(k >= 0.0) || !isfinite(k)) {
    fail(ZERO_E_INVAL, "k must be finite and >= 0");
    return -1.0;
  }
  const double p = static_cast<double>(psi);
  const double n = static_cast<double>(nd);
  const double params = 2.0 * p, grads = 2.0 * p, optim = k * p;
  switch (stage) {
    case ZERO_STAGE_DP: ok(); return params + grads + optim;
    case ZERO_STAGE_OS: ok(); return params + grads + optim / n;
    case ZERO_STAGE_OS_G: ok(); return params + (grads + optim) / n;
    case ZERO_STAGE_OS_G_P: ok(); return (params + grads + optim) / n;
    default: fail(ZERO_E_INVAL, "stage must be 0..3"); return -1.0;
  }
}

double zero_memory_model(uint64_t psi, uint32_t nd, int stage) {
  return zero_memory_model_k(psi, nd, stage, 12.0);
}

int zero_comm_volume(uint64_t psi, uint32_t nd, int stage, zero_comm_t* out) {
  if (!out) return fail(ZERO_E_INVAL, "out is NULL");
  if (nd == 0) return fail(ZERO_E_INVAL, "nd must be >= 1");
  if (stage < ZERO_STAGE_DP || stage > ZERO_STAGE_OS_G_P)
    return fail(ZERO_E_INVAL, "stage must be 0..3");
  out->reduce_scatters = 1;
  out->all_gathers = stage == ZERO_STAGE_OS_G_P ? 2 : 1;
  const double c = static_cast<double>(out->reduce_scatters + out->all_gathers);
  const double p = static_cast<double>(psi);
  out->elems = c * p;
  out->elems_sent_per_rank = c * p * static_cast<double>(nd - 1) / static_cast<double>(nd);
  out->bytes_sent_per_rank = 2.0 * out->elems_sent_per_rank;
  return ok();
}

int zero_shard_geometry(uint64_t psi, uint32_t nd, uint32_t rank, zero_geom_t* out) {
  if (!out) return fail(ZERO_E_INVAL, "out is NULL");
  if (nd == 0 || rank >= nd || psi == 0)
    return fail(ZERO_E_INVAL, "need psi > 0, nd > 0 and rank < nd");
  geometry(psi, nd, rank, out);
  return ok();
}

int zero_bucket_intersect(const zero_geom_t* g, uint64_t bucket_offset, uint64_t bucket_len,
                          uint64_t* lo, uint64_t* hi) {
  int rc = check_geom(g);
  if (rc) return rc;
  if (!lo || !hi) return fail(ZERO_E_INVAL, "lo/hi is NULL");
  if ((rc = check_bucket(g, bucket_offset, bucket_len))) return rc;
  uint64_t a = bucket_offset > g->offset ? bucket_offset : g->offset;
  uint64_t b = bucket_offset + bucket_len;
  if (b > g->offset + g->len) b = g->offset + g->len;
  if (b < a) b = a;
  *lo = a;
  *hi = b;
  return ok();
}

int zero_row_stride(uint64_t len, uint64_t* stride) {
  if (!stride) return fail(ZERO_E_INVAL, "stride is NULL");
  constexpr uint64_t kLine = 64, kPad = 1024, kMiBElems = (1u << 20) / 2;
  if (len > UINT64_MAX - (kLine - 1) - kPad)
    return fail(ZERO_E_RANGE, "len %llu too large", (unsigned long long)len);
  uint64_t s = (len + kLine - 1) / kLine * kLine;
  if (s != 0 && s % kMiBElems == 0) s += kPad;
  *stride = s;
  return ok();
}

int zero_reduce_shard(const zero_geom_t* g, uint64_t bucket_offset, uint64_t bucket_len,
                      const uint16_t* slices, uint64_t slice_stride, float* grad32,
                      uint16_t* grad16, void* hip_stream) {
  int rc = check_geom(g);
  if (rc) return rc;
  if ((rc = check_bucket(g, bucket_offset, bucket_len))) return rc;
  const uint64_t s_lo = g->offset, s_hi = g->offset + g->len;
  const uint64_t a = bucket_offset > s_lo ? bucket_offset : s_lo;
  const uint64_t b = (bucket_offset + bucket_len) < s_hi ? (bucket_offset + bucket_len) : s_hi;
  if (a >= b) return ok();  // nothing of this bucket is owned here
  // RN32(1/Nd) is 1.0f / float(Nd) only while Nd is exact in fp32
  if (g->nd > kMaxReduceNd)
    return fail(ZERO_E_RANGE, "nd %u exceeds the reduce's limit of 2^24 ranks", g->nd);
  if (!slices) return fail(ZERO_E_INVAL, "slices must not be NULL");
  if (!grad32 && !grad16) return fail(ZERO_E_INVAL, "grad32 and grad16 are both NULL");
  if (slice_stride < bucket_len)
    return fail(ZERO_E_RANGE, "slice_stride %llu < bucket_len %llu",
                (unsigned long long)slice_stride, (unsigned long long)bucket_len);
  if (g->nd > 1 && slice_stride > (UINT64_MAX / 2 - bucket_len) / (g->nd - 1))
    return fail(ZERO_E_RANGE, "slice buffer size overflows");
  if (!aligned(slices, 2) || (grad32 && !aligned(grad32, 4)) || (grad16 && !aligned(grad16, 2)))
    return fail(ZERO_E_ALIGN, "slices/grad16 need 2-byte and grad32 4-byte alignment");
  zero::DeviceCaps dcaps;
  if ((rc = device_caps(&dcaps))) return rc;
  zero::ReduceLaunch L;
  L.rows = slices;
  L.stride = slice_stride;
  L.nd = g->nd;
  L.c_lo = a - bucket_offset;
  L.c_hi = b - bucket_offset;
  // output index of column c is (bucket_offset + c) - shard offset; the
  // difference is taken modulo 2^64 and read back as a signed shift
  L.delta = static_cast<int64_t>(bucket_offset - s_lo);
  L.out32 = grad32;
  L.out16 = grad16;
  L.inv_nd = 1.0f / static_cast<float>(g->nd);
  hipError_t e = zero::launch_reduce(L, dcaps, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(ZERO_E_DEVICE, "reduce launch: %s", hipGetErrorString(e));
  return ok();
}

int zero_adam_scalars(double lr, double beta1, double beta2, double eps, uint64_t step,
                      float out[7]) {
  if (!out) return fail(ZERO_E_INVAL, "out is NULL");
  int rc = check_hparams(lr, beta1, beta2, eps, step);
  if (rc) return rc;
  derive_scalars(lr, beta1, beta2, eps, step, out);
  return ok();
}

int zero_adam_step_shard(const zero_geom_t* g, const zero_shard_t* s, double lr, double beta1,
                         double beta2, double eps, uint64_t step, void* hip_stream) {
  int rc = check_geom(g);
  if (rc) return rc;
  if (!s) return fail(ZERO_E_INVAL, "shard is NULL");
  if ((rc = check_hparams(lr, beta1, beta2, eps, step))) return rc;
  if (g->len == 0) return ok();  // an empty trailing shard
  if (!s->master || !s->m || !s->v || !s->grad)
    return fail(ZERO_E_INVAL, "master, m, v and grad must not be NULL");
  if (s->grad_is_fp16 != 0 && s->grad_is_fp16 != 1)
    return fail(ZERO_E_INVAL, "grad_is_fp16 must be 0 or 1");
  if (s->param16) {
    if (g->offset < s->param16_origin || s->param16_len < g->len ||
        g->offset - s->param16_origin > s->param16_len - g->len)
      return fail(ZERO_E_RANGE, "slot [%llu, +%llu) lies outside the fp16 window [%llu, +%llu)",
                  (unsigned long long)g->offset, (unsigned long long)g->len,
                  (unsigned long long)s->param16_origin, (unsigned long long)s->param16_len);
  }
  if (!aligned(s->master, 4) || !aligned(s->m, 4) || !aligned(s->v, 4) ||
      !aligned(s->grad, s->grad_is_fp16 ? 2 : 4) || (s->param16 && !aligned(s->param16, 2)))
    return fail(ZERO_E_ALIGN, "fp32 arrays need 4-byte, fp16 arrays 2-byte alignment");
  zero::DeviceCaps dcaps;
  if ((rc = device_caps(&dcaps))) return rc;
  float sc[7];
  derive_scalars(lr, beta1, beta2, eps, step, sc);
  zero::AdamLaunch L;
  L.master = s->master;
  L.m = s->m;
  L.v = s->v;
  L.grad = s->grad;
  L.grad_is_fp16 = s->grad_is_fp16;
  L.p16 = s->param16 ? s->param16 + (g->offset - s->param16_origin) : nullptr;
  L.n = g->len;
  L.b1 = sc[0];
  L.b2 = sc[1];
  L.c1 = sc[2];
  L.c2 = sc[3];
  L.eps = sc[4];
  L.step = sc[5];
  L.isb = sc[6];
  hipError_t e = zero::launch_adam(L, dcaps, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(ZERO_E_DEVICE, "adam launch: %s", hipGetErrorString(e));
  return ok();
}

int zero_gather_params(uint64_t psi, uint32_t nd, uint64_t lo, uint64_t len,
                       const uint16_t* shards, uint64_t shard_stride, uint16_t* out,
                       void* hip_stream) {
  if (nd == 0 || psi == 0) return fail(ZERO_E_INVAL, "need psi > 0 and nd > 0");
  if (lo > psi || len > psi - lo)
    return fail(ZERO_E_RANGE, "range [%llu, +%llu) leaves the parameter vector (psi=%llu)",
                (unsigned long long)lo, (unsigned long long)len, (unsigned long long)psi);
  if (len == 0) return ok();
  if (!shards || !out) return fail(ZERO_E_INVAL, "shards and out must not be NULL");
  const uint64_t s = psi / nd + (psi % nd != 0);
  if (shard_stride < s)
    return fail(ZERO_E_RANGE, "shard_stride %llu < shard size %llu",
                (unsigned long long)shard_stride, (unsigned long long)s);
  if (nd > 1 && shard_stride > (UINT64_MAX / 2 - s) / (nd - 1))
    return fail(ZERO_E_RANGE, "shard buffer size overflows");
  if (!aligned(shards, 2) || !aligned(out, 2))
    return fail(ZERO_E_ALIGN, "shards and out need 2-byte alignment");
  zero::GatherLaunch L;
  L.shards = shards;
  L.stride = shard_stride;
  L.s = s;
  L.lo = lo;
  L.n = len;
  L.out = out;
  hipError_t e = zero::launch_gather(L, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(ZERO_E_DEVICE, "gather launch: %s", hipGetErrorString(e));
  return ok();
}

int zero_launch_occupancy(int kernel, int* wgs_per_cu, uint32_t* lds_bytes) {
  if (!wgs_per_cu) return fail(ZERO_E_INVAL, "wgs_per_cu is NULL");
  if (kernel < ZERO_KERNEL_REDUCE_W16 || kernel > ZERO_KERNEL_ADAM_G16)
    return fail(ZERO_E_INVAL, "unknown kernel %d", kernel);
  zero::DeviceCaps dcaps;
  int rc = device_caps(&dcaps);
  if (rc) return rc;
  const bool red = kernel <= ZERO_KERNEL_REDUCE_W2;
  const void* fn = red ? zero::reduce_kernel_fn(zero::kReduceWidths[kernel])
                       : zero::adam_kernel_fn(kernel - ZERO_KERNEL_ADAM_G32);
  const unsigned lds = red ? dcaps.reduce_lds[kernel] : dcaps.adam_lds[kernel - ZERO_KERNEL_ADAM_G32];
  const int threads = red ? zero::kReduceThreads : zero::kAdamThreads;
  if ((rc = occupancy(fn, threads, lds, wgs_per_cu))) return rc;
  if (lds_bytes) *lds_bytes = lds;
  return ok();
}

const char* zero_last_error(void) { return g_err; }

}  // extern "C"
