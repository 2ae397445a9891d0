/*
 * zero.h -- C ABI of the per-rank data-parallel hot path of ZeRO stages 1 and 2
 * on one MI355X (gfx950).
 *
 * The method (upskillscore guide "ZeRO: particionar estados do treino entre
 * GPUs", section "Como funciona"; llm-engineer card "ZeRO-2", sections
 * "Gradient lifecycle" and "Why all-gather is still needed"): the flat
 * parameter vector of Psi elements is split into Nd contiguous rank-major
 * partitions.  In backward, each gradient bucket is reduce-scattered as soon as
 * it is ready; the owner of a partition keeps only the reduced gradient of its
 * own slice and releases the rest.  In the optimizer step each rank updates
 * only its partition of the fp32 master weights, momentum and variance (mixed-
 * precision Adam, K = 12 bytes per parameter) and its updated fp16 parameters
 * go to their slot of the flat fp16 parameter vector that the all-gather fills.
 *
 * This library is the one-GPU share of that path: zero_reduce_shard is the
 * owner's side of one bucket's reduce-scatter, with the Nd ranks' local
 * gradients handed over as Nd rows of one device buffer; zero_adam_step_shard is
 * the fused sharded Adam step and the fp16 slot write.  For stage 3, where the
 * parameters are partitioned too, zero_gather_params is the receive side of a
 * layer's parameter all-gather.  No collective runs here.
 *
 * Conventions for every entry point:
 *  - Sizes and offsets are element counts (uint64_t).  Flat indices address
 *    the Psi-long parameter vector in forward layer order.
 *  - Device pointers come from the caller, who owns every buffer; the library
 *    allocates nothing per call and keeps no pointer after it returns.
 *  - Device work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns at once; results are valid after the stream
 *    synchronises.  Calls that touch the same buffers must be ordered by the
 *    caller (same stream or events).
 *  - Kernels run on the calling thread's current HIP device; every device
 *    pointer of a call must be memory of that device.
 *  - A negative status is an error.  Arguments are validated before any HIP
 *    call, so a rejected call enqueues nothing and writes nothing.
 *    zero_last_error() returns a message for the calling thread's last error.
 *    Non-finite values in the data are not errors; they propagate per IEEE.
 *  - Several threads may call at once.  The only process-wide state is a cache
 *    of each device's compute-unit count and the dynamic LDS sizes that cap
 *    the streaming kernels' residency (zero_launch_occupancy), resolved under a
 *    lock on first use; the error message is per thread.
 */
#ifndef ZERO_H_
#define ZERO_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_OK 0
#define ZERO_E_INVAL (-1)  /* invalid argument: null pointer, Nd = 0, rank >= Nd, bad stage or hyperparameter, geometry mismatch */
#define ZERO_E_RANGE (-2)  /* a range leaves the parameter vector or a buffer (bucket beyond Psi, stride < length, slot outside the fp16 window) */
#define ZERO_E_ALIGN (-3)  /* a device pointer is not aligned to its element size */
#define ZERO_E_DEVICE (-4) /* the HIP runtime reported an error, or the device cannot hold a streaming kernel to its workgroups-per-CU cap (zero_launch_occupancy) */

/* Stages of zero_memory_model. */
#define ZERO_STAGE_DP 0     /* plain data parallelism: full replica */
#define ZERO_STAGE_OS 1     /* P_os: optimizer states partitioned */
#define ZERO_STAGE_OS_G 2   /* P_os+g: optimizer states and gradients partitioned */
#define ZERO_STAGE_OS_G_P 3 /* P_os+g+p: parameters partitioned too */

/* The partition of one data-parallel rank: flat range [offset, offset + len). */
typedef struct zero_geom {
  uint64_t psi;    /* parameters in the model */
  uint32_t nd;     /* data-parallel degree Nd */
  uint32_t rank;   /* this rank, 0 <= rank < nd */
  uint64_t offset; /* first flat index owned */
  uint64_t len;    /* elements owned */
} zero_geom_t;

/*
 * Model-state bytes per device (guide "ZeRO: particionar estados do treino
 * entre GPUs", section "Como funciona"; worked example in section "Na pratica"):
 * with 2 Psi bytes of fp16 parameters, 2 Psi of fp16 gradients and 12 Psi of
 * optimizer state,
 *   stage 0:  16 Psi            stage 2:  2 Psi + 14 Psi / Nd
 *   stage 1:  4 Psi + 12 Psi/Nd  stage 3:  16 Psi / Nd
 * (stage 2 keeps an fp16 gradient shard, the reading that reproduces the
 * guide's 16.6 GB for 7.5B parameters at Nd = 64).  Pure host arithmetic.
 * Returns the byte count (a real number), or a negative value if nd == 0 or
 * the stage is not 0..3.
 */
double zero_memory_model(uint64_t psi, uint32_t nd, int stage);

/*
 * The same accounting with a general optimizer-state multiplier (guide, "Como
 * funciona": K Psi bytes of optimizer state, K = 12 for mixed-precision Adam):
 *   stage 0: (4 + K) Psi          stage 2: 2 Psi + (2 + K) Psi / Nd
 *   stage 1: 4 Psi + K Psi / Nd   stage 3: (4 + K) Psi / Nd
 * zero_memory_model(psi, nd, stage) == zero_memory_model_k(psi, nd, stage, 12).
 * Returns the byte count, or a negative value if nd == 0, the stage is not
 * 0..3, or k is negative or not finite.
 */
double zero_memory_model_k(uint64_t psi, uint32_t nd, int stage, double k);

/* Per-step communication of one data-parallel rank. */
typedef struct zero_comm {
  uint32_t reduce_scatters;    /* gradient reduce-scatters per step */
  uint32_t all_gathers;        /* parameter all-gathers per step */
  double elems;                /* the guide's count: Psi per collective */
  double elems_sent_per_rank;  /* bandwidth-optimal collectives: (Nd - 1) / Nd of Psi each */
  double bytes_sent_per_rank;  /* fp16: 2 bytes per element */
} zero_comm_t;

/*
 * Communication volume per step (guide, "Como funciona": plain DP moves 2 Psi,
 * a reduce-scatter and an all-gather of Psi each; P_os+g keeps 2 Psi; P_os+g+p
 * needs two parameter all-gathers, in forward and backward, plus the gradient
 * reduce-scatter, 3 Psi or 1.5x; lastdictionary entry "ZeRO": stages 1 and 2
 * keep data parallelism's volume).  Fills *out: stages 0-2 one reduce-scatter
 * and one all-gather, stage 3 one reduce-scatter and two all-gathers.  Pure
 * host arithmetic.  Errors: ZERO_E_INVAL for out == NULL, nd == 0 or a stage
 * not 0..3.
 */
int zero_comm_volume(uint64_t psi, uint32_t nd, int stage, zero_comm_t *out);

/*
 * Partition of `rank` (card "ZeRO-2", "Why all-gather is still needed": the
 * all-gather of the rank shards in rank order rebuilds [A, B, C]): shard size
 * S = ceil(psi / nd); rank r owns [min(r S, psi), min((r + 1) S, psi)), so
 * trailing shards may be short or empty.  Fills *out.  Errors: ZERO_E_INVAL
 * for out == NULL, nd == 0, rank >= nd or psi == 0.
 */
int zero_shard_geometry(uint64_t psi, uint32_t nd, uint32_t rank, zero_geom_t *out);

/*
 * Flat range [*lo, *hi) of bucket [bucket_offset, bucket_offset + bucket_len)
 * that the rank owns; *lo == *hi when they do not meet (card "ZeRO-2", the
 * bucket diagram and "Gradient lifecycle": of each bucket reduce-scattered in
 * backward, a rank keeps the part that falls in its own partition).  Errors: ZERO_E_INVAL
 * (null pointer, geometry that zero_shard_geometry would not return),
 * ZERO_E_RANGE (bucket beyond psi).
 */
int zero_bucket_intersect(const zero_geom_t *g, uint64_t bucket_offset, uint64_t bucket_len,
                          uint64_t *lo, uint64_t *hi);

/*
 * Advised row stride, in elements, for the Nd fp16 gradient rows of a bucket
 * (or chunk) of `len` columns that a caller lays out for zero_reduce_shard:
 * len rounded up to a multiple of 64 elements (each row starts on a 128-byte
 * line), plus 1024 elements when that stride is a whole number of MiB.  The
 * reduce reads the Nd rows of a column tile at once, and on MI355X rows a power
 * of two apart read slower: at Nd = 400, rows 4 or 8 MiB apart stream 12-14%
 * slower than the same rows 2 KiB further apart, while on the other strides
 * measured the pad changes nothing beyond run-to-run noise.  Advice only:
 * zero_reduce_shard accepts any slice_stride >= bucket_len.  len == 0 gives 0.
 * Errors: ZERO_E_INVAL (stride NULL), ZERO_E_RANGE (the stride would not fit in
 * 64 bits).
 */
int zero_row_stride(uint64_t len, uint64_t *stride);

/*
 * The owner's reduce of one gradient bucket (guide, "Como funciona": each
 * gradient is reduced only at the process that owns its partition, via
 * reduce-scatter, then released; card "ZeRO-2", "Gradient lifecycle").
 *
 * slices: device, fp16 bit patterns, Nd rows; row k (at slices + k *
 *   slice_stride) is data-parallel rank k's local gradient over the flat range
 *   [bucket_offset, bucket_offset + bucket_len) -- a whole bucket, or any chunk
 *   of one.  Only the columns inside the rank's shard are read.  The buffer must
 *   hold (Nd - 1) * slice_stride + bucket_len elements; slice_stride >=
 *   bucket_len.
 * grad32: device, fp32, the rank's shard-local gradient (g->len elements), or
 *   NULL to keep only the fp16 gradient shard; for every flat i in
 *   bucket-intersect-shard,
 *     grad32[i - g->offset] = RN32(sum_{k = 0..Nd-1} fp32(row_k[i])) * RN32(1/Nd)
 *   with the additions done one at a time in ascending rank order from +0 (each
 *   rounded to fp32) and one fp32 multiply by the correctly rounded 1/Nd.
 *   Elements outside the intersection are not touched.
 * grad16: optional (NULL = none), device, fp16 bit patterns, g->len elements:
 *   the round-to-nearest-even fp16 of the fp32 value above, at the same
 *   elements.  This 2-byte gradient shard is the one the guide's stage-2
 *   accounting keeps (2 Psi + 14 Psi / Nd).  At least one of grad32 and grad16
 *   must be given.
 * Aliasing: an output may share memory with the rows only column for column,
 *   i.e. the output element of flat index i at the address of some row's
 *   element i.  This is how stage 1 (P_os) keeps its reduced shard inside its
 *   own retained full local gradient: grad16 = own_local_grad + g->offset where
 *   row `rank` is own_local_grad + bucket_offset.  Any other overlap is
 *   undefined.
 * The "release" of the rest of the local gradient is the caller freeing
 * `slices` after this call completes on the stream.  An empty intersection is
 * ZERO_OK and enqueues nothing.
 * Nd is at most 2^24 here (the largest Nd for which RN32(1/Nd) is the fp32
 * quotient 1 / fp32(Nd)).
 * Errors: ZERO_E_INVAL (slices NULL, both outputs NULL, bad geometry),
 * ZERO_E_RANGE (bucket beyond psi, slice_stride < bucket_len, size overflow,
 * Nd > 2^24 for a bucket that meets the shard),
 * ZERO_E_ALIGN (slices or grad16 not 2-byte, grad32 not 4-byte aligned),
 * ZERO_E_DEVICE (launch failed, or the launch's residency cap cannot be set on
 * this device).
 */
int zero_reduce_shard(const zero_geom_t *g, uint64_t bucket_offset, uint64_t bucket_len,
                      const uint16_t *slices, uint64_t slice_stride, float *grad32,
                      uint16_t *grad16, void *hip_stream);

/* The rank's optimizer-state shard and its fp16 parameter slot. */
typedef struct zero_shard {
  float *master;           /* device, fp32 master weights, g->len elements, updated in place */
  float *m;                /* device, fp32 first moment, g->len elements, updated in place */
  float *v;                /* device, fp32 second moment, g->len elements, updated in place */
  const void *grad;        /* device, the reduced gradient shard, g->len elements */
  int grad_is_fp16;        /* 0: grad is fp32; 1: grad is fp16 bit patterns */
  uint16_t *param16;       /* device, fp16 window of the flat parameter vector, or NULL (no slot write) */
  uint64_t param16_origin; /* flat index of param16[0] */
  uint64_t param16_len;    /* elements in the window */
} zero_shard_t;

/*
 * Per-step fp32 scalars of the Adam step (Kingma & Ba, Algorithm 1: the
 * bias corrections 1 - beta1^t and 1 - beta2^t of step t; the guide, "Como
 * funciona", names mixed-precision Adam as the optimizer), derived in fp64 and
 * rounded once:
 *   out[0] = b1 = RN32(beta1)          out[1] = b2 = RN32(beta2)
 *   out[2] = c1 = RN32(1 - beta1)      out[3] = c2 = RN32(1 - beta2)
 *   out[4] = e  = RN32(eps)
 *   out[5] = step = RN32(lr / (1 - beta1^t))
 *   out[6] = isb  = RN32(1 / sqrt(1 - beta2^t))
 * (1 - beta and the bias corrections are evaluated in fp64, beta^t with pow).
 * Errors: ZERO_E_INVAL for out == NULL, t == 0, beta outside [0, 1), eps <= 0,
 * or a non-finite lr.
 */
int zero_adam_scalars(double lr, double beta1, double beta2, double eps, uint64_t step,
                      float out[7]);

/*
 * One fused Adam step on the rank's shard (guide, "Como funciona": each process
 * updates only its own partition; lastdictionary entry "ZeRO", usage note: the
 * update itself is plain Adam).  Adam as published by Kingma & Ba (Algorithm 1,
 * bias-corrected, eps outside the square root, step t >= 1, no weight decay),
 * per element j < g->len, in fp32 with every operation rounded once and no
 * fused multiply-add, using the scalars of zero_adam_scalars:
 *   m'  = b1*m + c1*g
 *   v'  = b2*v + c2*(g*g)
 *   den = sqrt(v')*isb + e              (correctly rounded sqrt)
 *   th' = th - step*(m'/den)            (correctly rounded division)
 *   param16[g->offset - param16_origin + j] = fp16_rne(th')
 * Each element of g, master, m, v is read once and master, m, v and the fp16
 * slot are written once (28 bytes per element with an fp16 gradient, 30 with
 * fp32).  Only the slot [g->offset, g->offset + g->len) of the fp16 window is
 * written (card "ZeRO-2", "Why all-gather is still needed": that slot is the
 * rank's contribution to the all-gather of [A, B, C]).
 * Errors: ZERO_E_INVAL (null pointer, bad geometry or hyperparameter),
 * ZERO_E_RANGE (slot outside the fp16 window), ZERO_E_ALIGN (fp32 arrays not
 * 4-byte, fp16 arrays not 2-byte aligned), ZERO_E_DEVICE (launch failed, or the
 * launch's residency cap cannot be set on this device).
 */
int zero_adam_step_shard(const zero_geom_t *g, const zero_shard_t *s, double lr, double beta1,
                         double beta2, double eps, uint64_t step, void *hip_stream);

/*
 * The receive side of one layer's parameter all-gather in stage 3, P_os+g+p
 * (guide, "Como funciona": the parameters are partitioned too and a process
 * that needs another's partition receives it, two parameter all-gathers per
 * step; lastdictionary entry "ZeRO": each layer's parameters are gathered just
 * in time and discarded after use; card "ZeRO-2", "Why all-gather is still
 * needed": the partitions in rank order are the full vector).
 *
 * shards: device, fp16 bit patterns, Nd rows; row k (at shards + k *
 *   shard_stride) is rank k's parameter shard, flat [k S, min((k + 1) S, psi))
 *   with S = ceil(psi / nd) as in zero_shard_geometry; shard_stride >= S.
 * out: device, fp16, len elements: out[j] = the parameter of flat index lo + j.
 *   It must not overlap the shards.
 * Pure data movement (bit-exact).  len == 0 is ZERO_OK and enqueues nothing.
 * Errors: ZERO_E_INVAL (nd == 0, psi == 0, NULL buffer), ZERO_E_RANGE (range
 * beyond psi, shard_stride < S, size overflow), ZERO_E_ALIGN (a buffer not
 * 2-byte aligned), ZERO_E_DEVICE (launch failed).
 */
int zero_gather_params(uint64_t psi, uint32_t nd, uint64_t lo, uint64_t len,
                       const uint16_t *shards, uint64_t shard_stride, uint16_t *out,
                       void *hip_stream);

/* The streaming kernels whose residency the library caps (zero_launch_occupancy). */
#define ZERO_KERNEL_REDUCE_W16 0 /* the reduce with 16-byte row loads (aligned rows) */
#define ZERO_KERNEL_REDUCE_W8 1  /* ... 8-byte row loads */
#define ZERO_KERNEL_REDUCE_W4 2  /* ... 4-byte row loads */
#define ZERO_KERNEL_REDUCE_W2 3  /* ... 2-byte row loads */
#define ZERO_KERNEL_ADAM_G32 4   /* the fused Adam step, fp32 gradient */
#define ZERO_KERNEL_ADAM_G16 5   /* the fused Adam step, fp16 gradient */

/*
 * Launch residency of one capped kernel on the calling thread's current device.
 * No passage defines it: it is a measured property of MI355X.  The reduce and
 * the Adam step stream HBM faster when fewer workgroups share a compute unit
 * (at most 8 for the reduce, 10 for Adam), so every launch asks for dynamic
 * LDS that the kernels never touch.  On the first call that launches on a
 * device, the library resolves, per kernel, the LDS size at which the
 * runtime's occupancy calculator allows exactly that many workgroups per CU,
 * and it refuses to launch (ZERO_E_DEVICE) when no size does.
 * Fills *wgs_per_cu with the workgroups per CU the calculator allows at the
 * resolved size, and *lds_bytes (nullable) with that size.
 * Errors: ZERO_E_INVAL (unknown kernel, wgs_per_cu NULL), ZERO_E_DEVICE (no
 * device, or the cap cannot be reached on it).
 */
int zero_launch_occupancy(int kernel, int *wgs_per_cu, uint32_t *lds_bytes);

/* Message of the calling thread's last error ("" if none).  Valid until the
 * thread's next call into the library. */
const char *zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_H_ */
