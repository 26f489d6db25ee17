/*
 * fsdp_shard.h -- C ABI of libfsdpshard.so: one rank's share of the sharded
 * FlatParameter lifecycle of Fully Sharded Data Parallel, on one MI355X
 * (gfx950) GPU.
 *
 * Pages cited (page title, then section):
 *   [FSDP-math]  the aicassindra "transformer math" page on FSDP (tm_fsdp_math)
 *   [NOTE-003]   "NOTE-003: PyTorch FSDP"
 *   [Glossary]   glossary entry "fully sharded data parallel fsdp"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - A unit is T tensors, each row-major, laid end to end in the order given:
 *   tensor i occupies flat elements [off_i, off_i + n_i), off_i = sum_{j<i} n_j,
 *   U = sum_i n_i. F is the sharding factor and r this rank.
 *   S = ceil(U / F) is the shard length; the flat buffer is padded with +0.0 to
 *   F*S; rank k owns flat elements [k*S, (k+1)*S). shard_valid = the number of
 *   real (non-pad) elements in rank r's window = clamp(U - r*S, 0, S).
 * - bf16 buffers are passed as raw 16-bit patterns; fp32 as IEEE binary32.
 * - Device pointers are plain device addresses (e.g. torch data_ptr()). Any
 *   element-aligned address is accepted. The step calls take their vector
 *   path when the fp32 buffers are 16-byte aligned (8-byte for a bf16 output)
 *   and every gradient row's rank window starts on an 8-byte boundary; rows
 *   that are only 2-byte aligned take a shifted-row path (flat folds) or the
 *   scalar path (grouped folds), and state off 16-byte alignment takes the
 *   scalar path. Windows that start off a 128-byte line are read and written
 *   with their tiles in runs per XCD, which keeps the cost of the lines they
 *   share with neighbouring tiles near 3% of the row bytes. Arrays of pointers
 *   (grads, shards, tensors) are HOST arrays of device pointers, copied into
 *   kernel arguments by the call.
 * - Ownership: the caller owns every device buffer. The library owns only the
 *   opaque fsdp_unit (host memory) and allocates no device memory.
 * - Execution: every device entry point only enqueues work on `stream`
 *   (NULL = the null stream) and returns; there is no implicit
 *   synchronisation, allocation or host<->device copy. Arguments are checked
 *   and every launch is planned before anything is enqueued, so a call that
 *   fails a check has enqueued nothing. Before its first launch a call also
 *   checks the calling thread's HIP error state (hipPeekAtLastError): if an
 *   error from earlier work is pending it returns FSDP_ERR_HIP, enqueues
 *   nothing and leaves that error in place. FSDP_ERR_HIP after that means
 *   the runtime refused a launch: a call of one launch has then enqueued
 *   nothing; a call that needs several (fsdp_reduce_adamw_units, and
 *   fsdp_flatten_pad / fsdp_unflatten beyond 64 copy segments) keeps the
 *   launches before the refused one enqueued. A fault inside a kernel
 *   surfaces at the caller's next synchronisation, not as a return code.
 * - Empty windows: when a step call's shard_valid is 0 (a rank whose window
 *   holds only pad), it checks its counts and hyper-parameters and returns
 *   FSDP_OK without touching its buffer arguments, which may then be NULL;
 *   the same holds for fsdp_flatten_pad with len 0, and fsdp_unflatten reads
 *   no shard that holds only pad and writes no tensor of 0 elements.
 * - Aliasing: the byte ranges a call writes must not overlap each other or
 *   the ranges it reads (FSDP_ERR_ALIAS); master/exp_avg/exp_avg_sq are read
 *   and written in place by design.
 * - Positions at or beyond shard_valid (the pad) are never read or written by
 *   reduce/adamw entry points; only fsdp_flatten_pad writes pad (as zeros).
 * - fsdp_last_error() returns a thread-local message for the last failure.
 */
#ifndef FSDP_SHARD_H
#define FSDP_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define FSDP_ABI_VERSION 1
#define FSDP_MAX_RANKS 64        /* limit on F and on n_grads */
#define FSDP_MAX_TENSORS 65536   /* limit on T */

typedef enum {
  FSDP_OK = 0,
  FSDP_ERR_INVALID_ARG = 1,   /* null pointer, bad count, bad hyper-parameter */
  FSDP_ERR_RANGE = 2,         /* window or size outside what the unit allows */
  FSDP_ERR_ALIAS = 3,         /* overlapping input/output byte ranges */
  FSDP_ERR_UNSUPPORTED = 4,   /* dtype or element size not handled */
  FSDP_ERR_HIP = 5            /* the HIP runtime refused a launch */
} fsdp_status;

typedef enum { FSDP_F32 = 0, FSDP_BF16 = 1 } fsdp_dtype;

typedef struct fsdp_unit fsdp_unit;   /* opaque; immutable after create */

typedef struct {
  int64_t U;                /* params in the unit */
  int64_t S;                /* shard length ceil(U/F) */
  int64_t padded;           /* F*S */
  int64_t pad;              /* padded - U */
  int64_t shard_begin;      /* r*S */
  int64_t shard_valid;      /* clamp(U - r*S, 0, S) */
  int64_t persistent_bytes; /* 16*S: bf16 w + bf16 g + fp32 master, m, v */
  int32_t F;
  int32_t rank;
  int32_t n_tensors;
  int32_t reserved;
  uint64_t fingerprint;     /* FNV-1a of F, T and every dim, for cross-rank checks */
} fsdp_unit_info;

/* AdamW hyper-parameters of one step. Every scalar is given in double and is
 * rounded once to fp32 on the host: beta1, 1-beta1, beta2, 1-beta2,
 * 1-beta1^step, 1-beta2^step, lr, eps, weight_decay and grad_scale. */
typedef struct {
  double lr;            /* finite, >= 0 */
  double beta1;         /* in [0, 1) */
  double beta2;         /* in [0, 1) */
  double eps;           /* finite, > 0 */
  double weight_decay;  /* finite */
  double grad_scale;    /* finite; multiplies the fp32 sum (1/n_grads = mean) */
  int64_t step;         /* 1-based step count t of this update */
} fsdp_adamw_hparams;

int32_t fsdp_abi_version(void);

/* Unit indexer.
 * [FSDP-math, "The sharding unit: FlatParameter and the wrapping policy"]: a
 * wrapped module's parameters form one flat 1-D buffer, split evenly over the
 * ranks; each rank keeps one contiguous slice. [NOTE-003, "Key results"]: F
 * is the number of ranks parameters are sharded over (F = 1 is plain data
 * parallelism). [FSDP-math, "Per-unit memory and communication, in numbers"]:
 * persistent state is 16 bytes per parameter on 1/N of the parameters.
 * Host only. n_tensors tensors; tensor i has ndim[i] dims (0 = scalar, one
 * element) taken in order from `dims`. Requires 1 <= F <= 64, 0 <= rank < F,
 * 1 <= n_tensors <= 65536, dims >= 0, 1 <= U and 4*F*S < 2^62.
 * *out receives a new handle (free with fsdp_unit_destroy). Thread-safe: a
 * handle can be used from several threads at once. */
fsdp_status fsdp_unit_create(int32_t F, int32_t rank, int32_t n_tensors,
                             const int32_t* ndim, const int64_t* dims,
                             fsdp_unit** out);
fsdp_status fsdp_unit_destroy(fsdp_unit* unit);
fsdp_status fsdp_unit_query(const fsdp_unit* unit, fsdp_unit_info* info);
/* Flat offset and element count of tensor i. */
fsdp_status fsdp_unit_tensor(const fsdp_unit* unit, int32_t i, int64_t* offset,
                             int64_t* numel);

/* Flatten + pad (init time).
 * [FSDP-math, "The sharding unit: FlatParameter and the wrapping policy"]
 * and [NOTE-003, "Method" -> Key components: FlatParameter].
 * dst[q] = flat[begin + q] for 0 <= q < len, where flat is the unit's tensors
 * end to end followed by +0 (all-zero bits) up to F*S. A bit copy: dtype only
 * fixes the element size (FSDP_F32 = 4 bytes, FSDP_BF16 = 2 bytes).
 * `tensors`: host array of T device pointers, tensor i holding n_i elements.
 * `dst`: len elements. Requires 0 <= begin, len >= 0, begin + len <= F*S.
 * Rank r's shard is begin = r*S, len = S. */
fsdp_status fsdp_flatten_pad(const fsdp_unit* unit, fsdp_dtype dtype,
                             const void* const* tensors, int64_t begin, int64_t len,
                             void* dst, hipStream_t stream);

/* Reduce-scatter arithmetic, fp32 reduce of bf16 gradients.
 * [FSDP-math, "The backward cycle: all-gather, grads, reduce-scatter"]: the
 * ranks' full gradients are summed (the data-parallel average) and each rank
 * keeps the reduced slice matching its own parameter slice.
 * [Glossary, "FSDP Implementation (PyTorch)" -> Mixed Precision]: reductions
 * run in fp32.
 * `grads`: host array of n_grads (1..64) device pointers, each rank's full bf16
 * gradient of the unit (U elements, unpadded). For i < shard_valid:
 *   acc = widen(grads[0][r*S+i]); acc = acc + widen(grads[k][r*S+i]) for
 *   k = 1..n_grads-1 in order (binary32, round to nearest even);
 *   out[i] = acc * fp32(grad_scale).
 * `out`: fp32, at least shard_valid elements; nothing else is written. */
fsdp_status fsdp_reduce_shard(const fsdp_unit* unit, int32_t n_grads,
                              const void* const* grads, double grad_scale,
                              float* out, hipStream_t stream);

/* Sharded AdamW on the local slice, in place.
 * [FSDP-math, "The backward cycle: all-gather, grads, reduce-scatter"]: the
 * optimizer updates the rank's own slice in place; [Glossary, "FSDP Sharding
 * Strategy" -> Optimizer State Sharding]: the moments exist only for that
 * slice and the step needs no communication. Update rule (Adam with bias
 * correction, Kingma & Ba 2015; decoupled decay scaled by lr, Loshchilov &
 * Hutter 2019), one binary32 operation per step, no fused multiply-add:
 *   m' = b1*m + (1-b1)*g;  v' = b2*v + (1-b2)*(g*g)
 *   u  = (m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps)
 *   p' = p - lr*(u + wd*p);  w = bf16 round-to-nearest-even of p' (optional)
 * `grad`, `master`, `exp_avg`, `exp_avg_sq`: fp32, shard_valid elements used.
 * `param_bf16_out`: NULL, or shard_valid bf16 outputs (the parameter the next
 * all-gather ships, [NOTE-003, "Key components"]: mixed precision).
 * grad_scale in `hp` is ignored here. */
fsdp_status fsdp_adamw_shard(const fsdp_unit* unit, const float* grad, float* master,
                             float* exp_avg, float* exp_avg_sq, void* param_bf16_out,
                             const fsdp_adamw_hparams* hp, hipStream_t stream);

/* Fused reduce + AdamW: fsdp_reduce_shard with hp->grad_scale followed by
 * fsdp_adamw_shard on its fp32 result, in one pass over HBM (the reduced
 * gradient stays in registers). Bitwise equal to the two calls in sequence.
 * Same buffers and rules as those two entry points. */
fsdp_status fsdp_reduce_adamw_shard(const fsdp_unit* unit, int32_t n_grads,
                                    const void* const* grads, float* master,
                                    float* exp_avg, float* exp_avg_sq,
                                    void* param_bf16_out,
                                    const fsdp_adamw_hparams* hp, hipStream_t stream);

/* Reduce dtype bf16: the reduce-scatter arithmetic with bf16 partial sums.
 * [NOTE-003, "Recommendations"] (R3): mixed precision for communication volume;
 * [Glossary, "FSDP Implementation (PyTorch)" -> Mixed Precision]: the reduce
 * dtype is a choice. For i < shard_valid: p = grads[0][r*S+i]; for k = 1..n-1:
 * p = bf16_rne(widen(p) + widen(grads[k][r*S+i])) (an fp32 add, then rounding
 * to nearest even bf16); out[i] = widen(p) * fp32(grad_scale). Same buffers and
 * rules as fsdp_reduce_shard / fsdp_reduce_adamw_shard; only the numerics of
 * the sum differ (coarser, bounded by the summation bound in bf16). */
fsdp_status fsdp_reduce_shard_bf16acc(const fsdp_unit* unit, int32_t n_grads,
                                      const void* const* grads, double grad_scale, float* out,
                                      hipStream_t stream);
fsdp_status fsdp_reduce_adamw_shard_bf16acc(const fsdp_unit* unit, int32_t n_grads,
                                            const void* const* grads, float* master,
                                            float* exp_avg, float* exp_avg_sq,
                                            void* param_bf16_out,
                                            const fsdp_adamw_hparams* hp, hipStream_t stream);

/* Hybrid sharding (HSDP): the unit is sharded F ways inside each of `replicas`
 * (R) groups and replicated across groups. [NOTE-003, "Concepts"]: shard within
 * a group, replicate across groups; [Glossary, "Hybrid Sharding"]: gradients
 * are all-reduced across the groups and sharded within a group.
 * `grads`: host array of R*F device pointers, replica-major: row rho*F + f is
 * rank f of group rho, each the full bf16 unit gradient (U elements). For
 * i < shard_valid: each group left-folds its F rows in rank order in fp32
 * (the reduce-scatter inside the group), the R group sums are left-folded in
 * group order (the all-reduce across groups) and the result is multiplied by
 * fp32(grad_scale) (1/(R*F) gives the mean). R = 1 is fsdp_reduce_shard.
 * Requires 1 <= R*F <= 64. Same buffers and rules as the flat entry points. */
fsdp_status fsdp_reduce_shard_hybrid(const fsdp_unit* unit, int32_t replicas,
                                     const void* const* grads, double grad_scale, float* out,
                                     hipStream_t stream);
/* The hybrid reduction followed by AdamW in one pass, as fsdp_reduce_adamw_shard. */
fsdp_status fsdp_reduce_adamw_shard_hybrid(const fsdp_unit* unit, int32_t replicas,
                                           const void* const* grads, float* master,
                                           float* exp_avg, float* exp_avg_sq,
                                           void* param_bf16_out,
                                           const fsdp_adamw_hparams* hp, hipStream_t stream);

/* One unit's share of a multi-unit optimizer step (see fsdp_reduce_adamw_units). */
typedef struct {
  const fsdp_unit* unit;
  const void* const* grads;   /* host array of n_grads device pointers, U elements each */
  float* master;              /* shard_valid fp32 each, updated in place */
  float* exp_avg;
  float* exp_avg_sq;
  void* param_bf16_out;       /* NULL or shard_valid bf16 outputs */
} fsdp_unit_step;

/* The rank's optimizer step over many units at once: for every entry, exactly
 * what fsdp_reduce_adamw_shard computes for it (bitwise), with one set of
 * hyper-parameters (one step t, one grad_scale) and one n_grads for all.
 * [FSDP-math, "The backward cycle: all-gather, grads, reduce-scatter"]: after
 * the last reduce-scatter the optimizer updates every local slice in place;
 * [FSDP-math, "The sharding unit: FlatParameter and the wrapping policy"]: few
 * large operations rather than many small ones. Aligned entries with
 * n_grads <= 8 and fewer than 2^22 shard elements are stepped together, one
 * kernel launch per up to 30 units; larger or unaligned entries get one
 * launch each, in the order given. All entries are validated (including
 * overlaps between different units' buffers) and every launch is planned
 * before anything is enqueued; entries whose shard_valid is 0 are skipped (their
 * buffers may be NULL). n_units == 0 is a no-op. */
fsdp_status fsdp_reduce_adamw_units(int32_t n_units, const fsdp_unit_step* steps,
                                    int32_t n_grads, const fsdp_adamw_hparams* hp,
                                    hipStream_t stream);

/* All-gather arithmetic + unflatten into per-tensor bf16 parameters.
 * [FSDP-math, "The forward cycle: all-gather, compute, reshard"]: each rank
 * contributes its slice and ends with the unit's full weights, used as
 * ordinary per-tensor parameters; [NOTE-003, "Key components"]: parameters
 * travel in low precision.
 * `shards`: host array of F device pointers, shard k holding S elements of
 * `src_dtype` (rank k's slice). `tensors_bf16`: host array of T device
 * pointers, tensor i receiving n_i bf16 elements (they may be views into one
 * U-long buffer). For flat element g = off_i + j: k = g / S, out_i[j] =
 * shard_k[g - k*S], rounded to bf16 (nearest, ties to even; NaN -> 0x7FC0)
 * from fp32 or copied bit for bit from bf16. Pad slots are never read. */
fsdp_status fsdp_cast_unflatten(const fsdp_unit* unit, fsdp_dtype src_dtype,
                                const void* const* shards, void* const* tensors_bf16,
                                hipStream_t stream);

/* Unflatten with any element type on either side: fsdp_cast_unflatten with a
 * chosen output dtype. FSDP_F32 -> FSDP_F32 and FSDP_BF16 -> FSDP_BF16 copy
 * bits; FSDP_F32 -> FSDP_BF16 rounds to nearest even (NaN -> 0x7FC0);
 * FSDP_BF16 -> FSDP_F32 widens exactly. With fp32 on both sides this is the
 * export half of a full state dict: the F shards of master, exp_avg or
 * exp_avg_sq become whole per-tensor fp32 tensors ([Glossary, "Debugging
 * FSDP" -> Checkpoint/Resume]); fsdp_flatten_pad with FSDP_F32 is the resume
 * half. `tensors`: host array of T device pointers, tensor i receiving n_i
 * elements of dst_dtype. Shards holding only pad are not read (their pointer
 * may be NULL). */
fsdp_status fsdp_unflatten(const fsdp_unit* unit, fsdp_dtype src_dtype, fsdp_dtype dst_dtype,
                           const void* const* shards, void* const* tensors,
                           hipStream_t stream);

const char* fsdp_status_string(fsdp_status status);
const char* fsdp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_SHARD_H */
