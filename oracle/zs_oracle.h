/*
 * zs_oracle.h -- plain CPU oracle of the per-rank ZeRO-2 optimizer-shard step.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library. The GPU library
 * (libzeroshard) never calls it, and the two share no source: no headers, no
 * helpers, no tables.
 *
 * Sources, cited by page title and section:
 *   [Notes] untitled lecture notes on DP, DDP and DeepSpeed ZeRO
 *           (gitcode.csdn.net/69c4e349...): sections "一、DP", "二、DDP",
 *           "三、DeepSpeed ZeRO - 1", "四、DeepSpeed ZeRO - 2 & ZeRO - 3".
 *   [Intro] "并行训练框架DeepSpeed介绍" (an introduction to DeepSpeed,
 *           nanhubrain.csdn.net): part 一.3 "DeepSpeed核心技术", items (1)-(16).
 *   [L7]    "第 7 讲：Parallelism（上）" (CS336 lecture 7, cs336.sjfarm.cc):
 *           sections "数学等价性", "Ring AllReduce 算法", "Gradient Accumulation",
 *           "ZeRO Stage 1/2/3", "ZeRO 各阶段对比".
 *
 * Precision. The pages fix the formats: 16-bit (fp16/bf16) gradients and
 * parameters, fp32 master weights and fp32 Adam moments ([L7] memory table;
 * [Notes] 三, the owner converts gradients to FP32 before its update). Every
 * per-element operation here is therefore one IEEE-754 binary32 operation
 * with round-to-nearest-even, no contraction, denormals preserved, in the
 * order written. Per-step scalars (bias corrections, decay factor) are formed
 * in binary64 and rounded once to binary32.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - AdamW is named but never written out: standard Adam moments with
 *     bias correction and decoupled weight decay applied to the weight
 *     first, eps added after the bias-corrected square root.
 *   - Ring labelling: ZeRO's rank r owns partition r, so its chunk is summed
 *     starting at worker r+1 with r's own term added last (sigma = 0). The
 *     [Notes] 二 worked example uses sigma = 1 (GPU0 ends up holding B).
 *   - Average (divide by W) comes before the unscale (divide by the loss
 *     scale S); the overflow flag is "some unscaled fp32 gradient is not
 *     finite". On overflow the step is skipped and nothing changes.
 *   - Partition size P = ceil(phi / W); rank r owns [r*P, r*P + count_r).
 */
#ifndef ZS_ORACLE_H
#define ZS_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ZSO_BF16 = 0, ZSO_FP16 = 1 };

/* Precision of the partial sums the ring passes between ranks ("on the
 * wire"): fp32 (the default), or rounded to bf16 / fp16 at every hop, as
 * when the reduction runs in a 16-bit dtype ([L7] "ZeRO 与 FSDP": the FSDP
 * example's MixedPrecision reduce_dtype=bfloat16). */
enum { ZSO_WIRE_FP32 = 0, ZSO_WIRE_BF16 = 1, ZSO_WIRE_FP16 = 2 };

/* Returns 1 when the floating-point environment keeps subnormals and rounds
 * to nearest-even (the oracle's results assume both), else 0. */
int zso_fp_env_ok(void);

/* Partition map. [Notes] 二 (each chunk is phi/N of the flat buffer) and
 * [L7] "Ring AllReduce 算法" (the vector is cut into W chunks). P is phi/W
 * rounded up; rank r owns [r*P, r*P + count). Returns 0, or -1 for world == 0
 * or rank >= world. */
int zso_partition(uint64_t phi, uint32_t world, uint32_t rank,
                  uint64_t *chunk, uint64_t *offset, uint64_t *count);

/* Exact widening of a 16-bit float (bit pattern) to fp32. */
float zso_half_to_float(uint16_t bits, int dtype);
/* fp32 -> 16-bit float, round to nearest, ties to even; overflow -> inf;
 * NaN -> a quiet NaN of the same sign. */
uint16_t zso_float_to_half(float x, int dtype);
void zso_halves_to_floats(const uint16_t *in, float *out, uint64_t n, int dtype);
void zso_floats_to_halves(const float *in, uint16_t *out, uint64_t n, int dtype);

/* Full ring simulation over W ranks ([Notes] 二 three-GPU example; [L7]
 * "Ring AllReduce 算法"). bufs holds W rows, row k being rank k's flat buffer
 * of W*L fp32 values (chunk c = elements [c*L, (c+1)*L)). Runs `steps`
 * (<= W-1) scatter-reduce steps: at step s rank k sends its chunk
 * (k - s + sigma) mod W to rank k+1, which replaces its own copy by
 * (received + own). After W-1 steps rank k holds the full sum of chunk
 * (k + sigma) mod W. Returns 0, or -1 on bad arguments / allocation failure. */
int zso_ring_reduce_scatter(uint32_t world, uint64_t chunk_len, int sigma,
                            uint32_t steps, float *bufs);
/* All-gather phase of the same ring: at step s rank k forwards chunk
 * (k + sigma - s + 1) mod W to rank k+1, which overwrites its copy. */
int zso_ring_all_gather(uint32_t world, uint64_t chunk_len, int sigma,
                        uint32_t steps, float *bufs);
/* Chunk that rank `rank` holds after a complete scatter-reduce. */
uint32_t zso_ring_held_chunk(uint32_t world, uint32_t rank, int sigma);

/* The journey of rank r's own chunk around the ring (sigma = 0), element by
 * element: acc = G[r+1]; acc = acc + G[r+2]; ... ; acc = acc + G[r]
 * (indices mod W). part[k] points at element `offset` of worker k's flat
 * 16-bit gradient buffer (worker order, not ring order). */
void zso_ring_chunk_sum(uint32_t world, uint32_t rank,
                        const uint16_t *const *part, int dtype, uint64_t n,
                        float *sum_out);

/* The same journey with a 16-bit wire: every partial the ring sends is
 * rounded (nearest-even) to the wire type, i.e. acc = R(G[r+1]), then
 * acc = R(acc + G[r+s]) for s = 2..W, the last (the owner's) included.
 * wire = ZSO_WIRE_FP32 gives zso_ring_chunk_sum exactly. */
void zso_ring_chunk_sum_wire(uint32_t world, uint32_t rank,
                             const uint16_t *const *part, int dtype, int wire,
                             uint64_t n, float *sum_out);

/* Owner's reduction of one gradient bucket: a = sum / W (ring order), then
 * out = a (accumulate == 0) or out = out + a (accumulate != 0: later
 * micro-batches, [L7] "Gradient Accumulation"). Returns the overflow flag of
 * out / loss_scale (1 if any element is not finite). */
uint32_t zso_reduce_avg(uint32_t world, uint32_t rank,
                        const uint16_t *const *part, int dtype, uint64_t n,
                        float *out, int accumulate, float loss_scale);
/* zso_reduce_avg with the partial sums carried in `wire` precision. */
uint32_t zso_reduce_avg_wire(uint32_t world, uint32_t rank,
                             const uint16_t *const *part, int dtype, int wire,
                             uint64_t n, float *out, int accumulate,
                             float loss_scale);

/* 1 if any (a[i] / loss_scale) is not finite, else 0. */
uint32_t zso_check_overflow(const float *a, uint64_t n, float loss_scale);

/* Per-step AdamW scalars, formed in binary64 from the fp32 hyper-parameters
 * and rounded once to fp32. */
typedef struct {
  float alpha;  /* lr / (1 - beta1^t)          */
  float b2;     /* sqrt(1 - beta2^t)           */
  float delta;  /* 1 - lr * weight_decay       */
  float c1;     /* 1 - beta1                   */
  float c2;     /* 1 - beta2                   */
  float beta1, beta2, eps;
} zso_adamw_consts;
void zso_adamw_consts_make(float lr, float beta1, float beta2, float eps,
                           float weight_decay, uint32_t t,
                           zso_adamw_consts *out);

/* In-place AdamW over one partition, g = a / loss_scale. */
void zso_adamw(float *master, float *m, float *v, const float *a, uint64_t n,
               float loss_scale, const zso_adamw_consts *k);

typedef struct {
  uint32_t world, rank;
  uint64_t n;
  int grad_dtype, param_dtype;
  const uint16_t *const *part;  /* [world], worker order, at this rank's offset */
  const float *acc_in;          /* NULL, or fp32 gradient accumulated so far   */
  const float *master_in, *m_in, *v_in;
  float *master_out, *m_out, *v_out;
  uint16_t *param_out;          /* this rank's slice of the gather buffer      */
  float lr, beta1, beta2, eps, weight_decay, loss_scale;
  uint32_t step_t;
  int wire;                     /* ZSO_WIRE_*: precision of the ring partials */
} zso_step_args;

/* One whole shard step (ring sum, average, optional accumulate, unscale,
 * overflow check, AdamW, cast), split over `threads` disjoint index ranges.
 * Writes the out-set and param_out for every element and returns the flag;
 * when the flag is 1 the caller discards them (the step is skipped). */
uint32_t zso_shard_step(const zso_step_args *a, int threads);

/* Dynamic loss scaler ([Intro] 一.3 items (1) and (3) name dynamic loss
 * scaling without a rule). Reading: on overflow halve the scale, reset the
 * clean-step count and keep t; otherwise t += 1 and clean += 1, and once
 * clean reaches `interval` the scale doubles (from the next step on) and
 * clean restarts at 0. */
typedef struct {
  float scale;
  uint32_t clean;
  uint32_t interval;
  uint64_t t;        /* committed steps */
  uint64_t skipped;
} zso_scaler;
void zso_scaler_update(zso_scaler *s, uint32_t overflow);

/* Model-state bytes per GPU with (2 + 2 + K) bytes per parameter ([Notes] 三
 * and 四; [L7] "ZeRO Stage 1/2/3"): stage 0 (DDP) (4+K)psi; stage 1
 * 4psi + K psi/N; stage 2 2psi + (2+K)psi/N; stage 3 (4+K)psi/N. */
double zso_model_state_bytes(double psi, double n_gpus, int stage, double k);

/* Ring all-reduce time estimate ([L7] "通信时间估算"):
 * 2(W-1)*alpha + 2*M*(W-1)/(W*beta). */
double zso_ring_allreduce_time(double msg_bytes, double world, double alpha,
                               double beta);

#ifdef __cplusplus
}
#endif
#endif /* ZS_ORACLE_H */
