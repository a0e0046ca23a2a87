/*
 * zeroshard.h -- C ABI of libzeroshard: the per-rank ZeRO-2 optimizer-shard
 * step on AMD Instinct MI355X (gfx950).
 *
 * One call sequence updates this rank's shard of a model trained with
 * mixed precision under ZeRO stage 2:
 *   (a) owner's side of the gradient reduce-scatter: W workers' 16-bit
 *       gradient buffers are summed in fp32, in the order a ring
 *       scatter-reduce accumulates them, and averaged;
 *   (b) AdamW on the fp32 partition: unscale by the loss scale, overflow
 *       check, moments, bias correction, decoupled weight decay;
 *   (c) cast of the new fp32 master weights to 16 bits, written at this
 *       rank's offset of the flat all-gather buffer.
 *
 * Sources, cited by page title and section:
 *   [Notes] untitled lecture notes on DP, DDP and DeepSpeed ZeRO
 *           (gitcode.csdn.net/69c4e349...): "二、DDP" (ring all-reduce,
 *           bucketing), "三、DeepSpeed ZeRO - 1" (the owner's update
 *           sequence), "四、DeepSpeed ZeRO - 2 & ZeRO - 3".
 *   [Intro] "并行训练框架DeepSpeed介绍" (nanhubrain.csdn.net): part 一.3,
 *           items (1)-(3) mixed precision, BF16 and loss scaling, (12) ZeRO-2.
 *   [L7]    "第 7 讲：Parallelism（上）" (CS336 lecture 7): "数学等价性",
 *           "Ring AllReduce 算法", "Gradient Accumulation", "ZeRO Stage 2".
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device (HBM) addresses the caller allocated;
 *     the library never allocates or frees device memory and never keeps a
 *     pointer after the call returns; its only device memory of its own
 *     is the one-word static array of zs_step_commit_noalloc. Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     completes asynchronously; kernel faults surface at the caller's next
 *     synchronization. These calls wait by contract: zs_step_commit and
 *     zs_step_commit_noalloc (for their flag), zs_offload_step (for its flag
 *     and the gradient pieces), and zs_cpu_step and zs_cpu_update (host
 *     work); no other call synchronizes.
 *   - Host pointers (arrays of device pointers, hyper-parameter structs,
 *     outputs of zs_partition) are read or written during the call only.
 *   - 16-bit values are IEEE binary16 (ZS_FP16) or bfloat16 (ZS_BF16).
 *   - Any element offset is accepted; 16-byte-aligned operands take the
 *     widest vector path (8 elements; 4 in zs_step_fused and its variants,
 *     whose non-temporal stores then cover whole lines), others a narrower
 *     one of the same kernel.
 *   - n == 0 is a no-op that returns ZS_OK; element counts and offsets
 *     above 2^48 return ZS_ERR_UNSUPPORTED before anything is enqueued.
 *   - Status codes: ZS_OK on success; ZS_ERR_INVALID_ARG (null pointer,
 *     world == 0 or > ZS_MAX_WORLD, rank >= world, bad dtype or wire dtype, non-finite or
 *     zero loss scale, step_t == 0) before anything is enqueued;
 *     ZS_ERR_ALIAS when zs_step_fused's output set overlaps its input set;
 *     ZS_ERR_HIP when a launch fails (zs_last_error() has HIP's message).
 *   - Overflow is data, not an error: it is reported only through the
 *     uint32 flag, which calls set to 1 and never clear. The caller zeroes it
 *     before a step; several calls may OR into the same flag.
 *   - Concurrent calls on different streams are safe if their buffers are
 *     disjoint.
 */
#ifndef ZEROSHARD_H
#define ZEROSHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZS_ABI_VERSION 7
#define ZS_MAX_WORLD 64

typedef enum { ZS_BF16 = 0, ZS_FP16 = 1 } zs_dtype;

/* Precision of the partial sums the ring reduction passes between ranks.
 * ZS_WIRE_FP32 (0, the default) carries them in fp32 ([Notes] 三: the owner
 * works in FP32). ZS_WIRE_BF16 / ZS_WIRE_FP16 round every partial, the
 * owner's final sum included, to nearest-even 16 bits, as a reduction run in
 * a 16-bit dtype does ([L7] "ZeRO 与 FSDP": MixedPrecision reduce_dtype):
 *   s = R(G[r+1]);  s = R(s + G[r+s']) for s' = 2..W   (adds in fp32). */
typedef enum { ZS_WIRE_FP32 = 0, ZS_WIRE_BF16 = 1, ZS_WIRE_FP16 = 2 } zs_wire;

/* Layout of the fp32 state (master weights, m, v) that zs_step_fused and
 * the calls built on it read and write ([Notes] 三 keeps the three as the
 * owner's fp32 optimizer state of its partition; their layout in HBM is
 * this library's choice). ZS_STATE_SPLIT (0, the default): three arrays of
 * n floats (master_*, m_*, v_*). ZS_STATE_GROUPED: one buffer per set, in
 * groups of ZS_STATE_GROUP elements; group g holds the master weights of
 * elements [g*1024, (g+1)*1024), then their m, then their v, as three runs of
 * 1024 floats, so element i of the master weights is at float offset
 * 3*1024*(i/1024) + i%1024, its m 1024 floats further and its v 2048
 * floats further. The buffer holds ceil(n/1024) whole groups
 * (12288 bytes each); the slots past n in the last group are never read or
 * written. On MI355X the grouped layout moves the same bytes as one stream
 * in and one out instead of three each, and streamed faster. */
typedef enum { ZS_STATE_SPLIT = 0, ZS_STATE_GROUPED = 1 } zs_state_layout;
#define ZS_STATE_GROUP 1024

typedef enum {
  ZS_OK = 0,
  ZS_ERR_INVALID_ARG = 1,
  ZS_ERR_UNSUPPORTED = 2,
  ZS_ERR_ALIAS = 3,
  ZS_ERR_HIP = 4
} zs_status;

/* AdamW hyper-parameters of one step. lr, betas, eps and weight_decay are
 * the usual AdamW settings; loss_scale is the factor the gradients carry
 * (the update divides it out); step_t is the 1-based index of the step being
 * attempted, i.e. committed steps + 1 (skipped steps do not advance it).
 * Every entry point that takes them returns ZS_ERR_INVALID_ARG, before any
 * launch, unless 0 <= beta1, beta2 < 1 and lr, eps and weight_decay are
 * finite and >= 0 (outside these ranges the update is inf or NaN). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  float loss_scale;
  uint32_t step_t;
} zs_adamw_hparams;

/* ZS_ABI_VERSION of the loaded library. */
int zs_abi_version(void);
/* Static string naming a status code. */
const char *zs_status_string(int status);
/* Detail of this thread's last non-OK status ("" if none). Thread-local. */
const char *zs_last_error(void);

/* Partition map ([Notes] 二: each ring chunk is phi/N elements of the flat
 * buffer; [L7] "Ring AllReduce 算法": the vector is cut into W blocks).
 * chunk = ceil(phi / world); rank `rank` owns the flat elements
 * [offset, offset + count) with offset = rank * chunk and
 * count = min(chunk, max(0, phi - offset)). Host-only. Any output pointer
 * may be NULL. Errors: ZS_ERR_INVALID_ARG for world == 0 or rank >= world. */
int zs_partition(uint64_t phi, uint32_t world, uint32_t rank, uint64_t *chunk,
                 uint64_t *offset, uint64_t *count);

/* Owner's side of the gradient reduce-scatter ([Notes] 二 worked ring
 * example and 四: the owner collects and averages its part; [Intro] (12);
 * [L7] "ZeRO Stage 2": ReduceScatter replaces AllReduce).
 *   worker_grads : host array of `world` device pointers in worker order;
 *                  worker_grads[k] points at element `offset` of worker k's
 *                  flat 16-bit gradient buffer (n readable elements).
 *   For i < n:  s = G[r+1][i] + G[r+2][i] + ... + G[r+W-1][i] + G[r][i]
 *               (indices mod W, fp32, left to right: the order in which the
 *               ring's partial sum for chunk r picks up each worker, the
 *               owner's own term last), a = s / W (IEEE division), then
 *               grad_part[i] = a             if accumulate == 0,
 *               grad_part[i] = grad_part[i] + a otherwise (a later
 *               micro-batch, [L7] "Gradient Accumulation").
 *   wire_dtype   : zs_wire, the precision of the partial sums (0 = fp32;
 *                  with a 16-bit wire each partial is rounded as above).
 *   grad_part    : device fp32[n], written (read too when accumulating).
 *   overflow_flag: device uint32 or NULL; if set, becomes 1 when any
 *                  grad_part[i] / loss_scale is not finite.
 *   loss_scale   : used only for the flag. */
int zs_reduce_scatter_avg(const void *const *worker_grads, int grad_dtype,
                          int wire_dtype, uint32_t world, uint32_t rank,
                          uint64_t n, float *grad_part, int accumulate,
                          uint32_t *overflow_flag, float loss_scale,
                          void *stream);

/* Overflow check of dynamic loss scaling ([Intro] 一.3 items (1) and (3)).
 * Sets *overflow_flag = 1 when any grad_part[i] / loss_scale (fp32 IEEE
 * division) is inf or NaN; otherwise leaves it unchanged.
 * grad_part: device fp32[n]; overflow_flag: device uint32. */
int zs_check_overflow(const float *grad_part, uint64_t n, float loss_scale,
                      uint32_t *overflow_flag, void *stream);

/* AdamW on this rank's partition, in place ([Notes] 三: gradients to FP32
 * and unscaled, moments updated, then the FP32 master; [L7] memory table:
 * fp32 master, m, v; decoupled decay as in AdamW). With g = grad_part[i] /
 * loss_scale and the per-step scalars (formed in double, rounded once to
 * fp32) alpha = lr / (1 - beta1^t), b2 = sqrt(1 - beta2^t),
 * delta = 1 - lr*weight_decay, c1 = 1 - beta1, c2 = 1 - beta2:
 *   m' = beta1*m + c1*g;  v' = beta2*v + c2*(g*g);
 *   d  = sqrt(v')/b2 + eps;  master' = master*delta - alpha*(m'/d)
 * each operator one fp32 IEEE operation, in this order.
 *   master, m, v : device fp32[n], updated in place.
 *   grad_part    : device fp32[n], the averaged (still scaled) gradient.
 *   overflow_flag: device uint32 or NULL. When non-NULL and the flag is set
 *                  at kernel start, nothing is written (the step is skipped)
 *                  -- no host round trip is needed to gate the update. */
int zs_adamw_step(float *master, float *m, float *v, const float *grad_part,
                  uint64_t n, const zs_adamw_hparams *hp,
                  const uint32_t *overflow_flag, void *stream);

/* This rank's contribution to the parameter all-gather ([Notes] 三: the
 * owner refreshes its 16-bit parameters; [Intro] (12) and [L7] "ZeRO Stage
 * 1": AllGather of the updated parameters).
 *   gather_buf[offset + i] = round_to_nearest_even_16(master[i]), i < n.
 *   master     : device fp32[n].
 *   gather_buf : device 16-bit flat buffer (world * chunk elements in the
 *                usual layout); only [offset, offset + n) is written.
 *   overflow_flag: device uint32 or NULL; when set, nothing is written. */
int zs_cast_gather(const float *master, void *gather_buf, int param_dtype,
                   uint64_t offset, uint64_t n, const uint32_t *overflow_flag,
                   void *stream);

/* One whole shard step in a single pass over HBM: the owner's sequence of
 * [Notes] 三 (ZeRO-1: reduce the gradient partition this rank owns, convert
 * to fp32, update the fp32 optimizer state and master weights, refresh the
 * 16-bit parameters for the all-gather) as [L7] "ZeRO Stage 2" and
 * [Intro] 一.3 item (12) run it with the gradient sharded too, plus the
 * loss-scaling check of [Intro] 一.3 items (1) and (3) and the
 * micro-batch accumulation of [L7] "Gradient Accumulation": reduce-scatter
 * average (with optional accumulated micro-batches), unscale, overflow
 * check, AdamW and cast, with the arithmetic of the calls above, element
 * for element.
 * The update is written out of place, to an output set that must not
 * overlap the input set (ZS_ERR_ALIAS), so a step whose flag turns out set
 * leaves the input set untouched: the caller reads the flag, then either
 * swaps the sets (flag 0) or keeps the input set (flag 1, step skipped).
 * gather_buf belongs to the output set too.
 * With state_layout ZS_STATE_GROUPED, master_in and master_out each point
 * at a grouped state buffer of ceil(n/1024) groups (see zs_state_layout),
 * m_in, v_in, m_out and v_out must be NULL, and every operand must be
 * aligned for 4-element vectors (the state buffers and acc_in to 16 bytes,
 * the gradients and this rank's gather slice to 8); otherwise
 * ZS_ERR_INVALID_ARG (non-NULL m/v pointers, an unknown layout) or
 * ZS_ERR_UNSUPPORTED (alignment). acc_in, the gradients and the gather
 * buffer keep their flat layout.
 * Timing only (the values written never change): in either state layout
 * at world >= 40 on launches of at least 4 GB of model bytes, each wave
 * holds its stores until a window of the device's wall clock that every
 * CU reads alike (the last eighth of each 30.72 us period), so the chip's
 * writes reach memory together instead of mixed into its reads; every wait
 * ends within one period. For measurements the environment variables
 * ZS_FUSED_BLOCKS_PER_CU (blocks per CU, 0 = uncapped), ZS_FUSED_SUM
 * ("batched"), ZS_FUSED_W1 ("block256") and ZS_FUSED_WRITE_WINDOW ("off",
 * or "<period in us>,<open fraction>" for every rolling-sum launch: world
 * >= 5 with operands aligned for 4-element vectors;
 * periods under 64 wall-clock ticks mean no windows, and the open part is
 * at least 16 ticks) change the launch; they are read at every call. */
typedef struct {
  uint32_t world, rank;
  uint64_t n;
  int32_t grad_dtype, param_dtype;
  const void *const *worker_grads; /* host array [world], as above         */
  const float *acc_in;             /* NULL, or fp32[n] summed micro-batches */
  const float *master_in, *m_in, *v_in;  /* fp32[n] each, read only (or   */
  float *master_out, *m_out, *v_out;     /* the grouped buffers), written  */
  void *gather_buf;                /* 16-bit flat buffer                    */
  uint64_t gather_offset;          /* element offset of this rank's slice   */
  uint32_t *overflow_flag;         /* device uint32, OR-ed                  */
  zs_adamw_hparams hp;
  int32_t wire_dtype;              /* zs_wire; 0 = fp32 partial sums        */
  int32_t state_layout;            /* zs_state_layout; 0 = split arrays     */
} zs_step_args;

int zs_step_fused(const zs_step_args *args, void *stream);

/* One step of the ring all-gather of the 16-bit parameters over `world`
 * replicas of the flat buffer held on this GPU ([Notes] 二: each GPU passes
 * the chunk it holds to its successor, and after W-1 steps every GPU holds
 * every chunk; [Intro] (12) and [L7] "ZeRO Stage 1": AllGather of the
 * updated parameters). Chunks are the partition of zs_partition:
 * chunk c = elements [c*P, min(phi, (c+1)*P)), P = ceil(phi / world).
 * At step s (1 <= s < world) replica k's chunk (k + sigma - s + 1) mod W is
 * copied into replica (k + 1) mod W at the same offset; with sigma = 0 rank
 * k starts out holding chunk k (ZeRO's owner layout), sigma = 1 replays the
 * page's labelling. Running s = 1 .. W-1 in order on one stream completes
 * the gather.
 *   replicas: host array of `world` device pointers, each to phi 16-bit
 *             elements; they must not overlap (ZS_ERR_ALIAS).
 * Errors: ZS_ERR_INVALID_ARG for null pointers, world == 0 or > 64,
 * sigma >= world, step outside [1, world). */
int zs_all_gather_step(void *const *replicas, uint32_t world, uint64_t phi, uint32_t sigma,
                       uint32_t step, void *stream);

/* ZeRO-Offload update on the host ([Intro] 一.3 item (16): the update is
 * cheap, so optimizer states and gradients live in CPU memory while the
 * forward and backward stay on the GPU). The reduction stays on the GPU
 * (zs_reduce_scatter_avg); the caller copies the fp32 averaged gradient
 * partition to host memory, calls this, and copies the 16-bit parameters
 * back into the gather buffer.
 *   Pass 1: *overflow = 1 if any grad_part[i] / loss_scale is not finite;
 *           then nothing is written (the step is skipped).
 *   Pass 2: master, m, v updated in place with exactly the arithmetic of
 *           zs_adamw_step, and params16[i] = RNE16(master'[i]).
 *   master, m, v, grad_part: host fp32[n]; params16: host 16-bit[n].
 *   threads: worker threads (<= 0: the CPUs in the process's affinity mask,
 *            at most 64); every range runs with round-to-nearest,
 *            subnormals kept.
 * Blocks until done. Errors: ZS_ERR_INVALID_ARG for null pointers, a bad
 * param dtype, a non-finite or non-positive loss scale, step_t == 0 or
 * hyper-parameters outside their ranges (zs_adamw_hparams). */
int zs_cpu_step(float *master, float *m, float *v, const float *grad_part, uint64_t n,
                const zs_adamw_hparams *hp, void *params16, int param_dtype, int threads,
                uint32_t *overflow);

/* The update half of the ZeRO-Offload step ([Intro] 一.3 item (16): the
 * optimizer update runs on the CPU where the states live) without its
 * check: pass 2 of zs_cpu_step alone, for a caller that has already established
 * that no grad_part[i] / loss_scale is non-finite, e.g. with
 * zs_check_overflow on the device before the copy (which lets the update
 * start on the first pieces of the gradient while the rest is still in
 * flight). Same arithmetic, same arguments; with a non-finite gradient the
 * state is updated with it (nothing is checked). Blocks until done.
 * Errors: as zs_cpu_step. */
int zs_cpu_update(float *master, float *m, float *v, const float *grad_part, uint64_t n,
                  const zs_adamw_hparams *hp, void *params16, int param_dtype, int threads);

/* One whole ZeRO-Offload optimizer step after the reduction ([Intro] 一.3
 * item (16)), pipelined over PCIe: the GPU checks the partition
 * (zs_check_overflow's test) and its 4-byte flag reaches the host first; on
 * a clean step the gradient comes to the host in `pieces` consecutive
 * pieces, the host pool updates each piece as it lands (the arithmetic of
 * zs_cpu_update), and each finished piece's 16-bit parameters are copied
 * back while later pieces are still being updated. All copies run on
 * `stream`, after the work already queued there.
 *   grad_dev:    device fp32[n], the averaged, still loss-scaled gradient
 *                partition (zs_reduce_scatter_avg's output).
 *   grad_host:   host fp32[n] staging for it; params_host: host 16-bit[n]
 *                staging for the parameters. Both should be pinned
 *                (hipHostMalloc) for the copies to overlap the update.
 *   master, m, v: host fp32[n], updated in place on a clean step.
 *   params_dev:  device 16-bit[n], this rank's slice of the gather buffer.
 *   flag_dev:    device uint32 scratch (the call zeroes it); flag_host: a
 *                host uint32 (pinned) that receives the flag.
 *   threads:     as zs_cpu_step; pieces: 1 .. 1024 (boundaries at
 *                multiples of 64 elements).
 *   stream:      HIP stream (NULL = the default stream).
 *   *committed:  1 if the step was applied, 0 if it was skipped (then
 *                nothing on the host or in params_dev is written).
 * Blocks until the host update is done; the last parameter copies may still
 * be in flight on `stream`, so work queued there afterwards sees the new
 * parameters, and params_host must not be rewritten before `stream` passes
 * this point. Errors: ZS_ERR_INVALID_ARG (null pointer, bad dtype, pieces
 * out of range, host buffers that overlap, or arguments zs_cpu_update
 * refuses), ZS_ERR_UNSUPPORTED for n > 2^48, both before any HIP call;
 * ZS_ERR_HIP if a copy, the check or a wait fails (the call then waits for
 * the stream; the host state may be partly updated). n == 0 commits without
 * touching the GPU. */
int zs_offload_step(const float *grad_dev, float *grad_host, float *master, float *m, float *v,
                    void *params_host, void *params_dev, uint64_t n, const zs_adamw_hparams *hp,
                    int param_dtype, uint32_t *flag_dev, uint32_t *flag_host, int threads,
                    int pieces, void *stream, int *committed);

/* Host-side commit/skip bookkeeping of dynamic loss scaling ([Intro] 一.3
 * items (1) and (3) name it without a rule). With dynamic != 0: on overflow
 * the scale halves, clean_steps resets and step_t stays; otherwise
 * step_t += 1 and clean_steps += 1, and when clean_steps reaches
 * growth_interval the scale doubles for the next step and clean_steps
 * restarts at 0. With dynamic == 0 the scale never changes. Host-only.
 * Errors: ZS_ERR_INVALID_ARG for a NULL state. */
typedef struct {
  float scale;
  uint32_t clean_steps;
  uint32_t growth_interval;
  uint32_t dynamic;
  uint64_t step_t;   /* committed steps */
  uint64_t skipped;  /* skipped steps   */
} zs_loss_scaler;

int zs_scaler_update(zs_loss_scaler *s, uint32_t overflow);

/* One committed-or-skipped optimizer step, synchronously: the commit-or-skip
 * decision of dynamic loss scaling ([Intro] 一.3 items (1) and (3)) taken on
 * the host right after the fused pass, with one 4-byte device-to-host copy.
 *   1. zs_step_fused(a) with a->hp.loss_scale and a->hp.step_t replaced by
 *      scaler->scale and scaler->step_t + 1 (the other fields of a->hp are
 *      used as given);
 *   2. the uint32 at a->overflow_flag is copied to *host_flag (host memory;
 *      page-locked memory avoids a staging copy) and the call waits for it
 *      (busy-polling the host word and the stream) -- unlike the other
 *      kernel entry points, this call blocks until the step is done;
 *   3. zs_scaler_update(scaler, flag); *committed = (flag == 0).
 * The caller then swaps the input and output sets when *committed is 1.
 * ev_start / ev_stop: NULL, or hipEvent_t handles recorded on `stream`
 * immediately before and after the fused kernel (for timing). Errors: as zs_step_fused;
 * ZS_ERR_INVALID_ARG for a NULL scaler, host_flag or committed, or a
 * non-finite / non-positive scale; ZS_ERR_HIP if the copy or the
 * synchronization fails (including an earlier kernel fault on the stream);
 * on any error the scaler is left unchanged. */
int zs_step_commit(const zs_step_args *a, zs_loss_scaler *scaler, uint32_t *host_flag,
                   void *stream, void *ev_start, void *ev_stop, int *committed);

/* zs_step_commit for callers that cannot allocate device memory (code that
 * must not call hipMalloc, tight serving loops, harnesses that forbid it):
 * the same step, the same kernels and the same results, with the overflow
 * word kept in the library's own device memory instead of a->overflow_flag,
 * which is not used and may be NULL. The caller still passes every input and
 * output; the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine) and clears the word itself, with a one-thread kernel on
 * `stream` before the fused kernel, so nothing needs zeroing between calls.
 * The word is one uint32 per device, in a static device array that each
 * device holding the library keeps until the process ends; the library
 * resolves its address (hipGetSymbolAddress) on the first call with that
 * device current. Its size does not depend on n, so no size is refused for
 * it beyond what zs_step_fused refuses. Every call on one device shares that
 * word: calls that overlap on one device (other streams or host threads)
 * race and must be serialized by the caller. Arguments, blocking, ev_start /
 * ev_stop and the scaler update are as for zs_step_commit. Errors: as
 * zs_step_commit (a NULL a->overflow_flag is accepted); ZS_ERR_UNSUPPORTED
 * for a device ordinal above 63; ZS_ERR_HIP if the address of the word
 * cannot be resolved, before anything is enqueued. */
int zs_step_commit_noalloc(const zs_step_args *a, zs_loss_scaler *scaler, uint32_t *host_flag,
                           void *stream, void *ev_start, void *ev_stop, int *committed);

/* Device-resident commit-or-skip ([Intro] 一.3 items (1) and (3): dynamic
 * loss scaling skips the update of a step whose unscaled gradient is not
 * finite and adjusts the scale). The same rule as zs_scaler_update, kept in
 * device memory and applied by a kernel, so consecutive steps need no
 * device-to-host round trip and can be queued (or captured in a HIP graph)
 * back to back. The layout is public: the caller allocates
 * sizeof(zs_device_scaler) bytes of device memory (8-byte aligned), fills it
 * from zs_device_scaler_make's host image with one copy, and may copy it back
 * at any time the stream is idle to read the scaler.
 *   scale .. skipped : as in zs_loss_scaler; scale is the next step's.
 *   beta1_t, beta2_t : beta1^(step_t+1), beta2^(step_t+1) in binary64, the
 *                      powers the next step's bias corrections use; the
 *                      commit multiplies them by beta once per committed
 *                      step, the same repeated products zs_adamw_step forms.
 *   epoch            : steps run on this image (committed + skipped); the
 *                      commit advances it.
 *   flag_epoch       : epoch + 1 of the latest step whose check failed
 *                      (0: none). A fused pass that finds a non-finite
 *                      value stores its epoch + 1 here, so nothing has to
 *                      be cleared between steps.
 *   checked_epoch    : the epoch the latest fused pass ran with; its step
 *                      is skipped exactly when flag_epoch == checked_epoch
 *                      + 1.
 *   last_flag        : 1 if the most recent step was skipped, else 0.
 *   bad_scale        : steps that found the scale not finite or not > 0
 *                      (such a step is skipped like an overflow).
 *   last_alpha, last_bc2 : lr/(1-beta1^t) and sqrt(1-beta2^t), rounded to
 *                      fp32, as the most recent step used them. */
typedef struct {
  float scale;
  uint32_t clean_steps;
  uint32_t growth_interval;
  uint32_t dynamic;
  uint64_t step_t;
  uint64_t skipped;
  double beta1_t, beta2_t;
  uint64_t epoch;
  uint64_t flag_epoch;
  uint64_t checked_epoch;
  uint32_t last_flag;
  uint32_t bad_scale;
  float last_alpha, last_bc2;
} zs_device_scaler;

/* Host image of a device scaler ([Intro] 一.3 items (1) and (3): the
 * dynamic loss scale and its skip rule; the bias-correction powers of the
 * AdamW update that [Notes] 三 runs on the owner's fp32 state) that
 * continues from the host scaler `s` (beta powers formed by step_t + 1
 * repeated binary64 multiplications).
 * Errors: ZS_ERR_INVALID_ARG for NULL pointers, a scale that is not
 * finite and > 0, or a beta outside [0, 1). */
int zs_device_scaler_make(const zs_loss_scaler *s, float beta1, float beta2,
                          zs_device_scaler *out);

/* One optimizer step with the commit-or-skip decision taken on the device.
 * Enqueues on `stream`, never waits:
 *   1. the zs_step_fused pass with hp.loss_scale = dev->scale and the bias
 *      corrections from dev->beta1_t / dev->beta2_t (a->hp.loss_scale and
 *      a->hp.step_t are ignored; lr, betas, eps and weight decay come from
 *      a->hp); it records the epoch it ran with in dev->checked_epoch and,
 *      on a non-finite value, stores that epoch + 1 in dev->flag_epoch
 *      (a->overflow_flag is ignored);
 *   2. a commit kernel: when dev->flag_epoch == dev->checked_epoch + 1 it
 *      copies the input set into the output set and writes the cast of
 *      master_in into the gather slice, so the output set always holds the
 *      state after the step (updated, or unchanged when skipped); then it
 *      applies the zs_scaler_update rule to *dev, records last_flag and
 *      advances dev->epoch. With n == 0 there is no fused pass and the
 *      step commits.
 * The caller swaps the input and output sets after every call, without
 * looking at the flag. Micro-batches before the last one go through
 * zs_reduce_scatter_avg with no flag: a non-finite partial stays non-finite
 * through the fp32 accumulation, so the fused pass's check of
 * (acc_in + average) / scale sees it.
 * ev_start / ev_stop: NULL, or hipEvent_t handles recorded immediately
 * before and after the fused kernel. Calls that share a dev must be ordered
 * (one stream). Errors: as zs_step_fused (ZS_ERR_INVALID_ARG also for a
 * NULL or not 8-byte-aligned dev, ZS_ERR_ALIAS also for a dev that
 * overlaps an output buffer, master_in, m_in, v_in, acc_in or a worker's
 * gradient); argument errors return before anything
 * is enqueued. ZS_ERR_HIP from the second launch leaves the fused pass
 * enqueued without its commit: dev->epoch has not advanced, and the caller
 * must not swap the sets (rerunning the step is safe: the fused pass does
 * not write its input set and runs again at the same epoch). */
int zs_step_device(const zs_step_args *a, zs_device_scaler *dev, void *stream, void *ev_start,
                   void *ev_stop);

#ifdef __cplusplus
}
#endif
#endif /* ZEROSHARD_H */
