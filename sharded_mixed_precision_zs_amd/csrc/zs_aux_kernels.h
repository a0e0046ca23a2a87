/*
 * zs_aux_kernels.h -- device code of libzeroshard (gfx950) around the
 * fused step: the device-resident commit or skip, and one step of the ring
 * all-gather of the 16-bit parameters. Kept apart from zs_kernels.h, which
 * holds the hot path. Sources, cited by page title and section:
 *   [Notes] lecture notes on DP / DDP / DeepSpeed ZeRO (gitcode.csdn.net)
 *   [Intro] "并行训练框架DeepSpeed介绍"
 */
#ifndef ZS_AUX_KERNELS_H
#define ZS_AUX_KERNELS_H

#include "zs_kernels.h"

namespace zs {

/* ------------------------------------------------------------------------
 * Commit or skip on the device ([Intro] 一.3 items (1) and (3): a step whose
 * unscaled gradient is not finite is skipped and the loss scale adjusted).
 * Runs after the fused pass on the same stream. The fused pass recorded the
 * epoch it ran with (checked_epoch) and, if it found a non-finite value,
 * stored that epoch + 1 in flag_epoch; both were written by the previous
 * kernel, so every block reads them with plain loads and they stay fixed
 * while this kernel runs. A skipped step's blocks copy the input set into
 * the output set and recast master_in into the gather slice (grid-stride),
 * so the output set holds the state after the step either way. Thread 0 of
 * block 0 alone applies the scaler rule (the host's zs_scaler_update, field
 * for field), advances the beta powers on a commit and advances the epoch;
 * no other block reads what it writes, so the grid needs no arrival count,
 * atomic or fence, and nothing has to be cleared for the next step.
 * ---------------------------------------------------------------------- */

/* With no arrival count the grid size costs a committed step nothing
 * (32 to 512 blocks measured alike), while a skipped step's restore runs
 * near HBM rate from 256 blocks on. */
constexpr int kCommitBlock = 1024;  /* threads per commit block     */
constexpr int kCommitBlocks = 256;  /* at most this many blocks     */

/* Zeroes one uint32 word (a vector store from lane 0). zs_step_commit_noalloc
 * clears the overflow word it keeps in the library's device memory with it,
 * on the step's own stream. */
__global__ __launch_bounds__(64) void clear_word_kernel(uint32_t *word) {
  if (threadIdx.x == 0) *word = 0u;
}

struct CommitArgs {
  zs_device_scaler *dev;
  const float *master_in, *m_in, *v_in;
  float *master_out, *m_out, *v_out;
  uint16_t *param_out;  /* already at this rank's offset */
  uint64_t n;
  double beta1, beta2;
};

/* GR: the state in the grouped layout (master_in / master_out hold it); a
 * vector of up to 8 elements at a multiple of VEC never straddles a group. */
template <int VEC, int PDT, bool GR = false>
__device__ __forceinline__ void restore_vec(const CommitArgs &c, uint64_t i0) {
  const StateAt<GR> at(i0);
  const float *m_in = GR ? c.master_in : c.m_in, *v_in = GR ? c.master_in : c.v_in;
  float *m_out = GR ? c.master_out : c.m_out, *v_out = GR ? c.master_out : c.v_out;
  float x[VEC];
  ldf<VEC>(c.master_in + at.th, x);
  stf<VEC>(c.master_out + at.th, x);
  st16<VEC, PDT>(c.param_out + i0, x);
  ldf<VEC>(m_in + at.m, x);
  stf<VEC>(m_out + at.m, x);
  ldf<VEC>(v_in + at.v, x);
  stf<VEC>(v_out + at.v, x);
}

template <int VEC, int PDT, bool GR = false>
__global__ __launch_bounds__(kCommitBlock) void commit_kernel(CommitArgs c) {
  zs_device_scaler *d = c.dev;
  /* an empty partition had no fused pass (nothing to check, nothing
   * recorded): it commits at the current epoch; its grid is one block, so
   * reading the epoch that block 0 advances is safe */
  const bool empty = c.n == 0;
  const uint64_t e = empty ? d->epoch : d->checked_epoch;
  const bool skip = !empty && d->flag_epoch == e + 1;
  if (skip) {
    const uint64_t stride = (uint64_t)gridDim.x * kCommitBlock * VEC;
    for (uint64_t i0 = ((uint64_t)blockIdx.x * kCommitBlock + threadIdx.x) * VEC; i0 < c.n;
         i0 += stride) {
      if (i0 + VEC <= c.n) {
        restore_vec<VEC, PDT, GR>(c, i0);
      } else {
        for (uint64_t i = i0; i < c.n; ++i) restore_vec<1, PDT, GR>(c, i);
      }
    }
  }
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  const float scale = d->scale;
  const uint32_t clean0 = d->clean_steps, interval = d->growth_interval, dynamic = d->dynamic;
  if (skip) {
    if (dynamic) d->scale = scale * 0.5f;
    d->clean_steps = 0;
    d->skipped = d->skipped + 1;
  } else {
    d->step_t = d->step_t + 1;
    d->beta1_t = d->beta1_t * c.beta1;
    d->beta2_t = d->beta2_t * c.beta2;
    const uint32_t clean = clean0 + 1;
    if (dynamic && interval && clean >= interval) {
      d->scale = scale * 2.0f;
      d->clean_steps = 0;
    } else {
      d->clean_steps = clean;
    }
  }
  d->last_flag = skip ? 1u : 0u;
  d->epoch = e + 1;
}

/* ------------------------------------------------------------------------
 * One step of the ring all-gather over W replicas of the flat 16-bit
 * parameter buffer ([Notes] 二: after the scatter-reduce each GPU passes the
 * chunk total it holds to its successor; after W-1 such steps every GPU has
 * every chunk; [L7] "Ring AllReduce 算法", phase two). Rank k sends chunk
 * c_k = (k + sigma - step + 1) mod W to rank k+1. blockIdx.y is the sender;
 * each thread copies 8 elements (16 bytes) or, on the ragged end or with
 * misaligned chunks, one at a time.
 * ---------------------------------------------------------------------- */

struct GatherArgs {
  uint16_t *r[ZS_MAX_WORLD];   /* replica k's flat buffer */
  uint32_t world, sigma, step;
  uint64_t phi, chunk;
};

template <int VEC>
__global__ __launch_bounds__(kBlock) void gather_step_kernel(GatherArgs a) {
  const uint32_t k = blockIdx.y;
  const uint32_t c = (uint32_t)(((uint64_t)k + a.sigma + (uint64_t)a.world * a.step - a.step + 1) %
                                a.world);
  const uint64_t begin = (uint64_t)c * a.chunk;
  if (begin >= a.phi) return;
  const uint64_t len = a.phi - begin < a.chunk ? a.phi - begin : a.chunk;
  const uint16_t *src = a.r[k] + begin;
  uint16_t *dst = a.r[(k + 1) % a.world] + begin;
  const uint64_t i0 = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) * VEC;
  if (i0 >= len) return;
  if (VEC > 1 && i0 + VEC <= len) {
    /* 16 bytes per lane, lane-contiguous: a wave stores 1 KB of whole lines,
     * non-temporally (the next step reads them at most once) */
    Raw16<VEC> v = ld16<VEC, true>(src + i0);
    if constexpr (VEC == 8)
      __builtin_nontemporal_store(u32x4{v.w[0], v.w[1], v.w[2], v.w[3]},
                                  reinterpret_cast<u32x4 *>(dst + i0));
  } else {
    for (uint64_t i = i0; i < len && i < i0 + VEC; ++i) dst[i] = src[i];
  }
}

}  // namespace zs

#endif /* ZS_AUX_KERNELS_H */
