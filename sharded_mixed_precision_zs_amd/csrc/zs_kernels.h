/*
 * zs_kernels.h -- device code of libzeroshard (gfx950): per-element
 * arithmetic, vector loads/stores, the ring-order sum and the reduction,
 * update and fused-step kernels. The commit and all-gather kernels are in
 * zs_aux_kernels.h. The host side and the C ABI are in zeroshard.hip, which
 * includes both once. Sources, cited by page title and section:
 *   [Notes] lecture notes on DP / DDP / DeepSpeed ZeRO (gitcode.csdn.net)
 *   [Intro] "并行训练框架DeepSpeed介绍"
 *   [L7]    "第 7 讲：Parallelism（上）" (CS336 lecture 7)
 *
 * Design (all kernels are HBM-bandwidth bound; nothing here is a dense
 * contraction, so there is no MFMA):
 *   - one 64-bit element index per thread-vector; each thread owns VEC
 *     consecutive elements (VEC = 8 when every operand is 16-byte aligned:
 *     128-bit loads of 16-bit gradients, 2 x 128-bit loads of fp32 state);
 *   - the W-way gradient sum runs in fp32 registers in the fixed ring order,
 *     with non-temporal loads issued in batches ahead of the in-order adds;
 *   - the overflow flag is a wave ballot, one vector atomic OR per wave that
 *     saw a non-finite value;
 *   - 16-bit outputs use the hardware round-to-nearest-even converts
 *     (v_cvt_pk_bf16_f32, v_cvt_f16_f32);
 *   - built with -ffp-contract=off: every arithmetic operator is one IEEE
 *     binary32 operation; division and square root are the correctly rounded
 *     sequences, denormals are kept.
 */
#ifndef ZS_KERNELS_H
#define ZS_KERNELS_H

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "zeroshard.h"

namespace zs {

constexpr int kBlock = 256;     /* threads per workgroup (4 waves of 64)   */
constexpr int kLoadBatch = 8;   /* gradient vectors in flight per thread   */

/* Access shape of the fused kernel (template parameter SHAPE): how many
 * workers' gradient loads the sum issues ahead of its adds, and whether the
 * new state and parameters are stored non-temporally.
 *   kShapeB8     kLoadBatch ahead, plain stores;
 *   kShapeB16    16 ahead, plain stores;
 *   kShapeB16Nt  16 ahead, non-temporal stores;
 *   kShapeB8Nt   kLoadBatch ahead, non-temporal stores.
 * Non-temporal stores pay only when a wave's store covers whole lines: with
 * 4-element vectors a wave's 16-byte fp32 stores span 1 KB of contiguous
 * lines, while with 8-element vectors a lane's 32 bytes take two stores and
 * each 64-byte line is half-written by two instructions, which then leave
 * the L2 as separate writes (14 % more write bytes at W = 64, measured).
 * The library launches kShapeB8NtL (W <= 4) and kShapeR4NtL below
 * (W >= 5) on 4-element vectors, and kShapeB8 on the narrower vectors of
 * unaligned operands; the other shapes are kept for the measurement
 * library's variants. */
constexpr int kShapeB8 = 0, kShapeB16 = 1, kShapeB16Nt = 2, kShapeB8Nt = 3;
/* as kShapeB16Nt / kShapeB8Nt, with the fp32 state (and the accumulated
 * gradient) also loaded non-temporally: read once per step, like the
 * gradients (+1 to 1.8 % at W = 1 and W = 8 against plain state loads,
 * neutral at W = 64) */
constexpr int kShapeB16NtL = 4, kShapeB8NtL = 5;
/* kShapeR4NtL: the rolling sum (ring_sum_roll): four workers' loads ahead
 * of the adds at all times, each refilled as soon as its worker is added,
 * with the fp32 state loaded while the last workers are in flight;
 * non-temporal loads and stores as kShapeB8NtL. */
constexpr int kShapeR4NtL = 6;

constexpr int shape_batch(int shape) {
  return shape == kShapeR4NtL ? 4
         : shape == kShapeB8 || shape == kShapeB8Nt || shape == kShapeB8NtL ? kLoadBatch : 16;
}
constexpr bool shape_nt_stores(int shape) { return shape >= kShapeB16Nt; }
constexpr bool shape_nt_loads(int shape) { return shape >= kShapeB16NtL; }
constexpr bool shape_rolling(int shape) { return shape == kShapeR4NtL; }

/* ------------------------------------------------------------------------
 * Per-element arithmetic. Each line is written exactly in the order the
 * header documents; with contraction off, each operator rounds once.
 * ---------------------------------------------------------------------- */

struct AdamK {
  float alpha, b2, delta, c1, c2, beta1, beta2, eps;
};

struct Scales {
  float wf, inv_w;      /* world as float; 2^-k when world = 2^k         */
  float sf, inv_s;      /* loss scale; 2^-k when it is 2^k               */
  int w_pow2, s_pow2;   /* multiply by the exact reciprocal instead      */
};

__device__ __forceinline__ float average(float s, const Scales &k) {
  /* s / W; for W = 2^k the product with 2^-k is the same correctly
   * rounded value, without the division sequence. */
  return k.w_pow2 ? s * k.inv_w : s / k.wf;
}

__device__ __forceinline__ float unscale(float a, const Scales &k) {
  return k.s_pow2 ? a * k.inv_s : a / k.sf;
}

/* The loss-scale half of Scales for a scale read from device memory (the
 * device-resident commit flow): the same power-of-two test as the host's
 * (a normal 2^k, |k| <= 126, whose reciprocal 2^-k is exact). Values are
 * moved to scalar registers: they are the same for every lane. Returns false
 * when the scale is not finite and > 0 (the step is then skipped). */
__device__ __forceinline__ bool dev_scales(float sc, Scales &k) {
  const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(sc));
  const uint32_t e = (b >> 23) & 0xffu;
  k.sf = __uint_as_float(b);
  k.s_pow2 = (b & 0x807fffffu) == 0 && e >= 1 && e <= 253;
  k.inv_s = k.s_pow2 ? __uint_as_float((254u - e) << 23) : 0.0f;
  const float s = __uint_as_float(b);
  return s > 0.0f && __builtin_isfinite(s);
}

__device__ __forceinline__ float adamw_elem(float theta, float &m, float &v,
                                            float g, const AdamK &k) {
  float decayed = theta * k.delta;             /* decoupled weight decay  */
  float m1 = k.beta1 * m + k.c1 * g;           /* first moment            */
  float v1 = k.beta2 * v + k.c2 * (g * g);     /* second moment           */
  float d = sqrtf(v1) / k.b2 + k.eps;          /* bias-corrected rms      */
  float out = decayed - k.alpha * (m1 / d);    /* alpha = lr / (1-b1^t)   */
  m = m1;
  v = v1;
  return out;
}

/* ------------------------------------------------------------------------
 * 16-bit formats. A 32-bit word holds elements 2j (low half) and 2j+1.
 * ---------------------------------------------------------------------- */

template <int DT>
__device__ __forceinline__ float up_lo(uint32_t w) {
  if constexpr (DT == ZS_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}

template <int DT>
__device__ __forceinline__ float up_hi(uint32_t w) {
  if constexpr (DT == ZS_BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

/* Two fp32 -> one word of two 16-bit values, round to nearest even. */
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  if constexpr (DT == ZS_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

template <int DT>
__device__ __forceinline__ uint16_t pack1(float x) {
  if constexpr (DT == ZS_BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

/* ------------------------------------------------------------------------
 * Vector loads / stores of VEC elements (VEC in {8, 4, 2, 1}).
 * ---------------------------------------------------------------------- */

template <int VEC>
struct Raw16 {                         /* VEC 16-bit values, as loaded      */
  uint32_t w[VEC / 2 > 0 ? VEC / 2 : 1];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

/* NT = true marks the load non-temporal: gradients are read exactly once,
 * so they should not displace cache lines that are. */
template <int VEC, bool NT = false>
__device__ __forceinline__ Raw16<VEC> ld16(const uint16_t *__restrict__ p) {
  Raw16<VEC> r;
  if constexpr (VEC == 8) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
    u32x4 t;
    if constexpr (NT) t = __builtin_nontemporal_load(q); else t = *q;
    r.w[0] = t.x; r.w[1] = t.y; r.w[2] = t.z; r.w[3] = t.w;
  } else if constexpr (VEC == 4) {
    const u32x2 *q = reinterpret_cast<const u32x2 *>(p);
    u32x2 t;
    if constexpr (NT) t = __builtin_nontemporal_load(q); else t = *q;
    r.w[0] = t.x; r.w[1] = t.y;
  } else if constexpr (VEC == 2) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    if constexpr (NT) r.w[0] = __builtin_nontemporal_load(q); else r.w[0] = *q;
  } else {
    if constexpr (NT) r.w[0] = __builtin_nontemporal_load(p); else r.w[0] = *p;
  }
  return r;
}

template <int VEC, int DT>
__device__ __forceinline__ void upcast(const Raw16<VEC> &r, float (&x)[VEC]) {
  if constexpr (VEC == 1) {
    x[0] = up_lo<DT>(r.w[0]);
  } else {
#pragma unroll
    for (int j = 0; j < VEC / 2; ++j) {
      x[2 * j] = up_lo<DT>(r.w[j]);
      x[2 * j + 1] = up_hi<DT>(r.w[j]);
    }
  }
}

template <int VEC, int DT>
__device__ __forceinline__ void add_up(float (&s)[VEC], const Raw16<VEC> &r) {
  float x[VEC];
  upcast<VEC, DT>(r, x);
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = s[e] + x[e];
}

template <int VEC>
__device__ __forceinline__ void ldf(const float *__restrict__ p, float (&x)[VEC]) {
  if constexpr (VEC == 8) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else if constexpr (VEC == 4) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  } else if constexpr (VEC == 2) {
    float2 a = *reinterpret_cast<const float2 *>(p);
    x[0] = a.x; x[1] = a.y;
  } else {
    x[0] = *p;
  }
}

/* ldf with the loads marked non-temporal when NT (VEC 4 or 8) */
template <int VEC, bool NT>
__device__ __forceinline__ void ldf_p(const float *__restrict__ p, float (&x)[VEC]) {
  if constexpr (!NT || (VEC != 4 && VEC != 8)) {
    ldf<VEC>(p, x);
  } else {
    typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h) {
      f4 a = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p) + h);
      x[4 * h] = a.x; x[4 * h + 1] = a.y; x[4 * h + 2] = a.z; x[4 * h + 3] = a.w;
    }
  }
}

template <int VEC>
__device__ __forceinline__ void stf(float *__restrict__ p, const float (&x)[VEC]) {
  if constexpr (VEC == 8) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  } else if constexpr (VEC == 4) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  } else if constexpr (VEC == 2) {
    *reinterpret_cast<float2 *>(p) = make_float2(x[0], x[1]);
  } else {
    *p = x[0];
  }
}

/* stf / st16 with the stores marked non-temporal when NT: the new state
 * and parameters are not read again by this step. */
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int VEC, bool NT>
__device__ __forceinline__ void stf_p(float *__restrict__ p, const float (&x)[VEC]) {
  if constexpr (!NT) {
    stf<VEC>(p, x);
  } else if constexpr (VEC == 8) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4 *>(p + 4));
  } else if constexpr (VEC == 4) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4 *>(p));
  } else if constexpr (VEC == 2) {
    __builtin_nontemporal_store(f32x2{x[0], x[1]}, reinterpret_cast<f32x2 *>(p));
  } else {
    __builtin_nontemporal_store(x[0], p);
  }
}

template <int VEC, int DT>
__device__ __forceinline__ void st16(uint16_t *__restrict__ p, const float (&x)[VEC]) {
  if constexpr (VEC == 8) {
    *reinterpret_cast<uint4 *>(p) =
        make_uint4(pack2<DT>(x[0], x[1]), pack2<DT>(x[2], x[3]),
                   pack2<DT>(x[4], x[5]), pack2<DT>(x[6], x[7]));
  } else if constexpr (VEC == 4) {
    *reinterpret_cast<uint2 *>(p) =
        make_uint2(pack2<DT>(x[0], x[1]), pack2<DT>(x[2], x[3]));
  } else if constexpr (VEC == 2) {
    *reinterpret_cast<uint32_t *>(p) = pack2<DT>(x[0], x[1]);
  } else {
    *p = pack1<DT>(x[0]);
  }
}

template <int VEC, int DT, bool NT>
__device__ __forceinline__ void st16_p(uint16_t *__restrict__ p, const float (&x)[VEC]) {
  if constexpr (!NT) {
    st16<VEC, DT>(p, x);
  } else if constexpr (VEC == 8) {
    __builtin_nontemporal_store(u32x4{pack2<DT>(x[0], x[1]), pack2<DT>(x[2], x[3]),
                                      pack2<DT>(x[4], x[5]), pack2<DT>(x[6], x[7])},
                                reinterpret_cast<u32x4 *>(p));
  } else if constexpr (VEC == 4) {
    __builtin_nontemporal_store(u32x2{pack2<DT>(x[0], x[1]), pack2<DT>(x[2], x[3])},
                                reinterpret_cast<u32x2 *>(p));
  } else if constexpr (VEC == 2) {
    __builtin_nontemporal_store(pack2<DT>(x[0], x[1]), reinterpret_cast<uint32_t *>(p));
  } else {
    __builtin_nontemporal_store(pack1<DT>(x[0]), p);
  }
}

/* ------------------------------------------------------------------------
 * Ring-order sum. g.p[j] is worker (rank + 1 + j) mod W, so summing
 * p[0], p[1], ..., p[W-1] left to right adds the owner's term last: the
 * order in which the ring's running partial for this chunk visits the
 * workers ([Notes] 二 three-GPU example; [L7] "Ring AllReduce 算法").
 *
 * WIRE is the precision of the partial the ring passes on: ZS_WIRE_FP32
 * keeps it in fp32; ZS_WIRE_BF16 / ZS_WIRE_FP16 round it to nearest-even
 * 16 bits at every hop, the last (owner's) one included, as a reduction
 * run in a 16-bit dtype does ([L7] "ZeRO 与 FSDP", reduce_dtype).
 * ---------------------------------------------------------------------- */

struct GradPtrs {
  const uint16_t *p[ZS_MAX_WORLD];
};

template <int WIRE>
__device__ __forceinline__ float on_wire(float x) {
  if constexpr (WIRE == ZS_WIRE_BF16) return __uint_as_float((uint32_t)pack1<ZS_BF16>(x) << 16);
  else if constexpr (WIRE == ZS_WIRE_FP16) return (float)(_Float16)x;
  else return x;
}

template <int VEC, int DT, int WIRE>
__device__ __forceinline__ void set_up(float (&s)[VEC], const Raw16<VEC> &r) {
  upcast<VEC, DT>(r, s);
  if constexpr (WIRE != ZS_WIRE_FP32) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[e] = on_wire<WIRE>(s[e]);
  }
}

template <int VEC, int DT, int WIRE>
__device__ __forceinline__ void add_wire(float (&s)[VEC], const Raw16<VEC> &r) {
  float x[VEC];
  upcast<VEC, DT>(r, x);
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = on_wire<WIRE>(s[e] + x[e]);
}

template <int VEC, int DT, int WIRE>
__device__ __forceinline__ void ring_sum_w(const GradPtrs &g, uint32_t world, uint64_t i0,
                                           float (&s)[VEC]) {
  set_up<VEC, DT, WIRE>(s, ld16<VEC>(g.p[0] + i0));
  uint32_t j = 1;
  for (; j + kLoadBatch <= world; j += kLoadBatch) {
    Raw16<VEC> r[kLoadBatch];
#pragma unroll
    for (int b = 0; b < kLoadBatch; ++b) r[b] = ld16<VEC>(g.p[j + b] + i0);
#pragma unroll
    for (int b = 0; b < kLoadBatch; ++b) add_wire<VEC, DT, WIRE>(s, r[b]);
  }
  for (; j < world; ++j) add_wire<VEC, DT, WIRE>(s, ld16<VEC>(g.p[j] + i0));
}

/* One vector per thread; the wire precision is a uniform runtime choice. */
template <int VEC, int DT>
__device__ __forceinline__ void ring_sum(const GradPtrs &g, uint32_t world, int wire,
                                         uint64_t i0, float (&s)[VEC]) {
  if (wire == ZS_WIRE_BF16) ring_sum_w<VEC, DT, ZS_WIRE_BF16>(g, world, i0, s);
  else if (wire == ZS_WIRE_FP16) ring_sum_w<VEC, DT, ZS_WIRE_FP16>(g, world, i0, s);
  else ring_sum_w<VEC, DT, ZS_WIRE_FP32>(g, world, i0, s);
}

/* The same ring-order sum for U vectors per thread. Loads are issued
 * worker-major (all U vectors of one worker back to back, B workers ahead
 * of the adds) and marked non-temporal. */
template <int VEC, int U, int DT, int WIRE, int B = kLoadBatch>
__device__ __forceinline__ void ring_sum_uw(const GradPtrs &g, uint32_t world,
                                            const uint64_t (&i0)[U], float (&s)[U][VEC]) {
#pragma unroll
  for (int u = 0; u < U; ++u) set_up<VEC, DT, WIRE>(s[u], ld16<VEC, true>(g.p[0] + i0[u]));
  uint32_t j = 1;
  for (; j + B <= world; j += B) {
    Raw16<VEC> r[B][U];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) r[b][u] = ld16<VEC, true>(g.p[j + b] + i0[u]);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) add_wire<VEC, DT, WIRE>(s[u], r[b][u]);
  }
  for (; j < world; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) add_wire<VEC, DT, WIRE>(s[u], ld16<VEC, true>(g.p[j] + i0[u]));
}

/* The same ring-order sum as a rolling pipeline. ring_sum_uw issues a batch
 * of B workers' loads, adds them, and only then issues the next batch, so
 * each wave's loads drain to zero B times per W workers; here the loads of
 * worker j + B are issued as soon as worker j has been added, so a wave
 * keeps B * U loads in flight from its first worker to its last, and
 * `before` (the fp32 state loads) is issued together with the last
 * workers' loads instead of after the whole sum. The adds run in exactly
 * ring_sum_uw's order. Only the last round is irregular: the R < B workers
 * left after the last full refill are loaded with the state and added
 * last; roll_dispatch picks the instance for R so that every load and wait
 * count is fixed at compile time (the compiler's vector-memory wait counts
 * then keep B * U - U loads outstanding at each add; with a run-time
 * guard on the loads they would wait for everything). The scheduling
 * barriers keep the compiler from hoisting the unpacking of a whole batch
 * above the refill loads, which would drain the pipeline again. With
 * W < B + 1 there is nothing to roll and the batched sum runs, followed by
 * `before`. On MI355X, run at 6 to 8 one-wave blocks per CU (fewer bytes in
 * flight per CU than the batched sum at 12 to 16), it streamed the step 3 to
 * 8 % faster at W = 5 and W = 16 to 64 (interleaved timings on one GPU). */
template <int VEC, int U, int DT, int WIRE, int B, int R, typename F>
__device__ __forceinline__ void roll_last(const GradPtrs &g, uint32_t j, const uint64_t (&i0)[U],
                                          Raw16<VEC> (&r)[B][U], float (&s)[U][VEC],
                                          F &before) {
  Raw16<VEC> t[R > 0 ? R : 1][U];
#pragma unroll
  for (int b = 0; b < R; ++b)
#pragma unroll
    for (int u = 0; u < U; ++u) t[b][u] = ld16<VEC, true>(g.p[j + B + b] + i0[u]);
  before();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < B; ++b) {
#pragma unroll
    for (int u = 0; u < U; ++u) add_wire<VEC, DT, WIRE>(s[u], r[b][u]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int b = 0; b < R; ++b) {
#pragma unroll
    for (int u = 0; u < U; ++u) add_wire<VEC, DT, WIRE>(s[u], t[b][u]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int VEC, int U, int DT, int WIRE, int B, int R, typename F>
__device__ __forceinline__ void roll_dispatch(const GradPtrs &g, uint32_t j, const uint64_t (&i0)[U],
                                              Raw16<VEC> (&r)[B][U], float (&s)[U][VEC],
                                              F &before, uint32_t left) {
  if constexpr (R == 0) {
    roll_last<VEC, U, DT, WIRE, B, 0>(g, j, i0, r, s, before);
  } else {
    if (left == (uint32_t)R) roll_last<VEC, U, DT, WIRE, B, R>(g, j, i0, r, s, before);
    else roll_dispatch<VEC, U, DT, WIRE, B, R - 1>(g, j, i0, r, s, before, left);
  }
}

template <int VEC, int U, int DT, int WIRE, int B, typename F>
__device__ __forceinline__ void ring_sum_roll(const GradPtrs &g, uint32_t world,
                                              const uint64_t (&i0)[U], float (&s)[U][VEC],
                                              F &before) {
  if (world < (uint32_t)B + 1) {
    ring_sum_uw<VEC, U, DT, WIRE, B>(g, world, i0, s);
    before();
    return;
  }
  Raw16<VEC> r0[U], r[B][U];
#pragma unroll
  for (int u = 0; u < U; ++u) r0[u] = ld16<VEC, true>(g.p[0] + i0[u]);
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int u = 0; u < U; ++u) r[b][u] = ld16<VEC, true>(g.p[1 + b] + i0[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) set_up<VEC, DT, WIRE>(s[u], r0[u]);
  /* r holds workers j .. j + B - 1; refill while a whole next round exists */
  uint32_t j = 1;
  for (; j + 2 * B <= world; j += B) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
#pragma unroll
      for (int u = 0; u < U; ++u) add_wire<VEC, DT, WIRE>(s[u], r[b][u]);
#pragma unroll
      for (int u = 0; u < U; ++u) r[b][u] = ld16<VEC, true>(g.p[j + B + b] + i0[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  /* j + B <= world < j + 2B: world - j - B workers (0 .. B - 1) remain */
  roll_dispatch<VEC, U, DT, WIRE, B, B - 1>(g, j, i0, r, s, before, world - j - B);
}

/* Wave-level OR of the overflow flag: one vector atomic per wave that saw a
 * non-finite value, issued by its first such lane. */
__device__ __forceinline__ void flag_or(uint32_t *flag, bool bad) {
  unsigned long long m = __ballot(bad);
  if (m && bad && (threadIdx.x & 63u) == (unsigned)(__ffsll(m) - 1))
    atomicOr(flag, 1u);
}

/* ------------------------------------------------------------------------
 * Kernels. Thread t of block b owns elements [i0, i0 + VEC) with
 * i0 = (b * kBlock + t) * VEC; the thread holding the ragged end (fewer
 * than VEC elements left) walks them one at a time with VEC = 1 accesses.
 * The reducing kernels work on tiles of U vectors per thread: vector u of
 * thread t in block b starts at ((b * U + u) * kBlock + t) * VEC for the
 * floor(n / tile) full tiles; the remaining n % tile elements get blocks
 * of their own, one element per thread (see tiled_grid).
 * ---------------------------------------------------------------------- */

constexpr int kTileVecs = 2;  /* U: vectors per thread in the reducing kernels */

__device__ __forceinline__ uint64_t first_elem(int vec) {
  return ((uint64_t)blockIdx.x * kBlock + threadIdx.x) * (uint64_t)vec;
}

struct ReduceArgs {
  GradPtrs g;
  uint32_t world;
  int wire;        /* ZS_WIRE_*: precision of the ring's partials */
  uint64_t n;
  float *out;
  uint32_t *flag;  /* may be null */
  int accumulate;
  Scales k;
};

template <int VEC, int DT>
__device__ __forceinline__ bool reduce_vec(const ReduceArgs &a, const Scales &k, uint64_t i0) {
  float s[VEC], acc[VEC];
  if (a.accumulate) ldf<VEC>(a.out + i0, acc);
  ring_sum<VEC, DT>(a.g, a.world, a.wire, i0, s);
  bool bad = false;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float v = average(s[e], k);
    if (a.accumulate) v = acc[e] + v;
    s[e] = v;
    bad |= !__builtin_isfinite(unscale(v, k));
  }
  stf<VEC>(a.out + i0, s);
  return bad;
}

template <int VEC, int U, int DT, int WIRE, bool NTS>
__device__ __forceinline__ bool reduce_tile(const ReduceArgs &a, const Scales &k, uint64_t base) {
  uint64_t i0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) i0[u] = base + ((uint64_t)u * kBlock + threadIdx.x) * VEC;
  float s[U][VEC];
  ring_sum_uw<VEC, U, DT, WIRE>(a.g, a.world, i0, s);
  bool bad = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc[VEC];
    if (a.accumulate) ldf<VEC>(a.out + i0[u], acc);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float v = average(s[u][e], k);
      if (a.accumulate) v = acc[e] + v;
      s[u][e] = v;
      bad |= !__builtin_isfinite(unscale(v, k));
    }
    stf_p<VEC, NTS>(a.out + i0[u], s[u]);
  }
  return bad;
}

/* NTS: the fp32 partition is stored non-temporally (whole lines with
 * 4-element vectors); the launch uses it when nothing is accumulated. */
template <int VEC, int U, int DT, int WIRE, bool NTS>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceArgs a) {
  const uint64_t tile = (uint64_t)kBlock * U * VEC;
  const uint64_t full = a.n / tile;  /* blocks past `full` cover the tail */
  bool bad = false;
  if (blockIdx.x < full) {
    bad = reduce_tile<VEC, U, DT, WIRE, NTS>(a, a.k, (uint64_t)blockIdx.x * tile);
  } else {
    uint64_t i = full * tile + (uint64_t)(blockIdx.x - full) * kBlock + threadIdx.x;
    if (i < a.n) bad = reduce_vec<1, DT>(a, a.k, i);
  }
  if (a.flag) flag_or(a.flag, bad);
}

struct CheckArgs {
  const float *a;
  uint64_t n;
  uint32_t *flag;
  Scales k;
};

template <int VEC>
__global__ __launch_bounds__(kBlock) void check_kernel(CheckArgs c) {
  uint64_t i0 = first_elem(VEC);
  if (i0 >= c.n) return;
  bool bad = false;
  if (i0 + VEC <= c.n) {
    float x[VEC];
    ldf<VEC>(c.a + i0, x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) bad |= !__builtin_isfinite(unscale(x[e], c.k));
  } else {
    for (uint64_t i = i0; i < c.n; ++i)
      bad |= !__builtin_isfinite(unscale(c.a[i], c.k));
  }
  flag_or(c.flag, bad);
}

struct AdamArgs {
  float *master, *m, *v;
  const float *a;
  uint64_t n;
  const uint32_t *flag;  /* may be null */
  Scales k;
  AdamK h;
};

template <int VEC>
__device__ __forceinline__ void adam_vec(const AdamArgs &p, uint64_t i0) {
  float th[VEC], m[VEC], v[VEC], a[VEC];
  ldf<VEC>(p.master + i0, th);
  ldf<VEC>(p.m + i0, m);
  ldf<VEC>(p.v + i0, v);
  ldf<VEC>(p.a + i0, a);
#pragma unroll
  for (int e = 0; e < VEC; ++e)
    th[e] = adamw_elem(th[e], m[e], v[e], unscale(a[e], p.k), p.h);
  stf<VEC>(p.master + i0, th);
  stf<VEC>(p.m + i0, m);
  stf<VEC>(p.v + i0, v);
}

template <int VEC>
__global__ __launch_bounds__(kBlock) void adamw_kernel(AdamArgs p) {
  if (p.flag && *p.flag) return;  /* overflow: the step is skipped */
  uint64_t i0 = first_elem(VEC);
  if (i0 >= p.n) return;
  if (i0 + VEC <= p.n) {
    adam_vec<VEC>(p, i0);
  } else {
    for (uint64_t i = i0; i < p.n; ++i) adam_vec<1>(p, i);
  }
}

struct CastArgs {
  const float *master;
  uint16_t *out;  /* already at this rank's offset */
  uint64_t n;
  const uint32_t *flag;
};

template <int VEC, int DT>
__global__ __launch_bounds__(kBlock) void cast_kernel(CastArgs c) {
  if (c.flag && *c.flag) return;
  uint64_t i0 = first_elem(VEC);
  if (i0 >= c.n) return;
  if (i0 + VEC <= c.n) {
    float x[VEC];
    ldf<VEC>(c.master + i0, x);
    st16<VEC, DT>(c.out + i0, x);
  } else {
    for (uint64_t i = i0; i < c.n; ++i) c.out[i] = pack1<DT>(c.master[i]);
  }
}

struct FusedArgs {
  GradPtrs g;
  uint32_t world;
  int wire;        /* ZS_WIRE_*: precision of the ring's partials */
  uint64_t n;
  const float *acc_in;  /* may be null */
  const float *master_in, *m_in, *v_in;
  float *master_out, *m_out, *v_out;
  uint16_t *param_out;  /* already at this rank's offset */
  uint32_t *flag;
  Scales k;
  AdamK h;
  zs_device_scaler *dev;  /* non-null: scale, bias corrections and epoch come from it */
  double lr;              /* for the bias correction formed on the device */
  /* write windows (rolling shape only; win_period 0: none): a wave stores
   * only while wall_clock64() % win_period >= win_open */
  uint32_t win_period, win_open;
};

/* Chip-wide write windows. Every wave of a launch reads the same
 * constant-rate wall clock (wall_clock64(), hipDeviceAttributeWallClockRate
 * ticks per second), so "the clock modulo a period lies in its last
 * window" is a time slot that all CUs agree on without communicating. A
 * wave that has its results waits for that slot before it stores, so the
 * memory sees mostly reads for the rest of each period and the writes of
 * the whole chip together in the window, instead of a thin stream of
 * writes mixed into the reads at all times (on MI355X those mixed writes
 * cost about three times their own bytes' time). Loads are never held.
 * The wait ends within one period; a wave that reaches the window while it
 * is open stores at once. Timing only: what is stored does not change. */
__device__ __forceinline__ void await_write_window(uint32_t period, uint32_t open_at) {
  __builtin_amdgcn_sched_barrier(0);
  while ((uint32_t)((uint64_t)wall_clock64() % period) < open_at) __builtin_amdgcn_s_sleep(2);
  __builtin_amdgcn_sched_barrier(0);
}

/* Grouped state layout: for each group of kGroup elements the master
 * weights, m and v are stored as three consecutive runs of kGroup floats,
 * so element e of the master weights is at float offset
 * 3 kGroup (e / kGroup) + e % kGroup, of m kGroup further and of v 2 kGroup
 * further. One wave's 4-element vectors still cover whole lines, and the
 * state is one stream in and one out instead of three each. */
constexpr uint64_t kGroup = 1024;

__device__ __forceinline__ uint64_t grouped_at(uint64_t e) {
  return (e / kGroup) * (3 * kGroup) + e % kGroup;
}

/* Offsets of element e's master weight, m and v from the state base:
 * e, and the separate m and v arrays (GR false), or the grouped layout. */
template <bool GR>
struct StateAt {
  uint64_t th, m, v;
  __device__ __forceinline__ explicit StateAt(uint64_t e) {
    if constexpr (GR) {
      th = grouped_at(e);
      m = th + kGroup;
      v = th + 2 * kGroup;
    } else {
      th = m = v = e;
    }
  }
};

template <int VEC, int GDT, int PDT, bool GR = false>
__device__ __forceinline__ bool fused_vec(const FusedArgs &p, const Scales &sk, const AdamK &h,
                                          uint64_t i0) {
  float th[VEC], m[VEC], v[VEC], acc[VEC], s[VEC];
  const StateAt<GR> at(i0);
  const float *m_in = GR ? p.master_in : p.m_in, *v_in = GR ? p.master_in : p.v_in;
  float *m_out = GR ? p.master_out : p.m_out, *v_out = GR ? p.master_out : p.v_out;
  ldf<VEC>(p.master_in + at.th, th);
  ldf<VEC>(m_in + at.m, m);
  ldf<VEC>(v_in + at.v, v);
  if (p.acc_in) ldf<VEC>(p.acc_in + i0, acc);
  ring_sum<VEC, GDT>(p.g, p.world, p.wire, i0, s);
  bool bad = false;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float a = average(s[e], sk);
    if (p.acc_in) a = acc[e] + a;
    float g = unscale(a, sk);
    bad |= !__builtin_isfinite(g);
    th[e] = adamw_elem(th[e], m[e], v[e], g, h);
  }
  stf<VEC>(p.master_out + at.th, th);
  stf<VEC>(m_out + at.m, m);
  stf<VEC>(v_out + at.v, v);
  st16<VEC, PDT>(p.param_out + i0, th);
  return bad;
}

/* One tile of U vectors per thread. MULTI (W > 1) loads the state after
 * the gradient sum: on MI355X that order streamed 5-10 % faster than
 * loading the state first, registers to spare or not; the rolling shape
 * issues the state loads with the last workers' loads. With a single worker
 * (W = 1) there is no sum, one gradient load, and the state loads go
 * first. SHAPE (kShape*) sets the sum's load batch and the store policy;
 * T is the block's thread count (vector u of thread t starts at
 * base + (u * T + t) * VEC). */
template <int VEC, int U, bool MULTI, bool ACC, int GDT, int PDT, int WIRE, int SHAPE,
          int T = kBlock, bool GR = false>
__device__ __forceinline__ bool fused_tile(const FusedArgs &p, const Scales &sk, const AdamK &h,
                                           uint64_t base) {
  constexpr int B = shape_batch(SHAPE);
  constexpr bool NTS = shape_nt_stores(SHAPE);
  constexpr bool NTL = shape_nt_loads(SHAPE);
  uint64_t i0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) i0[u] = base + ((uint64_t)u * T + threadIdx.x) * VEC;
  float th[U][VEC], m[U][VEC], v[U][VEC], acc[U][VEC], s[U][VEC];
  const float *m_in = GR ? p.master_in : p.m_in, *v_in = GR ? p.master_in : p.v_in;
  float *m_out = GR ? p.master_out : p.m_out, *v_out = GR ? p.master_out : p.v_out;
  auto load_state = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const StateAt<GR> at(i0[u]);  /* a vector never straddles a group */
      ldf_p<VEC, NTL>(p.master_in + at.th, th[u]);
      ldf_p<VEC, NTL>(m_in + at.m, m[u]);
      ldf_p<VEC, NTL>(v_in + at.v, v[u]);
      if constexpr (ACC) ldf_p<VEC, NTL>(p.acc_in + i0[u], acc[u]);
    }
  };
  if constexpr (MULTI && shape_rolling(SHAPE)) {
    ring_sum_roll<VEC, U, GDT, WIRE, B>(p.g, p.world, i0, s, load_state);
  } else if constexpr (MULTI) {
    ring_sum_uw<VEC, U, GDT, WIRE, B>(p.g, p.world, i0, s);
    load_state();
  } else {
    load_state();
    ring_sum_uw<VEC, U, GDT, WIRE, B>(p.g, 1, i0, s);  /* one worker: no loop runs */
  }
  bool bad = false;
  auto store = [&](int u) {
    const StateAt<GR> at(i0[u]);
    stf_p<VEC, NTS>(p.master_out + at.th, th[u]);
    stf_p<VEC, NTS>(m_out + at.m, m[u]);
    stf_p<VEC, NTS>(v_out + at.v, v[u]);
    st16_p<VEC, PDT, NTS>(p.param_out + i0[u], th[u]);
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float a = average(s[u][e], sk);
      if constexpr (ACC) a = acc[u][e] + a;
      float g = unscale(a, sk);
      bad |= !__builtin_isfinite(g);
      th[u][e] = adamw_elem(th[u][e], m[u][e], v[u][e], g, h);
    }
    if constexpr (!shape_rolling(SHAPE)) store(u);
  }
  if constexpr (shape_rolling(SHAPE)) {
    if (p.win_period) await_write_window(p.win_period, p.win_open);
#pragma unroll
    for (int u = 0; u < U; ++u) store(u);
  }
  return bad;
}

/* Step constants of the device-resident flow: the loss scale and the
 * bias corrections alpha = lr / (1 - beta1^t), bc2 = sqrt(1 - beta2^t)
 * formed in binary64 from the running powers and rounded once to fp32,
 * exactly as the host forms them for an explicit step_t, and the step's
 * epoch. Block 0 records the pair it used, counts a bad scale and records
 * the epoch (checked_epoch, which the commit compares with flag_epoch);
 * returns false for a scale that is not finite and > 0. */
__device__ __forceinline__ bool dev_step_consts(const FusedArgs &p, Scales &sk, AdamK &h,
                                                uint64_t &epoch) {
  zs_device_scaler *d = p.dev;
  const bool ok = dev_scales(d->scale, sk);
  const double b1t = d->beta1_t, b2t = d->beta2_t;
  const float alpha = (float)(p.lr / (1.0 - b1t));
  const float bc2 = (float)__builtin_sqrt(1.0 - b2t);
  h.alpha = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(alpha)));
  h.b2 = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(bc2)));
  epoch = d->epoch;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    d->last_alpha = h.alpha;
    d->last_bc2 = h.b2;
    d->checked_epoch = epoch;
    if (!ok) d->bad_scale = d->bad_scale + 1u;
  }
  return ok;
}

/* The device-resident flow's overflow mark: a wave that saw a non-finite
 * value stores the step's epoch + 1 (one lane; every such store of a step
 * writes the same value, so no read-modify-write is needed). */
__device__ __forceinline__ void flag_epoch_mark(uint64_t *flag_epoch, uint64_t value, bool bad) {
  unsigned long long m = __ballot(bad);
  if (m && bad && (threadIdx.x & 63u) == (unsigned)(__ffsll(m) - 1))
    __hip_atomic_store(flag_epoch, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

/* ACC: an accumulated fp32 gradient of earlier micro-batches (acc_in) is
 * added before the unscale; a separate instance so the common case carries
 * no registers for it. T threads per block, tiles of T * U * VEC elements,
 * and the ragged end in blocks of T elements. GR: the fp32 state in the
 * grouped layout (master_in / master_out hold it; m and v pointers unused). */
template <int VEC, int U, bool MULTI, bool ACC, int GDT, int PDT, int WIRE, int SHAPE,
          int T = kBlock, bool GR = false>
__global__ __launch_bounds__(T) void fused_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)T * U * VEC;
  const uint64_t full = p.n / tile;  /* blocks past `full` cover the tail */
  Scales sk = p.k;
  AdamK h = p.h;
  uint64_t epoch = 0;
  bool bad = p.dev ? !dev_step_consts(p, sk, h, epoch) : false;
  if (blockIdx.x < full) {
    bad |= fused_tile<VEC, U, MULTI, ACC, GDT, PDT, WIRE, SHAPE, T, GR>(p, sk, h,
                                                                        (uint64_t)blockIdx.x * tile);
  } else {
    /* ragged end: one element per thread, spread over enough blocks that
     * no thread walks a chain of them */
    uint64_t i = full * tile + (uint64_t)(blockIdx.x - full) * T + threadIdx.x;
    if (i < p.n) bad |= fused_vec<1, GDT, PDT, GR>(p, sk, h, i);
  }
  if (p.dev) flag_epoch_mark(&p.dev->flag_epoch, epoch + 1, bad);
  else flag_or(p.flag, bad);
}

}  // namespace zs

#endif /* ZS_KERNELS_H */
