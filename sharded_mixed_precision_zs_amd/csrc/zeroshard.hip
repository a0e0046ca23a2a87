/*
 * zeroshard.hip -- libzeroshard: the per-rank ZeRO-2 optimizer-shard step for
 * AMD Instinct MI355X (gfx950, CDNA4). The C ABI is declared and documented in
 * include/zeroshard.h; the sources it cites are listed there:
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
 *     with loads issued in batches ahead of the in-order adds;
 *   - the overflow flag is a wave ballot, one vector atomic OR per wave that
 *     saw a non-finite value;
 *   - 16-bit outputs use the hardware round-to-nearest-even converts
 *     (v_cvt_pk_bf16_f32, v_cvt_f16_f32);
 *   - built with -ffp-contract=off: every arithmetic operator is one IEEE
 *     binary32 operation; division and square root are the correctly rounded
 *     sequences, denormals are kept.
 */
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zeroshard.h"

namespace zs {

constexpr int kBlock = 256;     /* threads per workgroup (4 waves of 64)   */
constexpr int kLoadBatch = 8;   /* gradient vectors in flight per thread   */

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

/* ------------------------------------------------------------------------
 * Ring-order sum. g.p[j] is worker (rank + 1 + j) mod W, so summing
 * p[0], p[1], ..., p[W-1] left to right adds the owner's term last: the
 * order in which the ring's running partial for this chunk visits the
 * workers ([Notes] 二 three-GPU example; [L7] "Ring AllReduce 算法").
 * ---------------------------------------------------------------------- */

struct GradPtrs {
  const uint16_t *p[ZS_MAX_WORLD];
};

template <int VEC, int DT>
__device__ __forceinline__ void ring_sum(const GradPtrs &g, uint32_t world,
                                         uint64_t i0, float (&s)[VEC]) {
  upcast<VEC, DT>(ld16<VEC>(g.p[0] + i0), s);
  uint32_t j = 1;
  for (; j + kLoadBatch <= world; j += kLoadBatch) {
    Raw16<VEC> r[kLoadBatch];
#pragma unroll
    for (int b = 0; b < kLoadBatch; ++b) r[b] = ld16<VEC>(g.p[j + b] + i0);
#pragma unroll
    for (int b = 0; b < kLoadBatch; ++b) add_up<VEC, DT>(s, r[b]);
  }
  for (; j < world; ++j) add_up<VEC, DT>(s, ld16<VEC>(g.p[j] + i0));
}

/* The same ring-order sum for U vectors per thread. Loads are issued
 * worker-major (all U vectors of one worker back to back, kLoadBatch
 * workers ahead of the adds) and marked non-temporal. */
template <int VEC, int U, int DT>
__device__ __forceinline__ void ring_sum_u(const GradPtrs &g, uint32_t world,
                                           const uint64_t (&i0)[U],
                                           float (&s)[U][VEC]) {
#pragma unroll
  for (int u = 0; u < U; ++u) upcast<VEC, DT>(ld16<VEC, true>(g.p[0] + i0[u]), s[u]);
  uint32_t j = 1;
  for (; j + kLoadBatch <= world; j += kLoadBatch) {
    Raw16<VEC> r[kLoadBatch][U];
#pragma unroll
    for (int b = 0; b < kLoadBatch; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) r[b][u] = ld16<VEC, true>(g.p[j + b] + i0[u]);
#pragma unroll
    for (int b = 0; b < kLoadBatch; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) add_up<VEC, DT>(s[u], r[b][u]);
  }
  for (; j < world; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) add_up<VEC, DT>(s[u], ld16<VEC, true>(g.p[j] + i0[u]));
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
 * thread t in block b starts at ((b * U + u) * kBlock + t) * VEC, and only
 * the last block, when the tile overhangs n, walks its elements one by one.
 * ---------------------------------------------------------------------- */

constexpr int kTileVecs = 2;  /* U: vectors per thread in the reducing kernels */

__device__ __forceinline__ uint64_t first_elem(int vec) {
  return ((uint64_t)blockIdx.x * kBlock + threadIdx.x) * (uint64_t)vec;
}

struct ReduceArgs {
  GradPtrs g;
  uint32_t world;
  uint64_t n;
  float *out;
  uint32_t *flag;  /* may be null */
  int accumulate;
  Scales k;
};

template <int VEC, int DT>
__device__ __forceinline__ bool reduce_vec(const ReduceArgs &a, uint64_t i0) {
  float s[VEC], acc[VEC];
  if (a.accumulate) ldf<VEC>(a.out + i0, acc);
  ring_sum<VEC, DT>(a.g, a.world, i0, s);
  bool bad = false;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float v = average(s[e], a.k);
    if (a.accumulate) v = acc[e] + v;
    s[e] = v;
    bad |= !__builtin_isfinite(unscale(v, a.k));
  }
  stf<VEC>(a.out + i0, s);
  return bad;
}

template <int VEC, int U, int DT>
__device__ __forceinline__ bool reduce_tile(const ReduceArgs &a, uint64_t base) {
  uint64_t i0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) i0[u] = base + ((uint64_t)u * kBlock + threadIdx.x) * VEC;
  float s[U][VEC];
  ring_sum_u<VEC, U, DT>(a.g, a.world, i0, s);
  bool bad = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc[VEC];
    if (a.accumulate) ldf<VEC>(a.out + i0[u], acc);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float v = average(s[u][e], a.k);
      if (a.accumulate) v = acc[e] + v;
      s[u][e] = v;
      bad |= !__builtin_isfinite(unscale(v, a.k));
    }
    stf<VEC>(a.out + i0[u], s[u]);
  }
  return bad;
}

template <int VEC, int U, int DT>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceArgs a) {
  const uint64_t tile = (uint64_t)kBlock * U * VEC;
  const uint64_t base = (uint64_t)blockIdx.x * tile;
  bool bad = false;
  if (base + tile <= a.n) {
    bad = reduce_tile<VEC, U, DT>(a, base);
  } else {
    /* ragged last tile: element by element (one block; few registers) */
    for (int u = 0; u < U; ++u) {
      uint64_t i0 = base + ((uint64_t)u * kBlock + threadIdx.x) * VEC;
      for (uint64_t i = i0; i < i0 + VEC && i < a.n; ++i) bad |= reduce_vec<1, DT>(a, i);
    }
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
  uint64_t n;
  const float *acc_in;  /* may be null */
  const float *master_in, *m_in, *v_in;
  float *master_out, *m_out, *v_out;
  uint16_t *param_out;  /* already at this rank's offset */
  uint32_t *flag;
  Scales k;
  AdamK h;
};

template <int VEC, int GDT, int PDT>
__device__ __forceinline__ bool fused_vec(const FusedArgs &p, uint64_t i0) {
  float th[VEC], m[VEC], v[VEC], acc[VEC], s[VEC];
  ldf<VEC>(p.master_in + i0, th);
  ldf<VEC>(p.m_in + i0, m);
  ldf<VEC>(p.v_in + i0, v);
  if (p.acc_in) ldf<VEC>(p.acc_in + i0, acc);
  ring_sum<VEC, GDT>(p.g, p.world, i0, s);
  bool bad = false;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float a = average(s[e], p.k);
    if (p.acc_in) a = acc[e] + a;
    float g = unscale(a, p.k);
    bad |= !__builtin_isfinite(g);
    th[e] = adamw_elem(th[e], m[e], v[e], g, p.h);
  }
  stf<VEC>(p.master_out + i0, th);
  stf<VEC>(p.m_out + i0, m);
  stf<VEC>(p.v_out + i0, v);
  st16<VEC, PDT>(p.param_out + i0, th);
  return bad;
}

/* One tile of U vectors per thread. MULTI (W > 1) loads the state after
 * the gradient sum, which keeps registers (and so waves in flight) for the
 * gradient streams; with a single worker (W = 1) there is no sum, one
 * gradient load, and the state loads go first. */
template <int VEC, int U, bool MULTI, bool ACC, int GDT, int PDT>
__device__ __forceinline__ bool fused_tile(const FusedArgs &p, uint64_t base) {
  uint64_t i0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) i0[u] = base + ((uint64_t)u * kBlock + threadIdx.x) * VEC;
  float th[U][VEC], m[U][VEC], v[U][VEC], acc[U][VEC], s[U][VEC];
  auto load_state = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ldf<VEC>(p.master_in + i0[u], th[u]);
      ldf<VEC>(p.m_in + i0[u], m[u]);
      ldf<VEC>(p.v_in + i0[u], v[u]);
      if constexpr (ACC) ldf<VEC>(p.acc_in + i0[u], acc[u]);
    }
  };
  if constexpr (MULTI) {
    ring_sum_u<VEC, U, GDT>(p.g, p.world, i0, s);
    load_state();
  } else {
    load_state();
#pragma unroll
    for (int u = 0; u < U; ++u) upcast<VEC, GDT>(ld16<VEC, true>(p.g.p[0] + i0[u]), s[u]);
  }
  bool bad = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float a = average(s[u][e], p.k);
      if constexpr (ACC) a = acc[u][e] + a;
      float g = unscale(a, p.k);
      bad |= !__builtin_isfinite(g);
      th[u][e] = adamw_elem(th[u][e], m[u][e], v[u][e], g, p.h);
    }
    stf<VEC>(p.master_out + i0[u], th[u]);
    stf<VEC>(p.m_out + i0[u], m[u]);
    stf<VEC>(p.v_out + i0[u], v[u]);
    st16<VEC, PDT>(p.param_out + i0[u], th[u]);
  }
  return bad;
}

/* ACC: an accumulated fp32 gradient of earlier micro-batches (acc_in) is
 * added before the unscale; a separate instance so the common case carries
 * no registers for it. */
template <int VEC, int U, bool MULTI, bool ACC, int GDT, int PDT>
__global__ __launch_bounds__(kBlock) void fused_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)kBlock * U * VEC;
  const uint64_t base = (uint64_t)blockIdx.x * tile;
  bool bad = false;
  if (base + tile <= p.n) {
    bad = fused_tile<VEC, U, MULTI, ACC, GDT, PDT>(p, base);
  } else {
    /* ragged last tile: element by element (one block; few registers) */
    for (int u = 0; u < U; ++u) {
      uint64_t i0 = base + ((uint64_t)u * kBlock + threadIdx.x) * VEC;
      for (uint64_t i = i0; i < i0 + VEC && i < p.n; ++i) bad |= fused_vec<1, GDT, PDT>(p, i);
    }
  }
  flag_or(p.flag, bad);
}

}  // namespace zs

namespace {

using namespace zs;

/* ------------------------------------------------------------------------
 * Host side: validation, scalar preparation, launch.
 * ---------------------------------------------------------------------- */

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, const char *detail = "") {
  snprintf(g_err, sizeof g_err, fmt, detail);
  return status;
}

int launch_result() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return ZS_OK;
}

bool valid_dtype(int dt) { return dt == ZS_BF16 || dt == ZS_FP16; }

/* Exact power of two with a normal reciprocal: then x * (1/p) == x / p. */
bool exact_pow2(float p, float *inv) {
  if (!(p > 0.0f) || !isfinite(p)) return false;
  int e;
  float m = frexpf(p, &e);         /* p = m * 2^e, m in [0.5, 1) */
  if (m != 0.5f) return false;
  int k = e - 1;                   /* p = 2^k */
  if (k < -126 || k > 126) return false;
  *inv = ldexpf(1.0f, -k);
  return true;
}

bool make_scales(uint32_t world, float loss_scale, Scales *k) {
  if (!(loss_scale > 0.0f) || !isfinite(loss_scale)) return false;
  k->wf = (float)world;
  k->w_pow2 = exact_pow2(k->wf, &k->inv_w) ? 1 : 0;
  if (!k->w_pow2) k->inv_w = 0.0f;
  k->sf = loss_scale;
  k->s_pow2 = exact_pow2(loss_scale, &k->inv_s) ? 1 : 0;
  if (!k->s_pow2) k->inv_s = 0.0f;
  return true;
}

/* Per-step scalars in double, rounded once to fp32. beta^t is formed by t
 * repeated multiplications. */
bool make_adam(const zs_adamw_hparams *hp, AdamK *k) {
  if (hp->step_t == 0) return false;
  double b1 = hp->beta1, b2 = hp->beta2, lr = hp->lr, wd = hp->weight_decay;
  double b1t = 1.0, b2t = 1.0;
  for (uint32_t t = 0; t < hp->step_t; ++t) {
    b1t *= b1;
    b2t *= b2;
  }
  k->alpha = (float)(lr / (1.0 - b1t));
  k->b2 = (float)sqrt(1.0 - b2t);
  k->delta = (float)(1.0 - lr * wd);
  k->c1 = (float)(1.0 - b1);
  k->c2 = (float)(1.0 - b2);
  k->beta1 = hp->beta1;
  k->beta2 = hp->beta2;
  k->eps = hp->eps;
  return true;
}

/* Widest vector width every operand's alignment allows: 16-bit operands
 * need 2*VEC bytes, fp32 operands min(16, 4*VEC) bytes. */
int pick_vec(const void *const *p16, int n16, const void *const *p32, int n32) {
  for (int vec = 8; vec > 1; vec /= 2) {
    bool ok = true;
    for (int i = 0; i < n16 && ok; ++i)
      ok = ((uintptr_t)p16[i] % (uintptr_t)(2 * vec)) == 0;
    uintptr_t a32 = (uintptr_t)(4 * vec < 16 ? 4 * vec : 16);
    for (int i = 0; i < n32 && ok; ++i) ok = ((uintptr_t)p32[i] % a32) == 0;
    if (ok) return vec;
  }
  return 1;
}

/* Blocks for n elements when every thread covers `per_thread` of them. */
unsigned grid_for(uint64_t n, int per_thread) {
  uint64_t per_block = (uint64_t)kBlock * (uint64_t)per_thread;
  return (unsigned)((n + per_block - 1) / per_block);
}

bool grid_ok(uint64_t n, int per_thread) {
  uint64_t per_block = (uint64_t)kBlock * (uint64_t)per_thread;
  return (n + per_block - 1) / per_block <= 0x7fffffffull;
}

int fill_ring(const void *const *worker_grads, uint32_t world, uint32_t rank,
              GradPtrs *g) {
  for (uint32_t j = 0; j < world; ++j) {
    const void *p = worker_grads[(rank + 1 + j) % world];
    if (!p) return fail(ZS_ERR_INVALID_ARG, "worker_grads has a null pointer%s");
    g->p[j] = static_cast<const uint16_t *>(p);
  }
  for (uint32_t j = world; j < ZS_MAX_WORLD; ++j) g->p[j] = nullptr;
  return ZS_OK;
}

bool overlaps(const void *a, uint64_t abytes, const void *b, uint64_t bbytes) {
  if (!a || !b || !abytes || !bbytes) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

}  // namespace

/* ========================================================================
 * C ABI
 * ====================================================================== */

extern "C" {

int zs_abi_version(void) { return ZS_ABI_VERSION; }

const char *zs_status_string(int status) {
  switch (status) {
    case ZS_OK: return "ZS_OK";
    case ZS_ERR_INVALID_ARG: return "ZS_ERR_INVALID_ARG";
    case ZS_ERR_UNSUPPORTED: return "ZS_ERR_UNSUPPORTED";
    case ZS_ERR_ALIAS: return "ZS_ERR_ALIAS";
    case ZS_ERR_HIP: return "ZS_ERR_HIP";
    default: return "ZS_UNKNOWN_STATUS";
  }
}

const char *zs_last_error(void) { return g_err; }

int zs_partition(uint64_t phi, uint32_t world, uint32_t rank, uint64_t *chunk,
                 uint64_t *offset, uint64_t *count) {
  if (world == 0 || rank >= world)
    return fail(ZS_ERR_INVALID_ARG, "partition needs 0 <= rank < world, world > 0%s");
  uint64_t p = phi / world + (phi % world != 0);
  uint64_t off = (uint64_t)rank * p;
  uint64_t cnt = off < phi ? (phi - off < p ? phi - off : p) : 0;
  if (chunk) *chunk = p;
  if (offset) *offset = off;
  if (count) *count = cnt;
  g_err[0] = 0;
  return ZS_OK;
}

int zs_reduce_scatter_avg(const void *const *worker_grads, int grad_dtype,
                          uint32_t world, uint32_t rank, uint64_t n,
                          float *grad_part, int accumulate,
                          uint32_t *overflow_flag, float loss_scale,
                          void *stream) {
  if (!worker_grads || !grad_part)
    return fail(ZS_ERR_INVALID_ARG, "null worker_grads or grad_part%s");
  if (world == 0 || world > ZS_MAX_WORLD || rank >= world)
    return fail(ZS_ERR_INVALID_ARG, "need 0 < world <= 64 and rank < world%s");
  if (!valid_dtype(grad_dtype)) return fail(ZS_ERR_INVALID_ARG, "bad grad dtype%s");
  ReduceArgs a;
  if (!make_scales(world, loss_scale, &a.k))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (n == 0) return ZS_OK;
  int rc = fill_ring(worker_grads, world, rank, &a.g);
  if (rc != ZS_OK) return rc;
  a.world = world;
  a.n = n;
  a.out = grad_part;
  a.flag = overflow_flag;
  a.accumulate = accumulate ? 1 : 0;
  const void *f32[] = {grad_part};
  int vec = pick_vec(reinterpret_cast<const void *const *>(a.g.p), (int)world, f32, 1);
  const int per_thread = vec * kTileVecs;
  if (!grid_ok(n, per_thread)) return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(grid_for(n, per_thread)), block(kBlock);
#define ZS_LAUNCH_REDUCE(V, D) \
  hipLaunchKernelGGL((reduce_kernel<V, kTileVecs, D>), grid, block, 0, s, a)
  if (grad_dtype == ZS_BF16) {
    switch (vec) {
      case 8: ZS_LAUNCH_REDUCE(8, ZS_BF16); break;
      case 4: ZS_LAUNCH_REDUCE(4, ZS_BF16); break;
      case 2: ZS_LAUNCH_REDUCE(2, ZS_BF16); break;
      default: ZS_LAUNCH_REDUCE(1, ZS_BF16); break;
    }
  } else {
    switch (vec) {
      case 8: ZS_LAUNCH_REDUCE(8, ZS_FP16); break;
      case 4: ZS_LAUNCH_REDUCE(4, ZS_FP16); break;
      case 2: ZS_LAUNCH_REDUCE(2, ZS_FP16); break;
      default: ZS_LAUNCH_REDUCE(1, ZS_FP16); break;
    }
  }
#undef ZS_LAUNCH_REDUCE
  return launch_result();
}

int zs_check_overflow(const float *grad_part, uint64_t n, float loss_scale,
                      uint32_t *overflow_flag, void *stream) {
  if (!grad_part || !overflow_flag)
    return fail(ZS_ERR_INVALID_ARG, "null grad_part or overflow_flag%s");
  CheckArgs c;
  if (!make_scales(1, loss_scale, &c.k))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (n == 0) return ZS_OK;
  c.a = grad_part;
  c.n = n;
  c.flag = overflow_flag;
  const void *f32[] = {grad_part};
  int vec = pick_vec(nullptr, 0, f32, 1);
  if (!grid_ok(n, vec)) return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(grid_for(n, vec)), block(kBlock);
  switch (vec) {
    case 8: hipLaunchKernelGGL(check_kernel<8>, grid, block, 0, s, c); break;
    case 4: hipLaunchKernelGGL(check_kernel<4>, grid, block, 0, s, c); break;
    case 2: hipLaunchKernelGGL(check_kernel<2>, grid, block, 0, s, c); break;
    default: hipLaunchKernelGGL(check_kernel<1>, grid, block, 0, s, c); break;
  }
  return launch_result();
}

int zs_adamw_step(float *master, float *m, float *v, const float *grad_part,
                  uint64_t n, const zs_adamw_hparams *hp,
                  const uint32_t *overflow_flag, void *stream) {
  if (!master || !m || !v || !grad_part || !hp)
    return fail(ZS_ERR_INVALID_ARG, "null master, m, v, grad_part or hparams%s");
  AdamArgs p;
  if (!make_scales(1, hp->loss_scale, &p.k))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (!make_adam(hp, &p.h)) return fail(ZS_ERR_INVALID_ARG, "step_t must be >= 1%s");
  if (n == 0) return ZS_OK;
  p.master = master;
  p.m = m;
  p.v = v;
  p.a = grad_part;
  p.n = n;
  p.flag = overflow_flag;
  const void *f32[] = {master, m, v, grad_part};
  int vec = pick_vec(nullptr, 0, f32, 4);
  if (!grid_ok(n, vec)) return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(grid_for(n, vec)), block(kBlock);
  switch (vec) {
    case 8: hipLaunchKernelGGL(adamw_kernel<8>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(adamw_kernel<4>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(adamw_kernel<2>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(adamw_kernel<1>, grid, block, 0, s, p); break;
  }
  return launch_result();
}

int zs_cast_gather(const float *master, void *gather_buf, int param_dtype,
                   uint64_t offset, uint64_t n, const uint32_t *overflow_flag,
                   void *stream) {
  if (!master || !gather_buf)
    return fail(ZS_ERR_INVALID_ARG, "null master or gather_buf%s");
  if (!valid_dtype(param_dtype)) return fail(ZS_ERR_INVALID_ARG, "bad param dtype%s");
  if (n == 0) return ZS_OK;
  CastArgs c;
  c.master = master;
  c.out = static_cast<uint16_t *>(gather_buf) + offset;
  c.n = n;
  c.flag = overflow_flag;
  const void *p16[] = {c.out};
  const void *f32[] = {master};
  int vec = pick_vec(p16, 1, f32, 1);
  if (!grid_ok(n, vec)) return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(grid_for(n, vec)), block(kBlock);
#define ZS_LAUNCH_CAST(V, D) hipLaunchKernelGGL((cast_kernel<V, D>), grid, block, 0, s, c)
  if (param_dtype == ZS_BF16) {
    switch (vec) {
      case 8: ZS_LAUNCH_CAST(8, ZS_BF16); break;
      case 4: ZS_LAUNCH_CAST(4, ZS_BF16); break;
      case 2: ZS_LAUNCH_CAST(2, ZS_BF16); break;
      default: ZS_LAUNCH_CAST(1, ZS_BF16); break;
    }
  } else {
    switch (vec) {
      case 8: ZS_LAUNCH_CAST(8, ZS_FP16); break;
      case 4: ZS_LAUNCH_CAST(4, ZS_FP16); break;
      case 2: ZS_LAUNCH_CAST(2, ZS_FP16); break;
      default: ZS_LAUNCH_CAST(1, ZS_FP16); break;
    }
  }
#undef ZS_LAUNCH_CAST
  return launch_result();
}

int zs_step_fused(const zs_step_args *a, void *stream) {
  if (!a) return fail(ZS_ERR_INVALID_ARG, "null args%s");
  if (!a->worker_grads || !a->master_in || !a->m_in || !a->v_in || !a->master_out ||
      !a->m_out || !a->v_out || !a->gather_buf || !a->overflow_flag)
    return fail(ZS_ERR_INVALID_ARG, "null pointer in zs_step_args%s");
  if (a->world == 0 || a->world > ZS_MAX_WORLD || a->rank >= a->world)
    return fail(ZS_ERR_INVALID_ARG, "need 0 < world <= 64 and rank < world%s");
  if (!valid_dtype(a->grad_dtype) || !valid_dtype(a->param_dtype))
    return fail(ZS_ERR_INVALID_ARG, "bad grad or param dtype%s");
  FusedArgs p;
  if (!make_scales(a->world, a->hp.loss_scale, &p.k))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (!make_adam(&a->hp, &p.h)) return fail(ZS_ERR_INVALID_ARG, "step_t must be >= 1%s");
  const uint64_t n = a->n;
  if (n == 0) return ZS_OK;
  int rc = fill_ring(a->worker_grads, a->world, a->rank, &p.g);
  if (rc != ZS_OK) return rc;

  uint16_t *param_out = static_cast<uint16_t *>(a->gather_buf) + a->gather_offset;
  /* The output set must not overlap any input (the skip relies on the
   * input set being untouched) nor itself. */
  const uint64_t b4 = 4 * n, b2 = 2 * n;
  const void *outs[] = {a->master_out, a->m_out, a->v_out, param_out};
  const uint64_t out_bytes[] = {b4, b4, b4, b2};
  const void *ins[] = {a->master_in, a->m_in, a->v_in, a->acc_in};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], b4))
        return fail(ZS_ERR_ALIAS, "zs_step_fused: an output overlaps an input%s");
    for (uint32_t w = 0; w < a->world; ++w)
      if (overlaps(outs[i], out_bytes[i], p.g.p[w], b2))
        return fail(ZS_ERR_ALIAS, "zs_step_fused: an output overlaps a gradient buffer%s");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return fail(ZS_ERR_ALIAS, "zs_step_fused: two outputs overlap%s");
  }

  p.world = a->world;
  p.n = n;
  p.acc_in = a->acc_in;
  p.master_in = a->master_in;
  p.m_in = a->m_in;
  p.v_in = a->v_in;
  p.master_out = a->master_out;
  p.m_out = a->m_out;
  p.v_out = a->v_out;
  p.param_out = param_out;
  p.flag = a->overflow_flag;

  const void *p16[ZS_MAX_WORLD + 1];
  for (uint32_t w = 0; w < a->world; ++w) p16[w] = p.g.p[w];
  p16[a->world] = param_out;
  const void *f32[] = {a->master_in, a->m_in, a->v_in, a->master_out, a->m_out,
                       a->v_out, a->acc_in ? a->acc_in : a->master_in};
  int vec = pick_vec(p16, (int)a->world + 1, f32, 7);
  const int per_thread = vec * kTileVecs;
  if (!grid_ok(n, per_thread)) return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(grid_for(n, per_thread)), block(kBlock);
  const int mode = (a->world > 1 ? 1 : 0) | (a->acc_in ? 2 : 0);
#define ZS_FUSED_K(V, L, A, G, P) \
  hipLaunchKernelGGL((fused_kernel<V, kTileVecs, L, A, G, P>), grid, block, 0, s, p)
#define ZS_LAUNCH_FUSED(V, G, P)                          \
  do {                                                    \
    switch (mode) {                                       \
      case 0: ZS_FUSED_K(V, false, false, G, P); break;   \
      case 1: ZS_FUSED_K(V, true, false, G, P); break;    \
      case 2: ZS_FUSED_K(V, false, true, G, P); break;    \
      default: ZS_FUSED_K(V, true, true, G, P); break;    \
    }                                                     \
  } while (0)
#define ZS_FUSED_VEC(G, P)                  \
  switch (vec) {                            \
    case 8: ZS_LAUNCH_FUSED(8, G, P); break; \
    case 4: ZS_LAUNCH_FUSED(4, G, P); break; \
    case 2: ZS_LAUNCH_FUSED(2, G, P); break; \
    default: ZS_LAUNCH_FUSED(1, G, P); break; \
  }
  if (a->grad_dtype == ZS_BF16 && a->param_dtype == ZS_BF16) {
    ZS_FUSED_VEC(ZS_BF16, ZS_BF16)
  } else if (a->grad_dtype == ZS_FP16 && a->param_dtype == ZS_FP16) {
    ZS_FUSED_VEC(ZS_FP16, ZS_FP16)
  } else if (a->grad_dtype == ZS_BF16) {
    ZS_FUSED_VEC(ZS_BF16, ZS_FP16)
  } else {
    ZS_FUSED_VEC(ZS_FP16, ZS_BF16)
  }
#undef ZS_FUSED_VEC
#undef ZS_LAUNCH_FUSED
#undef ZS_FUSED_K
  return launch_result();
}

int zs_scaler_update(zs_loss_scaler *s, uint32_t overflow) {
  if (!s) return fail(ZS_ERR_INVALID_ARG, "null scaler%s");
  if (overflow) {
    if (s->dynamic) s->scale = s->scale * 0.5f;
    s->clean_steps = 0;
    s->skipped += 1;
  } else {
    s->step_t += 1;
    s->clean_steps += 1;
    if (s->dynamic && s->growth_interval && s->clean_steps >= s->growth_interval) {
      s->scale = s->scale * 2.0f;
      s->clean_steps = 0;
    }
  }
  g_err[0] = 0;
  return ZS_OK;
}

}  // extern "C"
