/*
 * offload_cpu.cpp -- the ZeRO-Offload variant of the shard update: AdamW and
 * the 16-bit cast run on the host, where the optimizer states live, while
 * the GPU keeps the gradient reduction ([Intro] "并行训练框架DeepSpeed介绍",
 * 一.3 item (16): the update is cheap, so optimizer states and gradients move
 * to CPU memory; the forward/backward stay on the GPU).
 *
 * Same arithmetic as the device kernels, element for element: g = a / S,
 * m' = b1*m + c1*g, v' = b2*v + c2*(g*g), d = sqrt(v')/bc2 + eps,
 * master' = master*delta - alpha*(m'/d), params = RNE16(master'), every
 * operator one IEEE binary32 operation (built with -ffp-contract=off, so no
 * fused multiply-add), per-step scalars formed in double. The x86 vector
 * division and square root are correctly rounded; worker threads set MXCSR
 * to round-to-nearest with subnormals kept.
 */
#include <immintrin.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "zeroshard.h"

namespace {

struct Consts {
  float alpha, bc2, delta, c1, c2, beta1, beta2, eps, scale;
};

constexpr unsigned kMxcsrNearest = 0x1F80;  /* RNE, no FTZ/DAZ, all masked */

float adamw_one(float theta, float &m, float &v, float g, const Consts &k) {
  float decayed = theta * k.delta;
  float m1 = k.beta1 * m + k.c1 * g;
  float v1 = k.beta2 * v + k.c2 * (g * g);
  float d = sqrtf(v1) / k.bc2 + k.eps;
  float out = decayed - k.alpha * (m1 / d);
  m = m1;
  v = v1;
  return out;
}

uint16_t bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);  /* quiet NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t fp16_rne(float x) { return _cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT); }

__attribute__((target("avx512f,avx512bw"))) bool check_avx512(const float *a, uint64_t lo,
                                                                uint64_t hi, float scale) {
  const __m512 s = _mm512_set1_ps(scale);
  const __m512 inf = _mm512_set1_ps(INFINITY);
  uint64_t i = lo;
  for (; i + 16 <= hi; i += 16) {
    __m512 g = _mm512_div_ps(_mm512_loadu_ps(a + i), s);
    __m512 ag = _mm512_abs_ps(g);
    /* not finite <=> not (|g| < inf), NaN compares false */
    if (_mm512_cmp_ps_mask(ag, inf, _CMP_LT_OQ) != 0xffff) return true;
  }
  for (; i < hi; ++i)
    if (!isfinite(a[i] / scale)) return true;
  return false;
}

__attribute__((target("avx512f,avx512bw"))) void update_avx512(
    float *master, float *m, float *v, const float *a, uint64_t lo, uint64_t hi,
    const Consts &k, uint16_t *out, int dtype) {
  const __m512 s = _mm512_set1_ps(k.scale), delta = _mm512_set1_ps(k.delta);
  const __m512 b1 = _mm512_set1_ps(k.beta1), c1 = _mm512_set1_ps(k.c1);
  const __m512 b2 = _mm512_set1_ps(k.beta2), c2 = _mm512_set1_ps(k.c2);
  const __m512 bc2 = _mm512_set1_ps(k.bc2), eps = _mm512_set1_ps(k.eps);
  const __m512 alpha = _mm512_set1_ps(k.alpha);
  const __m512i round = _mm512_set1_epi32(0x7fff), one = _mm512_set1_epi32(1);
  const __m512i quiet = _mm512_set1_epi32(0x0040);
  uint64_t i = lo;
  for (; i + 16 <= hi; i += 16) {
    __m512 g = _mm512_div_ps(_mm512_loadu_ps(a + i), s);
    __m512 th = _mm512_loadu_ps(master + i);
    __m512 mm = _mm512_loadu_ps(m + i);
    __m512 vv = _mm512_loadu_ps(v + i);
    __m512 decayed = _mm512_mul_ps(th, delta);
    __m512 m1 = _mm512_add_ps(_mm512_mul_ps(b1, mm), _mm512_mul_ps(c1, g));
    __m512 v1 = _mm512_add_ps(_mm512_mul_ps(b2, vv), _mm512_mul_ps(c2, _mm512_mul_ps(g, g)));
    __m512 d = _mm512_add_ps(_mm512_div_ps(_mm512_sqrt_ps(v1), bc2), eps);
    __m512 th1 = _mm512_sub_ps(decayed, _mm512_mul_ps(alpha, _mm512_div_ps(m1, d)));
    _mm512_storeu_ps(master + i, th1);
    _mm512_storeu_ps(m + i, m1);
    _mm512_storeu_ps(v + i, v1);
    __m256i h;
    if (dtype == ZS_BF16) {
      __m512i u = _mm512_castps_si512(th1);
      __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(u, 16), one);
      __m512i r = _mm512_srli_epi32(_mm512_add_epi32(_mm512_add_epi32(u, round), lsb), 16);
      __mmask16 nan = _mm512_cmp_ps_mask(th1, th1, _CMP_UNORD_Q);
      r = _mm512_mask_or_epi32(r, nan, _mm512_srli_epi32(u, 16), quiet);
      h = _mm512_cvtepi32_epi16(r);
    } else {
      h = _mm512_cvtps_ph(th1, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    }
    _mm256_storeu_si256(reinterpret_cast<__m256i *>(out + i), h);
  }
  for (; i < hi; ++i) {
    float th1 = adamw_one(master[i], m[i], v[i], a[i] / k.scale, k);
    master[i] = th1;
    out[i] = dtype == ZS_BF16 ? bf16_rne(th1) : fp16_rne(th1);
  }
}

bool check_scalar(const float *a, uint64_t lo, uint64_t hi, float scale) {
  for (uint64_t i = lo; i < hi; ++i)
    if (!isfinite(a[i] / scale)) return true;
  return false;
}

void update_scalar(float *master, float *m, float *v, const float *a, uint64_t lo, uint64_t hi,
                   const Consts &k, uint16_t *out, int dtype) {
  for (uint64_t i = lo; i < hi; ++i) {
    float th1 = adamw_one(master[i], m[i], v[i], a[i] / k.scale, k);
    master[i] = th1;
    out[i] = dtype == ZS_BF16 ? bf16_rne(th1) : fp16_rne(th1);
  }
}

/* Runs fn(lo, hi) over `threads` contiguous ranges, each on a fresh thread
 * with MXCSR set to round-to-nearest, subnormals kept. */
template <typename F>
void parallel_ranges(uint64_t n, int threads, F fn) {
  std::vector<std::thread> pool;
  pool.reserve((size_t)threads);
  for (int t = 0; t < threads; ++t) {
    uint64_t lo = n * (uint64_t)t / (uint64_t)threads, hi = n * (uint64_t)(t + 1) / (uint64_t)threads;
    pool.emplace_back([=] {
      _mm_setcsr(kMxcsrNearest);
      fn(t, lo, hi);
    });
  }
  for (auto &th : pool) th.join();
}

}  // namespace

extern "C" int zs_cpu_step(float *master, float *m, float *v, const float *grad_part, uint64_t n,
                           const zs_adamw_hparams *hp, void *params16, int param_dtype,
                           int threads, uint32_t *overflow) {
  if (!master || !m || !v || !grad_part || !hp || !params16 || !overflow) return ZS_ERR_INVALID_ARG;
  if (param_dtype != ZS_BF16 && param_dtype != ZS_FP16) return ZS_ERR_INVALID_ARG;
  if (!(hp->loss_scale > 0.0f) || !isfinite(hp->loss_scale) || hp->step_t == 0)
    return ZS_ERR_INVALID_ARG;
  *overflow = 0;
  if (n == 0) return ZS_OK;
  Consts k;
  double b1 = hp->beta1, b2 = hp->beta2, lr = hp->lr, wd = hp->weight_decay;
  double b1t = 1.0, b2t = 1.0;
  for (uint32_t t = 0; t < hp->step_t; ++t) {
    b1t *= b1;
    b2t *= b2;
  }
  k.alpha = (float)(lr / (1.0 - b1t));
  k.bc2 = (float)sqrt(1.0 - b2t);
  k.delta = (float)(1.0 - lr * wd);
  k.c1 = (float)(1.0 - b1);
  k.c2 = (float)(1.0 - b2);
  k.beta1 = hp->beta1;
  k.beta2 = hp->beta2;
  k.eps = hp->eps;
  k.scale = hp->loss_scale;

  if (threads <= 0) threads = (int)std::min(64u, std::max(1u, std::thread::hardware_concurrency()));
  threads = (int)std::min<uint64_t>((uint64_t)threads, std::max<uint64_t>(1, n / 4096));
  const bool avx512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
  uint16_t *out = static_cast<uint16_t *>(params16);

  /* Pass 1: the overflow check over the whole partition (skip before
   * touching any state). */
  std::vector<char> bad((size_t)threads, 0);
  parallel_ranges(n, threads, [&](int t, uint64_t lo, uint64_t hi) {
    bad[(size_t)t] = avx512 ? check_avx512(grad_part, lo, hi, k.scale)
                            : check_scalar(grad_part, lo, hi, k.scale);
  });
  for (char b : bad)
    if (b) {
      *overflow = 1;
      return ZS_OK;
    }
  /* Pass 2: AdamW in place and the 16-bit parameters. */
  parallel_ranges(n, threads, [&](int, uint64_t lo, uint64_t hi) {
    if (avx512) update_avx512(master, m, v, grad_part, lo, hi, k, out, param_dtype);
    else update_scalar(master, m, v, grad_part, lo, hi, k, out, param_dtype);
  });
  return ZS_OK;
}
