/*
 * zs_oracle.c -- plain CPU oracle of the per-rank ZeRO-2 optimizer-shard step.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE (see zs_oracle.h for the sources,
 * the precision rules and the readings). Built with gcc -O2 -std=c11
 * -ffp-contract=off and no fast-math, so every float expression below is one
 * binary32 operation per operator, rounded to nearest-even, in source order.
 */
#include "zs_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

static uint32_t bits_of(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

static float float_of(uint32_t u) {
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

int zso_fp_env_ok(void) {
  volatile float tiny = 1.0e-38f, k = 1.0e-3f;  /* product is subnormal      */
  volatile float one = 1.0f, eps = 5.9604645e-8f; /* 2^-24: a tie at 1.0     */
  float sub = tiny * k;
  float tie = one + eps;                          /* RNE keeps 1.0           */
  return sub != 0.0f && tie == 1.0f;
}

/* ---- partition ([Notes] 二; [L7] "Ring AllReduce 算法") ------------------- */

int zso_partition(uint64_t phi, uint32_t world, uint32_t rank,
                  uint64_t *chunk, uint64_t *offset, uint64_t *count) {
  if (world == 0 || rank >= world) return -1;
  uint64_t p = phi / world + (phi % world != 0);
  uint64_t off = (uint64_t)rank * p;
  uint64_t cnt = 0;
  if (off < phi) cnt = (phi - off < p) ? phi - off : p;
  if (chunk) *chunk = p;
  if (offset) *offset = off;
  if (count) *count = cnt;
  return 0;
}

/* ---- 16-bit formats ([Intro] 一.3 item (2): BF16 keeps FP32's exponent
 * range with a 7-bit fraction; FP16 has a 10-bit fraction) --------------- */

float zso_half_to_float(uint16_t h, int dtype) {
  if (dtype == ZSO_BF16) return float_of((uint32_t)h << 16);
  /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  float mag;
  if (e == 0)
    mag = ldexpf((float)f, -24);            /* zero or subnormal: f * 2^-24 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexpf((float)(1024 + f), e - 25); /* (1.f) * 2^(e-15)           */
  return sign ? -mag : mag;
}

/* Round-to-nearest-even of a non-negative integer m shifted right by sh. */
static uint32_t rne_shift(uint32_t m, int sh) {
  if (sh <= 0) return m;
  if (sh > 31) return 0;
  uint32_t q = m >> sh;
  uint32_t rem = m & ((1u << sh) - 1u);
  uint32_t half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  return q;
}

uint16_t zso_float_to_half(float x, int dtype) {
  uint32_t u = bits_of(x);
  uint32_t sign = u >> 31;
  uint32_t mag = u & 0x7fffffffu;
  int e_field = (int)(mag >> 23);
  uint32_t frac = mag & 0x7fffffu;

  if (dtype == ZSO_BF16) {
    /* Keep the top 16 bits, rounding the dropped 16 to nearest-even.    */
    if (e_field == 255 && frac) return (uint16_t)((sign << 15) | 0x7fc0u);
    if (e_field == 255) return (uint16_t)((sign << 15) | 0x7f80u);
    uint32_t q = rne_shift(mag, 16);        /* carries into the exponent, */
    return (uint16_t)((sign << 15) | q);    /* and to inf past bf16 max   */
  }

  /* binary16 */
  if (e_field == 255)
    return (uint16_t)((sign << 15) | (frac ? 0x7e00u : 0x7c00u));
  if (e_field == 0) return (uint16_t)(sign << 15); /* |x| < 2^-126 -> 0     */
  int e = e_field - 127;                     /* x = M * 2^(e-23)           */
  uint32_t m24 = frac | 0x800000u;
  int e_eff = e < -14 ? -14 : e;             /* binary16 subnormal floor   */
  int sh = 13 + (e_eff - e);                 /* quantum 2^(e_eff-10)       */
  uint32_t q = rne_shift(m24, sh);           /* q in [0, 2048]             */
  /* Normal: bits = (e+15)<<10 | (q-1024); subnormal: bits = q. Both equal
   * ((e_eff+14)<<10) + q, and q == 2048 / q == 1024 carry correctly.     */
  uint32_t b = ((uint32_t)(e_eff + 14) << 10) + q;
  if (b >= 0x7c00u) b = 0x7c00u;             /* overflow -> inf            */
  return (uint16_t)((sign << 15) | b);
}

void zso_halves_to_floats(const uint16_t *in, float *out, uint64_t n,
                          int dtype) {
  for (uint64_t i = 0; i < n; ++i) out[i] = zso_half_to_float(in[i], dtype);
}

void zso_floats_to_halves(const float *in, uint16_t *out, uint64_t n,
                          int dtype) {
  for (uint64_t i = 0; i < n; ++i) out[i] = zso_float_to_half(in[i], dtype);
}

/* ---- ring all-reduce, simulated rank by rank ----------------------------
 * [Notes] 二: three GPUs each hold the gradients of A, B, C; in every step
 * each GPU passes one chunk (or running partial sum) to its successor,
 * which adds its own value; after W-1 steps each GPU holds one chunk's
 * total (scatter-reduce), and W-1 more steps circulate the totals
 * (all-gather). [L7] "Ring AllReduce 算法" states the same in general W. */

static uint32_t mod_w(int64_t x, uint32_t w) {
  int64_t r = x % (int64_t)w;
  return (uint32_t)(r < 0 ? r + w : r);
}

int zso_ring_reduce_scatter(uint32_t world, uint64_t chunk_len, int sigma,
                            uint32_t steps, float *bufs) {
  if (world == 0 || steps >= world) return -1;
  uint64_t row = (uint64_t)world * chunk_len;
  float *msg = (float *)malloc(sizeof(float) * (row ? row : 1));
  if (!msg) return -1;
  for (uint32_t s = 1; s <= steps; ++s) {
    /* Everyone sends at once: snapshot all outgoing chunks first. */
    for (uint32_t k = 0; k < world; ++k) {
      uint32_t c = mod_w((int64_t)k - s + sigma, world);
      memcpy(msg + k * chunk_len, bufs + k * row + c * chunk_len,
             sizeof(float) * chunk_len);
    }
    for (uint32_t k = 0; k < world; ++k) {
      uint32_t dst = (k + 1) % world;
      uint32_t c = mod_w((int64_t)k - s + sigma, world);
      float *own = bufs + dst * row + c * chunk_len;
      const float *in = msg + k * chunk_len;
      for (uint64_t i = 0; i < chunk_len; ++i) own[i] = in[i] + own[i];
    }
  }
  free(msg);
  return 0;
}

int zso_ring_all_gather(uint32_t world, uint64_t chunk_len, int sigma,
                        uint32_t steps, float *bufs) {
  if (world == 0 || steps >= world) return -1;
  uint64_t row = (uint64_t)world * chunk_len;
  float *msg = (float *)malloc(sizeof(float) * (row ? row : 1));
  if (!msg) return -1;
  for (uint32_t s = 1; s <= steps; ++s) {
    for (uint32_t k = 0; k < world; ++k) {
      uint32_t c = mod_w((int64_t)k + sigma - s + 1, world);
      memcpy(msg + k * chunk_len, bufs + k * row + c * chunk_len,
             sizeof(float) * chunk_len);
    }
    for (uint32_t k = 0; k < world; ++k) {
      uint32_t dst = (k + 1) % world;
      uint32_t c = mod_w((int64_t)k + sigma - s + 1, world);
      memcpy(bufs + dst * row + c * chunk_len, msg + k * chunk_len,
             sizeof(float) * chunk_len);
    }
  }
  free(msg);
  return 0;
}

uint32_t zso_ring_held_chunk(uint32_t world, uint32_t rank, int sigma) {
  return mod_w((int64_t)rank + sigma, world);
}

void zso_ring_chunk_sum(uint32_t world, uint32_t rank,
                        const uint16_t *const *part, int dtype, uint64_t n,
                        float *sum_out) {
  for (uint64_t i = 0; i < n; ++i) {
    /* The partial starts at the owner's successor and travels the ring;
     * every rank it reaches adds its own value, the owner last. */
    float acc = zso_half_to_float(part[(rank + 1) % world][i], dtype);
    for (uint32_t s = 2; s <= world; ++s)
      acc = acc + zso_half_to_float(part[(rank + s) % world][i], dtype);
    sum_out[i] = acc;
  }
}

/* What a 16-bit wire does to a partial sum: round it to the wire type. */
static float on_wire(float x, int wire) {
  if (wire == ZSO_WIRE_BF16) return zso_half_to_float(zso_float_to_half(x, ZSO_BF16), ZSO_BF16);
  if (wire == ZSO_WIRE_FP16) return zso_half_to_float(zso_float_to_half(x, ZSO_FP16), ZSO_FP16);
  return x;
}

/* One element of the journey, partials carried in `wire` precision. */
static float ring_elem(uint32_t world, uint32_t rank, const uint16_t *const *part,
                       int dtype, int wire, uint64_t i) {
  float acc = on_wire(zso_half_to_float(part[(rank + 1) % world][i], dtype), wire);
  for (uint32_t s = 2; s <= world; ++s)
    acc = on_wire(acc + zso_half_to_float(part[(rank + s) % world][i], dtype), wire);
  return acc;
}

void zso_ring_chunk_sum_wire(uint32_t world, uint32_t rank,
                             const uint16_t *const *part, int dtype, int wire,
                             uint64_t n, float *sum_out) {
  for (uint64_t i = 0; i < n; ++i) sum_out[i] = ring_elem(world, rank, part, dtype, wire, i);
}

/* ---- owner's average, accumulation and overflow check --------------------
 * [Notes] 三 and 四: the owner gathers the W contributions of its part and
 * takes their mean; [L7] "数学等价性": the mean of the W worker gradients
 * is the full-batch gradient. [L7] "Gradient Accumulation": micro-batch
 * gradients are summed before the single update. */

uint32_t zso_reduce_avg_wire(uint32_t world, uint32_t rank,
                             const uint16_t *const *part, int dtype, int wire,
                             uint64_t n, float *out, int accumulate,
                             float loss_scale) {
  uint32_t flag = 0;
  const float wf = (float)world;
  for (uint64_t i = 0; i < n; ++i) {
    float a = ring_elem(world, rank, part, dtype, wire, i) / wf;
    if (accumulate) a = out[i] + a;
    out[i] = a;
    float g = a / loss_scale;
    if (!isfinite(g)) flag = 1;
  }
  return flag;
}

uint32_t zso_reduce_avg(uint32_t world, uint32_t rank,
                        const uint16_t *const *part, int dtype, uint64_t n,
                        float *out, int accumulate, float loss_scale) {
  return zso_reduce_avg_wire(world, rank, part, dtype, ZSO_WIRE_FP32, n, out, accumulate,
                             loss_scale);
}

uint32_t zso_check_overflow(const float *a, uint64_t n, float loss_scale) {
  for (uint64_t i = 0; i < n; ++i)
    if (!isfinite(a[i] / loss_scale)) return 1;
  return 0;
}

/* ---- AdamW ([Notes] 三: gradients to FP32 and unscaled, first and second
 * moments updated, then the FP32 master weight, then the FP16 copy; [L7]
 * memory table: FP32 master, m, v; [L7] DDP example names AdamW) --------- */

void zso_adamw_consts_make(float lr, float beta1, float beta2, float eps,
                           float weight_decay, uint32_t t,
                           zso_adamw_consts *out) {
  double b1 = beta1, b2 = beta2, l = lr, wd = weight_decay;
  double b1t = 1.0, b2t = 1.0;
  for (uint32_t k = 0; k < t; ++k) {
    b1t *= b1;
    b2t *= b2;
  }
  out->alpha = (float)(l / (1.0 - b1t));
  out->b2 = (float)sqrt(1.0 - b2t);
  out->delta = (float)(1.0 - l * wd);
  out->c1 = (float)(1.0 - b1);
  out->c2 = (float)(1.0 - b2);
  out->beta1 = beta1;
  out->beta2 = beta2;
  out->eps = eps;
}

/* One element of the update; returns the new master weight. */
static float adamw_elem(float theta, float *m, float *v, float g,
                        const zso_adamw_consts *k) {
  float decayed = theta * k->delta;                  /* decoupled decay    */
  float m1 = k->beta1 * *m + k->c1 * g;              /* first moment       */
  float v1 = k->beta2 * *v + k->c2 * (g * g);        /* second moment      */
  float d = sqrtf(v1) / k->b2 + k->eps;              /* bias-corrected rms */
  float theta1 = decayed - k->alpha * (m1 / d);      /* alpha holds 1/bc1  */
  *m = m1;
  *v = v1;
  return theta1;
}

void zso_adamw(float *master, float *m, float *v, const float *a, uint64_t n,
               float loss_scale, const zso_adamw_consts *k) {
  for (uint64_t i = 0; i < n; ++i) {
    float g = a[i] / loss_scale;
    master[i] = adamw_elem(master[i], &m[i], &v[i], g, k);
  }
}

/* ---- whole step, threaded over disjoint ranges -------------------------- */

typedef struct {
  const zso_step_args *a;
  const zso_adamw_consts *k;
  uint64_t lo, hi;
  uint32_t flag;
} step_job;

static void *step_range(void *arg) {
  step_job *job = (step_job *)arg;
  const zso_step_args *a = job->a;
  const float wf = (float)a->world;
  uint32_t flag = 0;
  for (uint64_t i = job->lo; i < job->hi; ++i) {
    float s = ring_elem(a->world, a->rank, a->part, a->grad_dtype, a->wire, i);
    float avg = s / wf;
    if (a->acc_in) avg = a->acc_in[i] + avg;
    float g = avg / a->loss_scale;
    if (!isfinite(g)) flag = 1;
    float m = a->m_in[i], v = a->v_in[i];
    float theta = adamw_elem(a->master_in[i], &m, &v, g, job->k);
    a->master_out[i] = theta;
    a->m_out[i] = m;
    a->v_out[i] = v;
    a->param_out[i] = zso_float_to_half(theta, a->param_dtype);
  }
  job->flag = flag;
  return NULL;
}

uint32_t zso_shard_step(const zso_step_args *a, int threads) {
  zso_adamw_consts k;
  zso_adamw_consts_make(a->lr, a->beta1, a->beta2, a->eps, a->weight_decay,
                        a->step_t, &k);
  if (threads < 1) threads = 1;
  if ((uint64_t)threads > a->n) threads = a->n ? (int)a->n : 1;
  step_job *jobs = (step_job *)calloc((size_t)threads, sizeof(step_job));
  pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
  if (!jobs || !tids) {
    free(jobs);
    free(tids);
    return 0xffffffffu;
  }
  for (int t = 0; t < threads; ++t) {
    jobs[t].a = a;
    jobs[t].k = &k;
    jobs[t].lo = a->n * (uint64_t)t / (uint64_t)threads;
    jobs[t].hi = a->n * (uint64_t)(t + 1) / (uint64_t)threads;
  }
  for (int t = 1; t < threads; ++t)
    pthread_create(&tids[t], NULL, step_range, &jobs[t]);
  step_range(&jobs[0]);
  uint32_t flag = jobs[0].flag;
  for (int t = 1; t < threads; ++t) {
    pthread_join(tids[t], NULL);
    flag |= jobs[t].flag;
  }
  free(jobs);
  free(tids);
  return flag;
}

/* ---- dynamic loss scaler (reading; see the header) ---------------------- */

void zso_scaler_update(zso_scaler *s, uint32_t overflow) {
  if (overflow) {
    s->scale = s->scale * 0.5f;
    s->clean = 0;
    s->skipped += 1;
    return;
  }
  s->t += 1;
  s->clean += 1;
  if (s->clean >= s->interval) {
    s->scale = s->scale * 2.0f;
    s->clean = 0;
  }
}

/* ---- accounting ([Notes] 三 and 四 with K = 12; [L7] ZeRO stages) -------- */

double zso_model_state_bytes(double psi, double n_gpus, int stage, double k) {
  switch (stage) {
    case 0: return (2.0 + 2.0 + k) * psi;
    case 1: return (2.0 + 2.0) * psi + k * psi / n_gpus;
    case 2: return 2.0 * psi + (2.0 + k) * psi / n_gpus;
    case 3: return (2.0 + 2.0 + k) * psi / n_gpus;
    default: return -1.0;
  }
}

double zso_ring_allreduce_time(double msg_bytes, double world, double alpha,
                               double beta) {
  return 2.0 * (world - 1.0) * alpha +
         2.0 * msg_bytes * (world - 1.0) / (world * beta);
}
