/*
 * Exercises every function of the CPU oracle on small inputs, for a build
 * under AddressSanitizer + UndefinedBehaviorSanitizer or ThreadSanitizer
 * (test infrastructure; run by tests/test_sanitizers.py). Exits non-zero on
 * an inconsistency; the sanitizers abort on a memory error, undefined
 * behaviour or a data race.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zs_oracle.h"

static unsigned long long rs = 88172645463325252ull;
static unsigned rnd(void) {
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return (unsigned)(rs >> 32);
}
static float rf(float scale) { return ((float)(rnd() & 0xffffff) / 16777216.0f - 0.5f) * scale; }

#define CHECK(c)                                             \
  do {                                                       \
    if (!(c)) {                                              \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                              \
    }                                                        \
  } while (0)

static int partitions(void) {
  const unsigned long long phis[] = {0, 1, 7, 1000, 4099};
  for (int a = 0; a < 5; ++a)
    for (unsigned w = 1; w <= 17; ++w) {
      unsigned long long total = 0;
      for (unsigned r = 0; r < w; ++r) {
        uint64_t chunk, off, cnt;
        CHECK(zso_partition(phis[a], w, r, &chunk, &off, &cnt) == 0);
        total += cnt;
      }
      CHECK(total == phis[a]);
      uint64_t c, o, n;
      CHECK(zso_partition(phis[a], w, w, &c, &o, &n) == -1);
    }
  return 0;
}

static int rings(void) {
  for (unsigned w = 1; w <= 6; ++w)
    for (int sigma = 0; sigma < 2; ++sigma) {
      const uint64_t L = 5;
      size_t cnt = (size_t)w * w * L;
      float *b = malloc(cnt * sizeof(float));
      for (size_t i = 0; i < cnt; ++i) b[i] = (float)(int)(rnd() % 64);
      CHECK(zso_ring_reduce_scatter(w, L, sigma, w - 1, b) == 0);
      CHECK(zso_ring_all_gather(w, L, sigma, w - 1, b) == 0);
      CHECK(zso_ring_reduce_scatter(w, L, sigma, w, b) == -1);
      CHECK(zso_ring_held_chunk(w, 0, sigma) < w);
      /* after the gather every rank holds the same buffer */
      for (unsigned k = 1; k < w; ++k) CHECK(memcmp(b, b + (size_t)k * w * L, w * L * 4) == 0);
      free(b);
    }
  return 0;
}

static int reductions(void) {
  const unsigned worlds[] = {1, 3, 8};
  const uint64_t n = 1031;
  for (int a = 0; a < 3; ++a)
    for (int dt = 0; dt < 2; ++dt) {
      unsigned w = worlds[a];
      uint16_t *g = malloc((size_t)w * n * 2);
      const uint16_t *parts[8];
      for (unsigned k = 0; k < w; ++k) {
        for (uint64_t i = 0; i < n; ++i) g[k * n + i] = zso_float_to_half(rf(2.0f), dt);
        parts[k] = g + k * n;
      }
      float *s = malloc(n * 4), *acc = malloc(n * 4);
      zso_ring_chunk_sum(w, 0, parts, dt, n, s);
      for (int wire = 0; wire < 3; ++wire) {
        zso_ring_chunk_sum_wire(w, w - 1, parts, dt, wire, n, s);
        CHECK(zso_reduce_avg_wire(w, 0, parts, dt, wire, n, acc, 0, 1024.0f) == 0);
        CHECK(zso_reduce_avg_wire(w, 0, parts, dt, wire, n, acc, 1, 1024.0f) == 0);
      }
      CHECK(zso_reduce_avg(w, 0, parts, dt, n, acc, 0, 3.0f) == 0);
      CHECK(zso_check_overflow(acc, n, 3.0f) == 0);
      acc[n - 1] = INFINITY;
      CHECK(zso_check_overflow(acc, n, 3.0f) == 1);
      free(g);
      free(s);
      free(acc);
    }
  return 0;
}

static int steps(void) {
  const uint64_t n = 4099;
  const unsigned w = 3;
  uint16_t *g = malloc((size_t)w * n * 2);
  const uint16_t *parts[3];
  for (unsigned k = 0; k < w; ++k) {
    for (uint64_t i = 0; i < n; ++i) g[k * n + i] = zso_float_to_half(rf(8.0f), ZSO_BF16);
    parts[k] = g + k * n;
  }
  float *st = malloc(n * 4 * 13);
  float *master = st, *m = st + n, *v = st + 2 * n, *acc = st + 3 * n;
  float *out[2][3] = {{st + 4 * n, st + 5 * n, st + 6 * n}, {st + 7 * n, st + 8 * n, st + 9 * n}};
  float *tmp = st + 10 * n;
  for (uint64_t i = 0; i < n; ++i) {
    master[i] = rf(0.04f);
    m[i] = rf(2e-4f);
    v[i] = fabsf(rf(2e-6f));
    acc[i] = rf(1.0f);
  }
  uint16_t *p16 = malloc(n * 4);
  zso_adamw_consts k;
  zso_adamw_consts_make(1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 7, &k);
  memcpy(tmp, master, n * 4);
  float *tm = malloc(n * 4), *tv = malloc(n * 4);
  memcpy(tm, m, n * 4);
  memcpy(tv, v, n * 4);
  zso_adamw(tmp, tm, tv, acc, n, 16.0f, &k);
  for (int wire = 0; wire < 3; ++wire)
    for (int use_acc = 0; use_acc < 2; ++use_acc) {
      uint32_t flags[2];
      const int threads[2] = {1, 4};
      for (int t = 0; t < 2; ++t) {
        zso_step_args a;
        memset(&a, 0, sizeof a);
        a.world = w;
        a.rank = 1;
        a.n = n;
        a.grad_dtype = ZSO_BF16;
        a.param_dtype = ZSO_FP16;
        a.part = parts;
        a.acc_in = use_acc ? acc : NULL;
        a.master_in = master;
        a.m_in = m;
        a.v_in = v;
        a.master_out = out[t][0];
        a.m_out = out[t][1];
        a.v_out = out[t][2];
        a.param_out = p16 + (size_t)t * n;
        a.lr = 1e-3f;
        a.beta1 = 0.9f;
        a.beta2 = 0.999f;
        a.eps = 1e-8f;
        a.weight_decay = 0.01f;
        a.loss_scale = 1024.0f;
        a.step_t = 3;
        a.wire = wire;
        flags[t] = zso_shard_step(&a, threads[t]);
      }
      CHECK(flags[0] == flags[1]);
      for (int j = 0; j < 3; ++j) CHECK(memcmp(out[0][j], out[1][j], n * 4) == 0);
      CHECK(memcmp(p16, p16 + n, n * 2) == 0);
    }
  zso_scaler sc = {65536.0f, 0, 4, 0, 0};
  for (int i = 0; i < 20; ++i) zso_scaler_update(&sc, (i % 7) == 3);
  CHECK(sc.t + sc.skipped == 20);
  CHECK(zso_model_state_bytes(7.5e9, 64, 2, 12) > 0);
  CHECK(zso_ring_allreduce_time(14e9, 8, 0, 450e9) > 0);
  float f[4] = {1.0f, -0.0f, INFINITY, NAN};
  uint16_t h[4];
  float back[4];
  zso_floats_to_halves(f, h, 4, ZSO_FP16);
  zso_halves_to_floats(h, back, 4, ZSO_FP16);
  CHECK(back[0] == 1.0f && isinf(back[2]) && isnan(back[3]));
  free(g);
  free(st);
  free(p16);
  free(tm);
  free(tv);
  return 0;
}

int main(void) {
  if (!zso_fp_env_ok()) return 2;
  if (partitions() || rings() || reductions() || steps()) return 1;
  printf("oracle driver ok\n");
  return 0;
}
