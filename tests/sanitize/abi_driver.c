/*
 * Exercises the host-only logic of libzeroshard (partition, scaler update,
 * device-scaler image, status strings, and argument rejection of the kernel
 * entry points, which returns before any HIP call) for a build of the
 * library with AddressSanitizer + UndefinedBehaviorSanitizer on its host
 * code (test infrastructure; run by tests/test_sanitizers.py). No GPU work:
 * the pointers below are never dereferenced.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zeroshard.h"

/* the layout the Python binding mirrors */
_Static_assert(sizeof(zs_step_args) == 152, "zs_step_args size");
_Static_assert(offsetof(zs_step_args, wire_dtype) == 140, "wire_dtype offset");
_Static_assert(offsetof(zs_step_args, state_layout) == 144, "state_layout offset");

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

#define FAKE ((uintptr_t)0x7F0000000000ull)

int main(void) {
  CHECK(zs_abi_version() == ZS_ABI_VERSION);
  for (int s = -1; s < 7; ++s) CHECK(strlen(zs_status_string(s)) > 0);
  for (uint64_t phi = 0; phi < 300; phi += 7)
    for (uint32_t w = 1; w <= 9; ++w) {
      uint64_t total = 0;
      for (uint32_t r = 0; r < w; ++r) {
        uint64_t c, o, n;
        CHECK(zs_partition(phi, w, r, &c, &o, &n) == ZS_OK);
        total += n;
      }
      CHECK(total == phi);
      CHECK(zs_partition(phi, w, w, NULL, NULL, NULL) == ZS_ERR_INVALID_ARG);
      CHECK(strlen(zs_last_error()) > 0);
    }
  zs_loss_scaler sc = {65536.0f, 0, 4, 1, 0, 0};
  for (int i = 0; i < 40; ++i) CHECK(zs_scaler_update(&sc, (i % 9) == 4) == ZS_OK);
  CHECK(sc.step_t + sc.skipped == 40);
  CHECK(zs_scaler_update(NULL, 0) == ZS_ERR_INVALID_ARG);
  zs_device_scaler img;
  CHECK(zs_device_scaler_make(&sc, 0.9f, 0.999f, &img) == ZS_OK);
  CHECK(img.step_t == sc.step_t && img.beta1_t > 0.0 && img.beta1_t < 1.0);
  sc.scale = INFINITY;
  CHECK(zs_device_scaler_make(&sc, 0.9f, 0.999f, &img) == ZS_ERR_INVALID_ARG);

  const void *grads[3] = {(void *)FAKE, (void *)(FAKE + 0x100000), (void *)(FAKE + 0x200000)};
  CHECK(zs_reduce_scatter_avg(grads, 0, 0, 3, 3, 10, (float *)(FAKE + 0x300000), 0, NULL, 1.0f,
                              NULL) == ZS_ERR_INVALID_ARG);
  CHECK(zs_reduce_scatter_avg(grads, 0, 7, 3, 0, 10, (float *)(FAKE + 0x300000), 0, NULL, 1.0f,
                              NULL) == ZS_ERR_INVALID_ARG);
  zs_step_args a;
  memset(&a, 0, sizeof a);
  a.world = 3;
  a.rank = 0;
  a.n = 1000;
  a.worker_grads = grads;
  uintptr_t base = FAKE + 0x1000000;
  a.master_in = (const float *)base;
  a.m_in = (const float *)(base + 0x100000);
  a.v_in = (const float *)(base + 0x200000);
  a.master_out = (float *)base; /* aliases master_in */
  a.m_out = (float *)(base + 0x400000);
  a.v_out = (float *)(base + 0x500000);
  a.gather_buf = (void *)(base + 0x600000);
  a.overflow_flag = (uint32_t *)(base + 0x700000);
  zs_adamw_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1.0f, 1};
  a.hp = hp;
  CHECK(zs_step_fused(&a, NULL) == ZS_ERR_ALIAS);
  CHECK(zs_step_device(&a, (zs_device_scaler *)(base + 0x800000), NULL, NULL, NULL) ==
        ZS_ERR_ALIAS);
  CHECK(zs_step_device(&a, NULL, NULL, NULL, NULL) == ZS_ERR_INVALID_ARG);
  a.master_out = (float *)(base + 0x300000);
  a.grad_dtype = 9;
  CHECK(zs_step_fused(&a, NULL) == ZS_ERR_INVALID_ARG);
  void *reps[3] = {(void *)FAKE, (void *)(FAKE + 100), (void *)(FAKE + 0x200000)};
  CHECK(zs_all_gather_step(reps, 3, 1000, 0, 1, NULL) == ZS_ERR_ALIAS);
  CHECK(zs_all_gather_step(reps, 3, 1000, 0, 3, NULL) == ZS_ERR_INVALID_ARG);
  printf("abi driver ok\n");
  return 0;
}
