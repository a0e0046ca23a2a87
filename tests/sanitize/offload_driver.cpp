/*
 * Exercises zs_cpu_step (the ZeRO-Offload host update, product code) for a
 * build under AddressSanitizer + UndefinedBehaviorSanitizer or
 * ThreadSanitizer (test infrastructure; run by tests/test_sanitizers.py):
 * ragged sizes, one and several worker threads (results must not depend on
 * the thread count), both parameter dtypes, and the skip on a non-finite
 * gradient at either end; and the piecewise update behind zs_offload_step
 * (zs_host::update_in_pieces) with host-side hooks: pieces that arrive
 * late, each piece announced once and only when final, a failing arrival.
 * Exits non-zero on an inconsistency.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <thread>
#include <vector>

#include "zeroshard.h"
#include "zs_offload_pieces.h"

static unsigned long long rs = 0x9E3779B97F4A7C15ull;
static float rf(float scale) {
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return ((float)((rs >> 40) & 0xffffff) / 16777216.0f - 0.5f) * scale;
}

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main() {
  const uint64_t sizes[] = {0, 1, 15, 16, 17, 4099, 100003};
  zs_adamw_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1024.0f, 5};
  for (uint64_t n : sizes)
    for (int dtype = 0; dtype < 2; ++dtype) {
      /* one spare element so that n == 0 still passes valid pointers */
      std::vector<float> master(n + 1), m(n + 1), v(n + 1), g(n + 1);
      for (uint64_t i = 0; i < n; ++i) {
        master[i] = rf(0.04f);
        m[i] = rf(2e-4f);
        v[i] = fabsf(rf(2e-6f));
        g[i] = rf(4.0f);
      }
      std::vector<float> st[2][3];
      std::vector<uint16_t> p[2];
      const int threads[2] = {1, 3};
      for (int t = 0; t < 2; ++t) {
        st[t][0] = master;
        st[t][1] = m;
        st[t][2] = v;
        p[t].assign(n + 1, 0);
        uint32_t ovf = 7;
        CHECK(zs_cpu_step(st[t][0].data(), st[t][1].data(), st[t][2].data(), g.data(), n, &hp,
                          p[t].data(), dtype, threads[t], &ovf) == ZS_OK);
        CHECK(ovf == 0);
      }
      for (int j = 0; j < 3; ++j)
        CHECK(n == 0 || memcmp(st[0][j].data(), st[1][j].data(), n * 4) == 0);
      CHECK(n == 0 || memcmp(p[0].data(), p[1].data(), n * 2) == 0);
      if (n == 0) continue;
      for (uint64_t pos : {(uint64_t)0, n - 1}) {
        std::vector<float> bad = g;
        bad[pos] = pos ? NAN : -INFINITY;
        std::vector<float> a = master, b = m, c = v;
        std::vector<uint16_t> q(n, 0x1234);
        uint32_t ovf = 0;
        CHECK(zs_cpu_step(a.data(), b.data(), c.data(), bad.data(), n, &hp, q.data(), dtype, 4,
                          &ovf) == ZS_OK);
        CHECK(ovf == 1);
        CHECK(memcmp(a.data(), master.data(), n * 4) == 0 && q[n - 1] == 0x1234);
      }
    }
  /* Many short runs back to back with changing thread counts (the worker
   * pool's run boundaries), then two host threads calling at once (runs are
   * serialized); each result must equal a one-thread reference. */
  {
    const uint64_t n = 70001;  /* up to 17 threads (n / 4096) */
    std::vector<float> g(n), m0(n), v0(n), t0(n);
    for (uint64_t i = 0; i < n; ++i) {
      t0[i] = rf(0.04f);
      m0[i] = rf(2e-4f);
      v0[i] = fabsf(rf(2e-6f));
      g[i] = rf(4.0f);
    }
    std::vector<float> rt = t0, rm = m0, rv = v0;
    std::vector<uint16_t> rp(n);
    uint32_t ovf;
    CHECK(zs_cpu_step(rt.data(), rm.data(), rv.data(), g.data(), n, &hp, rp.data(), 0, 1, &ovf) ==
          ZS_OK);
    for (int rep = 0; rep < 200; ++rep) {
      std::vector<float> a = t0, b = m0, c = v0;
      std::vector<uint16_t> q(n);
      CHECK(zs_cpu_step(a.data(), b.data(), c.data(), g.data(), n, &hp, q.data(), 0,
                        1 + rep % 7, &ovf) == ZS_OK);
      CHECK(memcmp(a.data(), rt.data(), n * 4) == 0 && memcmp(q.data(), rp.data(), n * 2) == 0);
    }
    int bad = 0;
    auto caller = [&](int seed) {
      for (int rep = 0; rep < 50; ++rep) {
        std::vector<float> a = t0, b = m0, c = v0;
        std::vector<uint16_t> q(n);
        uint32_t o;
        if (zs_cpu_step(a.data(), b.data(), c.data(), g.data(), n, &hp, q.data(), 0,
                        2 + (seed + rep) % 5, &o) != ZS_OK ||
            memcmp(a.data(), rt.data(), n * 4) != 0)
          __atomic_fetch_add(&bad, 1, __ATOMIC_RELAXED);
      }
    };
    std::thread x(caller, 1), y(caller, 2);
    x.join();
    y.join();
    CHECK(bad == 0);
    /* runs spaced past the pool's spin window, so the workers (and the
     * caller waiting for them) go to sleep and are woken through the
     * condition variables */
    for (int rep = 0; rep < 12; ++rep) {
      std::this_thread::sleep_for(std::chrono::milliseconds(2));
      std::vector<float> a = t0, b = m0, c = v0;
      std::vector<uint16_t> q(n);
      CHECK(zs_cpu_step(a.data(), b.data(), c.data(), g.data(), n, &hp, q.data(), 0,
                        2 + rep % 6, &ovf) == ZS_OK);
      CHECK(memcmp(a.data(), rt.data(), n * 4) == 0 && memcmp(q.data(), rp.data(), n * 2) == 0);
    }
  }
  /* update_in_pieces against zs_cpu_update: several piece and thread
   * counts, empty pieces, late arrivals; every piece announced once, after
   * its elements are final; a failing arrival stops at that piece. */
  {
    const uint64_t n = 90011;
    std::vector<float> g(n), m0(n), v0(n), t0(n);
    for (uint64_t i = 0; i < n; ++i) {
      t0[i] = rf(0.04f);
      m0[i] = rf(2e-4f);
      v0[i] = fabsf(rf(2e-6f));
      g[i] = rf(4.0f);
    }
    std::vector<float> rt = t0, rm = m0, rv = v0;
    std::vector<uint16_t> rp(n);
    CHECK(zs_cpu_update(rt.data(), rm.data(), rv.data(), g.data(), n, &hp, rp.data(), 0, 1) ==
          ZS_OK);
    struct Ctx {
      const uint64_t *cuts;
      const float *ref;
      const float *master;
      std::vector<int> arrived_calls, updated_calls;
      int fail_at;
      int bad;
    };
    auto arrived = [](void *c, int k) -> int {
      Ctx *x = static_cast<Ctx *>(c);
      __atomic_fetch_add(&x->arrived_calls[(size_t)k], 1, __ATOMIC_RELAXED);
      if (k % 3 == 1) std::this_thread::sleep_for(std::chrono::microseconds(300));
      return k == x->fail_at ? 1 : 0;
    };
    auto updated = [](void *c, int k) {
      Ctx *x = static_cast<Ctx *>(c);
      __atomic_fetch_add(&x->updated_calls[(size_t)k], 1, __ATOMIC_RELAXED);
      const uint64_t lo = x->cuts[k], hi = x->cuts[k + 1];
      if (hi > lo && memcmp(x->master + lo, x->ref + lo, (hi - lo) * 4) != 0)
        __atomic_fetch_add(&x->bad, 1, __ATOMIC_RELAXED);
    };
    const int piece_counts[] = {1, 2, 7, 33};
    const int thread_counts[] = {1, 3, 8};
    for (int pieces : piece_counts)
      for (int threads : thread_counts)
        for (int fail_at : {-1, 2}) {
          if (fail_at >= pieces) continue;
          std::vector<uint64_t> cuts((size_t)pieces + 1);
          for (int k = 0; k < pieces; ++k)
            cuts[(size_t)k] = (k == 1 ? 0 : n * (uint64_t)k / (uint64_t)pieces / 64 * 64);
          cuts[(size_t)pieces] = n;  /* piece 0 is empty when pieces > 1 */
          std::vector<float> a = t0, b = m0, c = v0;
          std::vector<uint16_t> q(n, 0);
          Ctx ctx{cuts.data(), rt.data(), a.data(), std::vector<int>((size_t)pieces, 0),
                  std::vector<int>((size_t)pieces, 0), fail_at, 0};
          zs_host::PieceHooks hooks{&ctx, +arrived, +updated};
          const int rc = zs_host::update_in_pieces(a.data(), b.data(), c.data(), g.data(), n, &hp,
                                                   q.data(), 0, threads, cuts.data(), pieces,
                                                   hooks);
          CHECK(ctx.bad == 0);
          if (fail_at < 0) {
            CHECK(rc == ZS_OK);
            for (int k = 0; k < pieces; ++k)
              CHECK(ctx.arrived_calls[(size_t)k] == 1 && ctx.updated_calls[(size_t)k] == 1);
            CHECK(memcmp(a.data(), rt.data(), n * 4) == 0 &&
                  memcmp(b.data(), rm.data(), n * 4) == 0 &&
                  memcmp(c.data(), rv.data(), n * 4) == 0 &&
                  memcmp(q.data(), rp.data(), n * 2) == 0);
          } else {
            CHECK(rc == ZS_ERR_HIP);
            for (int k = 0; k < pieces; ++k) {
              CHECK(ctx.updated_calls[(size_t)k] == (k < fail_at ? 1 : 0));
              CHECK(ctx.arrived_calls[(size_t)k] == (k <= fail_at ? 1 : 0));
            }
            const uint64_t done = cuts[(size_t)fail_at];
            CHECK(memcmp(a.data(), rt.data(), done * 4) == 0);
            CHECK(memcmp(a.data() + done, t0.data() + done, (n - done) * 4) == 0);
          }
        }
    /* bad cuts and hooks are refused */
    std::vector<float> a = t0, b = m0, c = v0;
    std::vector<uint16_t> q(n, 0);
    Ctx ctx{nullptr, rt.data(), a.data(), std::vector<int>(4, 0), std::vector<int>(4, 0), -1, 0};
    zs_host::PieceHooks hooks{&ctx, +arrived, +updated};
    const uint64_t bad1[] = {0, 500, 100, n};
    const uint64_t bad2[] = {1, 500, 1000, n};
    const uint64_t bad3[] = {0, 500, 1000, n - 1};
    for (const uint64_t *bc : {bad1, bad2, bad3})
      CHECK(zs_host::update_in_pieces(a.data(), b.data(), c.data(), g.data(), n, &hp, q.data(), 0,
                                      2, bc, 3, hooks) == ZS_ERR_INVALID_ARG);
    zs_host::PieceHooks none{&ctx, nullptr, +updated};
    const uint64_t good[] = {0, n};
    CHECK(zs_host::update_in_pieces(a.data(), b.data(), c.data(), g.data(), n, &hp, q.data(), 0, 2,
                                    good, 1, none) == ZS_ERR_INVALID_ARG);
    CHECK(memcmp(a.data(), t0.data(), n * 4) == 0);
  }
  uint32_t ovf;
  float x = 0;
  uint16_t h = 0;
  CHECK(zs_cpu_step(nullptr, &x, &x, &x, 1, &hp, &h, 0, 1, &ovf) == ZS_ERR_INVALID_ARG);
  printf("offload driver ok\n");
  return 0;
}
