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
#include <sched.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "zeroshard.h"
#include "zs_hparams.h"
#include "zs_host_powers.h"
#include "zs_offload_pieces.h"

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

/* A persistent pool of worker threads, created on first use and grown on
 * demand, so a step does not pay for thread creation. Every worker runs
 * with MXCSR set to round-to-nearest, subnormals kept (the caller's thread,
 * which takes task 0, switches for the duration of run()). One run() at a
 * time: calls from several host threads are serialized. Every worker checks
 * out of every run, with or without a task, and run() returns only after
 * all have: no worker can still be claiming tasks of a finished run when
 * the next one starts. The workers live until the process ends.
 *
 * Hand-off is an atomic generation counter. After a run a worker polls it
 * for kSpinMicros before it sleeps on the condition variable, and run()
 * polls the check-out count before it sleeps, so back-to-back runs (a step
 * updated piece by piece as its gradient arrives) cost no futex wake-ups:
 * with every worker asleep, a dispatch had cost more than a 64 Ki-element
 * update (79 against 16 us per call at 8 threads). The poll pauses for the
 * first kPauseMicros and then yields the core between tests: with as many
 * workers as CPUs, pure spinning starved the caller's thread and the GPU
 * runtime's threads between pieces and made a pipelined ZeRO-Offload step
 * 10-30 % slower, while yielding measured even with the sleeping pool
 * there. Sleeping is lost-wakeup safe: the sleeper counts
 * itself (sleepers_ / runner_waiting_) before it re-tests the condition
 * under mu_, and the waker changes the condition before it reads that count
 * (all sequentially consistent), then notifies after taking mu_. */
class Pool {
 public:
  static Pool &instance() {
    static Pool *p = new Pool();  /* never destroyed: workers may be parked */
    return *p;
  }

  /* fn(task) for task in [0, tasks); returns when all are done. */
  void run(int tasks, const std::function<void(int)> &fn) {
    std::lock_guard<std::mutex> serial(run_mu_);
    grow(tasks - 1);
    fn_ = &fn;
    tasks_ = tasks;
    next_.store(1, std::memory_order_relaxed);
    pending_.store((int)workers_.size(), std::memory_order_relaxed);
    generation_.fetch_add(1);  /* publishes the fields above */
    if (sleepers_.load() > 0) {
      { std::lock_guard<std::mutex> lk(mu_); }
      cv_work_.notify_all();
    }
    const unsigned saved = _mm_getcsr();
    _mm_setcsr(kMxcsrNearest);
    fn(0);
    _mm_setcsr(saved);
    if (!spin_until([&] { return pending_.load() == 0; })) {
      std::unique_lock<std::mutex> lk(mu_);
      runner_waiting_.store(true);
      cv_done_.wait(lk, [&] { return pending_.load() == 0; });
      runner_waiting_.store(false);
    }
    fn_ = nullptr;
  }

 private:
  static constexpr int kSpinMicros = 200;
  static constexpr int kPauseMicros = 8;

  /* Polls until pred() holds or kSpinMicros pass: with pause for the first
   * kPauseMicros, then yielding the core between tests. */
  template <typename P>
  static bool spin_until(P pred) {
    const auto t0 = std::chrono::steady_clock::now();
    bool yielding = false;
    for (unsigned i = 1;; ++i) {
      if (pred()) return true;
      if (yielding) std::this_thread::yield();
      else _mm_pause();
      if ((i & 63u) == 0 || yielding) {
        const auto dt = std::chrono::steady_clock::now() - t0;
        if (dt > std::chrono::microseconds(kSpinMicros)) return pred();
        yielding = dt > std::chrono::microseconds(kPauseMicros);
      }
    }
  }

  /* Called by run() before it opens the next generation; generation_ only
   * changes inside run(), so a new worker starts out waiting for exactly
   * that next generation. */
  void grow(int want) {
    while ((int)workers_.size() < want) {
      const uint64_t current = generation_.load();
      workers_.emplace_back([this, current] { loop(current); });
    }
  }

  void loop(uint64_t seen) {
    _mm_setcsr(kMxcsrNearest);
    for (;;) {
      if (!spin_until([&] { return generation_.load() != seen; })) {
        std::unique_lock<std::mutex> lk(mu_);
        sleepers_.fetch_add(1);
        cv_work_.wait(lk, [&] { return generation_.load() != seen; });
        sleepers_.fetch_sub(1);
      }
      /* run() waits for this worker's check-out before it can open another
       * generation, so this is exactly the next one */
      seen = generation_.load();
      const std::function<void(int)> *fn = fn_;
      const int tasks = tasks_;
      for (int t = next_.fetch_add(1); t < tasks; t = next_.fetch_add(1)) (*fn)(t);
      if (pending_.fetch_sub(1) == 1 && runner_waiting_.load()) {
        { std::lock_guard<std::mutex> lk(mu_); }
        cv_done_.notify_one();
      }
    }
  }

  std::mutex run_mu_, mu_;
  std::condition_variable cv_work_, cv_done_;
  std::vector<std::thread> workers_;
  const std::function<void(int)> *fn_ = nullptr;  /* published by generation_ */
  int tasks_ = 0;                                 /* published by generation_ */
  std::atomic<int> next_{0};
  std::atomic<int> pending_{0};
  std::atomic<uint64_t> generation_{0};
  std::atomic<int> sleepers_{0};
  std::atomic<bool> runner_waiting_{false};
};

/* Runs fn(t, lo, hi) over `threads` contiguous ranges on the pool. */
template <typename F>
void parallel_ranges(uint64_t n, int threads, F fn) {
  Pool::instance().run(threads, [&](int t) {
    uint64_t lo = n * (uint64_t)t / (uint64_t)threads;
    uint64_t hi = n * (uint64_t)(t + 1) / (uint64_t)threads;
    fn(t, lo, hi);
  });
}

}  // namespace

namespace {

/* Argument checks shared by both entry points, and the per-step scalars:
 * binary64, beta^t by t repeated products, rounded once to fp32 (the
 * device kernels' make-up of the same constants). */
int prepare(const float *master, const float *m, const float *v, const float *grad_part,
            uint64_t n, const zs_adamw_hparams *hp, const void *params16, int param_dtype,
            Consts *k) {
  if (!master || !m || !v || !grad_part || !hp || !params16) return ZS_ERR_INVALID_ARG;
  if (n > (1ull << 48)) return ZS_ERR_UNSUPPORTED;
  if (param_dtype != ZS_BF16 && param_dtype != ZS_FP16) return ZS_ERR_INVALID_ARG;
  if (!(hp->loss_scale > 0.0f) || !isfinite(hp->loss_scale) || hp->step_t == 0)
    return ZS_ERR_INVALID_ARG;
  if (zs_host::hparams_problem(hp)) return ZS_ERR_INVALID_ARG;
  double b1 = hp->beta1, b2 = hp->beta2, lr = hp->lr, wd = hp->weight_decay;
  double b1t, b2t;
  zs_host::beta_powers(hp->beta1, hp->beta2, hp->step_t, &b1t, &b2t);
  k->alpha = (float)(lr / (1.0 - b1t));
  k->bc2 = (float)sqrt(1.0 - b2t);
  k->delta = (float)(1.0 - lr * wd);
  k->c1 = (float)(1.0 - b1);
  k->c2 = (float)(1.0 - b2);
  k->beta1 = hp->beta1;
  k->beta2 = hp->beta2;
  k->eps = hp->eps;
  k->scale = hp->loss_scale;
  return ZS_OK;
}

/* CPUs this process may run on (its affinity mask; a container or job
 * share is usually far below the machine's count), at most 64. */
int default_threads() {
  cpu_set_t set;
  CPU_ZERO(&set);
  int cpus = 0;
  if (sched_getaffinity(0, sizeof set, &set) == 0) cpus = CPU_COUNT(&set);
  if (cpus <= 0) cpus = (int)std::thread::hardware_concurrency();
  return std::min(64, std::max(1, cpus));
}

int thread_count(int threads, uint64_t n) {
  if (threads <= 0) threads = default_threads();
  return (int)std::min<uint64_t>((uint64_t)threads, std::max<uint64_t>(1, n / 4096));
}

bool have_avx512() {
  return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
}

/* Pass 2: AdamW in place and the 16-bit parameters. */
void update_all(float *master, float *m, float *v, const float *grad_part, uint64_t n,
                const Consts &k, uint16_t *out, int param_dtype, int threads) {
  const bool avx512 = have_avx512();
  parallel_ranges(n, threads, [&](int, uint64_t lo, uint64_t hi) {
    if (avx512) update_avx512(master, m, v, grad_part, lo, hi, k, out, param_dtype);
    else update_scalar(master, m, v, grad_part, lo, hi, k, out, param_dtype);
  });
}

}  // namespace

extern "C" int zs_cpu_step(float *master, float *m, float *v, const float *grad_part, uint64_t n,
                           const zs_adamw_hparams *hp, void *params16, int param_dtype,
                           int threads, uint32_t *overflow) {
  if (!overflow) return ZS_ERR_INVALID_ARG;
  Consts k;
  int rc = prepare(master, m, v, grad_part, n, hp, params16, param_dtype, &k);
  if (rc != ZS_OK) return rc;
  *overflow = 0;
  if (n == 0) return ZS_OK;
  threads = thread_count(threads, n);
  const bool avx512 = have_avx512();
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
  update_all(master, m, v, grad_part, n, k, static_cast<uint16_t *>(params16), param_dtype,
             threads);
  return ZS_OK;
}

extern "C" int zs_cpu_update(float *master, float *m, float *v, const float *grad_part,
                             uint64_t n, const zs_adamw_hparams *hp, void *params16,
                             int param_dtype, int threads) {
  Consts k;
  int rc = prepare(master, m, v, grad_part, n, hp, params16, param_dtype, &k);
  if (rc != ZS_OK) return rc;
  if (n == 0) return ZS_OK;
  update_all(master, m, v, grad_part, n, k, static_cast<uint16_t *>(params16), param_dtype,
             thread_count(threads, n));
  return ZS_OK;
}

namespace {

/* Waits (pause, then yielding the core) until flag leaves `from`. */
int wait_while(const std::atomic<int> &flag, int from) {
  for (unsigned i = 0;; ++i) {
    const int s = flag.load();
    if (s != from) return s;
    if (i < 2048) _mm_pause();
    else std::this_thread::yield();
  }
}

}  // namespace

int zs_host::update_in_pieces(float *master, float *m, float *v, const float *grad, uint64_t n,
                              const zs_adamw_hparams *hp, void *params16, int param_dtype,
                              int threads, const uint64_t *cuts, int pieces,
                              const PieceHooks &hooks) {
  Consts k;
  int rc = prepare(master, m, v, grad, n, hp, params16, param_dtype, &k);
  if (rc != ZS_OK) return rc;
  if (!cuts || pieces <= 0 || !hooks.arrived || !hooks.updated) return ZS_ERR_INVALID_ARG;
  if (cuts[0] != 0 || cuts[pieces] != n) return ZS_ERR_INVALID_ARG;
  for (int p = 0; p < pieces; ++p)
    if (cuts[p] > cuts[p + 1]) return ZS_ERR_INVALID_ARG;
  if (n == 0) return ZS_OK;
  threads = thread_count(threads, n);
  const bool avx512 = have_avx512();
  uint16_t *out = static_cast<uint16_t *>(params16);
  /* per piece: 0 not yet claimed, 1 a thread waits in arrived(), 2 arrived,
   * -1 arrived() failed; and the threads still working on it */
  std::unique_ptr<std::atomic<int>[]> state(new std::atomic<int>[pieces]);
  std::unique_ptr<std::atomic<int>[]> left(new std::atomic<int>[pieces]);
  for (int p = 0; p < pieces; ++p) {
    state[p].store(0);
    left[p].store(threads);
  }
  std::atomic<bool> failed{false};
  Pool::instance().run(threads, [&](int t) {
    for (int p = 0; p < pieces; ++p) {
      int s = state[p].load();
      if (s == 0) {
        int expected = 0;
        if (state[p].compare_exchange_strong(expected, 1)) {
          s = hooks.arrived(hooks.ctx, p) == 0 ? 2 : -1;
          state[p].store(s);
        } else {
          s = expected;
        }
      }
      if (s == 1) s = wait_while(state[p], 1);
      if (s < 0) {
        failed.store(true);
        return;
      }
      const uint64_t len = cuts[p + 1] - cuts[p];
      const uint64_t lo = cuts[p] + len * (uint64_t)t / (uint64_t)threads;
      const uint64_t hi = cuts[p] + len * (uint64_t)(t + 1) / (uint64_t)threads;
      if (hi > lo) {
        if (avx512) update_avx512(master, m, v, grad, lo, hi, k, out, param_dtype);
        else update_scalar(master, m, v, grad, lo, hi, k, out, param_dtype);
      }
      if (left[p].fetch_sub(1) == 1) hooks.updated(hooks.ctx, p);
    }
  });
  return failed.load() ? ZS_ERR_HIP : ZS_OK;
}
