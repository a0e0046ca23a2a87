/*
 * zeroshard.hip -- libzeroshard: the per-rank ZeRO-2 optimizer-shard step for
 * AMD Instinct MI355X (gfx950, CDNA4). Host side: argument validation,
 * per-step scalars, vector-width choice, launches and the C ABI declared and
 * documented in include/zeroshard.h. The device code is in zs_kernels.h (hot
 * path) and zs_aux_kernels.h (commit, all-gather).
 */
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <math.h>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "zeroshard.h"

#include "zs_aux_kernels.h"
#include "zs_hparams.h"
#include "zs_host_powers.h"
#include "zs_host_setup.h"
#include "zs_offload_pieces.h"

/* ------------------------------------------------------------------------
 * Device memory of zs_step_commit_noalloc: the overflow word its fused pass
 * ORs into and its readback copies to the host, so that the caller need not
 * allocate one: one 4-byte word, held by every device the library runs on
 * until the process ends. In host code this name is a stand-in for the
 * variable, not a device address: host code uses only the address
 * scratch_word() resolves for the current device.
 * ---------------------------------------------------------------------- */
constexpr int kScratchWords = 1;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

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

/* Element counts and offsets above 2^48 are refused before any size
 * arithmetic (byte extents below are 4 * n and must not wrap). */
constexpr uint64_t kMaxElems = 1ull << 48;

bool too_big(uint64_t n) { return n > kMaxElems; }

bool valid_wire(int w) { return w == ZS_WIRE_FP32 || w == ZS_WIRE_BF16 || w == ZS_WIRE_FP16; }

/* zs_step_commit polls the stream for errors this often while it waits. */
constexpr int kQueryMicros = 1000;

/* The device address of `scratch` on each device ordinal, resolved the first
 * time zs_step_commit_noalloc runs with that device current (each device
 * holds its own copy at its own address). */
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch[kMaxScratchDevices] = {};

int scratch_word(uint32_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZS_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(ZS_ERR_UNSUPPORTED, "zs_step_commit_noalloc: device ordinal above 63%s");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return fail(ZS_ERR_HIP, "zs_step_commit_noalloc: hipGetSymbolAddress failed: %s",
                  hipGetErrorString(e));
    if (!ptr || (uintptr_t)ptr % 256 != 0)
      return fail(ZS_ERR_HIP, "zs_step_commit_noalloc: bad device address of its scratch%s");
    g_scratch[dev] = static_cast<uint32_t *>(ptr);
  }
  *out = g_scratch[dev];
  return ZS_OK;
}

using zs_host::make_adam;
using zs_host::make_scales;

/* ------------------------------------------------------------------------
 * Block size, tile and residency of the fused kernel. Each thread owns U
 * 4-element vectors of a tile (T * U * 4 elements per block of T threads)
 * and the blocks per CU are capped with dynamic LDS that the kernel never
 * touches. HBM delivered more on MI355X with fewer bytes in flight per CU
 * than the registers allow, by an amount that depends on W; from W = 5 on
 * the rolling sum (each wave streaming without draining) lets the fewest
 * waves win. Both state layouts share the rule from W = 4 on (the grouped
 * layout's is fused_shape_grouped below); for the split layout, interleaved
 * timings on one GPU against the alternatives (all computing the same
 * bits):
 *   - W = 1: one-wave blocks, U = 1, 12 per CU (as the grouped layout):
 *     +5 to +8 % over 256-thread blocks with U = 2 at 2 per CU on 0.5 to 2 G
 *     parameters (three GPUs); on 117 M the two traded places by GPU
 *     (ZS_FUSED_W1 = block256 selects the earlier shape for measurements).
 *   - W = 2: one-wave blocks, U = 1, 16 per CU: +7.6 to +12 % over four
 *     vectors in 256-thread blocks at 3 per CU.
 *   - W = 3: 256-thread blocks, U = 2, 3 blocks per CU from 20 000
 *     2048-element tiles on, 4 below.
 *   - W = 4: one-wave blocks, U = 2, the batched sum, 12 per CU.
 *   - W >= 5: one-wave blocks, U = 2, the rolling sum, 8 per CU up to
 *     W = 12 and 6 above (write windows as below). On 117 M parameters
 *     against the previous split-layout launches (256-thread blocks at 3
 *     per CU up to W = 16, batched one-wave blocks at 12 per CU above):
 *     W = 4 +4.5 %, W = 5 +4 %, W = 8 +7 %, W = 12 +4 %, W = 16 +4 %,
 *     W = 17 +6 %, W = 24 +3.5 %, W = 32 +2 %, W = 64 +16 % (with windows;
 *     +6 % without); W = 8 on 15.6 M +1 %.
 * Operands aligned for 2- or 1-element vectors only keep 256-thread
 * blocks, U = 2 (1 when W = 1), plain stores and 2, 3 or no cap.
 * ZS_FUSED_BLOCKS_PER_CU (0 = no cap, 1..32 = that many blocks) overrides
 * the cap, for measurements; it is read at every launch.
 * ---------------------------------------------------------------------- */

struct DeviceLds {
  int lds_per_cu = 0;  /* bytes */
};

DeviceLds device_lds() {
  static thread_local int cached_dev = -1;
  static thread_local DeviceLds cached;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DeviceLds{};
  if (dev != cached_dev) {
    DeviceLds d;
    if (hipDeviceGetAttribute(&d.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess)
      return DeviceLds{};
    cached = d;
    cached_dev = dev;
  }
  return cached;
}

/* Read at every launch, so one process can time several settings. */
int env_blocks_per_cu() {
  const char *s = getenv("ZS_FUSED_BLOCKS_PER_CU");
  if (!s || !*s) return -1;
  int x = atoi(s);
  return x < 0 || x > 32 ? -1 : x;
}

/* ZS_FUSED_W1=block256 (measurements): the split layout's W = 1 launch in
 * the earlier shape (256-thread blocks, two vectors per thread, 2 per CU). */
bool env_w1_block256() {
  const char *s = getenv("ZS_FUSED_W1");
  return s && !strcmp(s, "block256");
}

/* ZS_FUSED_SUM=batched (measurements): the grouped layout's W >= 5 shape
 * with the batched sum (kShapeB8NtL) in place of the rolling one; the cap
 * stays the rolling shape's unless ZS_FUSED_BLOCKS_PER_CU sets one. */
bool env_batched_sum() {
  const char *s = getenv("ZS_FUSED_SUM");
  return s && !strcmp(s, "batched");
}

/* Vector width, threads per block, vectors per thread, access shape
 * (zs::kShape*) and blocks per CU (0: no cap) of the fused kernel for
 * `vec`-aligned operands. */
constexpr int fused_vec_of(int aligned_vec) { return aligned_vec >= 4 ? 4 : aligned_vec; }
constexpr int kFusedWaveBlock = 64; /* one wave */
constexpr uint64_t kFusedManyTiles = 20000; /* 2048-element tiles */

struct FusedShape {
  int threads;
  int tile_vecs;
  int access;
  int cap;
};

FusedShape fused_shape(int vec, uint32_t world, uint64_t n) {
  if (vec < 4) return {kBlock, world > 1 ? 2 : 1, kShapeB8, world == 1 ? 2 : world <= 8 ? 3 : 0};
  if (world == 1)
    return env_w1_block256() ? FusedShape{kBlock, 2, kShapeB8NtL, 2}
                             : FusedShape{kFusedWaveBlock, 1, kShapeB8NtL, 12};
  if (world == 2) return {kFusedWaveBlock, 1, kShapeB8NtL, 16};
  if (world == 3) return {kBlock, 2, kShapeB8NtL, n / 2048 >= kFusedManyTiles ? 3 : 4};
  if (world == 4) return {kFusedWaveBlock, 2, kShapeB8NtL, 12};
  return {kFusedWaveBlock, 2, kShapeR4NtL, world <= 12 ? 8 : 6};
}

/* The grouped state layout runs one-wave blocks: one vector per thread at
 * 12 per CU for W = 1 and at 16 per CU for W = 2 and 3; two vectors per
 * thread from W = 4 on, with the batched sum at 12 per CU for W = 4 and the
 * rolling sum (kShapeR4NtL) from W = 5 on, at 8 per CU up to W = 12 and
 * at 6 above. With the rolling sum each wave keeps its loads in flight
 * without draining, and fewer waves per CU streamed faster (about 24 KB of
 * loads in flight per CU). Against the previous choice (the batched sum
 * everywhere, 16 per CU up to W = 16 and 12 above), interleaved on one
 * GPU, bits equal: W = 1 +3 % (two GPUs), W = 4 with fp16 gradients and
 * an accumulated input +7.7 %, W = 5 +3 %, W = 8 even, W = 16 +8 %,
 * W = 24 and 32 +5 %, W = 64 +5 to +6 % (three GPUs). */
FusedShape fused_shape_grouped(uint32_t world) {
  if (world == 1) return {kFusedWaveBlock, 1, kShapeB8NtL, 12};
  if (world <= 3) return {kFusedWaveBlock, 1, kShapeB8NtL, 16};
  if (world == 4) return {kFusedWaveBlock, 2, kShapeB8NtL, 12};
  return {kFusedWaveBlock, 2, kShapeR4NtL, world <= 12 ? 8 : 6};
}

/* ------------------------------------------------------------------------
 * Write windows (await_write_window in zs_kernels.h) for the rolling shape
 * at W >= 40 on launches of at least 4 GB of model bytes: a period of
 * 30.72 us with the last eighth open for stores, and no cap on blocks per
 * CU (the registers allow 20 one-wave blocks), since waves that wait for
 * the window still hold their slots. The launch ends up to about one
 * period after its last loads, hence the size floor. Interleaved on one
 * GPU against the same kernel without windows at its own best cap (6),
 * bits equal: W = 64 on 117 M parameters 2.70-2.83 ms against 2.98-3.03
 * (+7 to +10 %, four GPUs; periods of 25.6-40.96 us with windows of 1/8
 * to 3/16 within 1 %), on 34 M +12 %, 20 M (3.1 GB) +1 %, 10 M (1.5 GB)
 * -8 %; W = 48 +2 to +6.5 %, W = 40 +2 % (5.3 and 10.6 GB), -3 % at 2.1 GB;
 * W = 36 -1 %, W = 32 -4 %, W = 24 and below slower still (shorter tiles
 * leave too few tiles per period in each slot), W = 1 slower at every
 * period tried (half its bytes are writes).
 * ZS_FUSED_WRITE_WINDOW overrides this, for measurements and tests: "off",
 * or "<period in us>,<open fraction>" for every rolling-shape launch.
 * ---------------------------------------------------------------------- */
constexpr uint32_t kWindowWorld = 40;
constexpr double kWindowBytes = 4e9;
constexpr double kWindowPeriodUs = 30.72, kWindowOpen = 0.125;

struct WriteWindow {
  uint32_t period = 0, open_at = 0;  /* wall-clock ticks; period 0: none */
};

/* Wall-clock ticks per microsecond of the current device, 0 if unknown. */
double wall_ticks_per_us() {
  static thread_local int cached_dev = -1;
  static thread_local double cached = 0.0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0.0;
  if (dev != cached_dev) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) khz = 0;
    cached = khz > 0 ? khz / 1000.0 : 0.0;
    cached_dev = dev;
  }
  return cached;
}

WriteWindow write_window(const FusedShape &fs, uint32_t world, uint64_t n, bool acc) {
  WriteWindow w;
  if (fs.access != kShapeR4NtL) return w;
  double period_us = kWindowPeriodUs, open = kWindowOpen;
  const char *e = getenv("ZS_FUSED_WRITE_WINDOW");
  if (e && *e) {
    if (!strcmp(e, "off")) return w;
    if (sscanf(e, "%lf,%lf", &period_us, &open) != 2 || !(period_us > 0.0) || !(open > 0.0) ||
        !(open < 1.0))
      return w;
  } else {
    const double bytes = (double)n * (2.0 * world + 26.0 + (acc ? 4.0 : 0.0));
    if (world < kWindowWorld || bytes < kWindowBytes) return w;
  }
  /* at least 64 ticks per period and 16 open, so that a wave polling the
   * clock between short sleeps cannot keep missing the open part */
  const double ticks = wall_ticks_per_us() * period_us;
  if (!(ticks >= 64.0 && ticks < 4.0e9)) return w;
  w.period = (uint32_t)ticks;
  const uint32_t win = (uint32_t)(w.period * open);
  w.open_at = w.period - (win > 16 ? win : 16);
  return w;
}

/* Bytes of a grouped state buffer for n elements: whole groups. */
uint64_t grouped_state_bytes(uint64_t n) {
  return (n + ZS_STATE_GROUP - 1) / ZS_STATE_GROUP * (uint64_t)(3 * ZS_STATE_GROUP * 4);
}

/* Dynamic LDS bytes that hold the fused kernel to `cap` blocks per CU (0:
 * no cap), or to ZS_FUSED_BLOCKS_PER_CU when that is set: LDS per CU / cap
 * less 1 KB up to 8 blocks; above that LDS per CU / cap rounded down to
 * 1 KB, with no cap when that would let one more block fit. */
size_t fused_lds_bytes(int cap) {
  const int forced = env_blocks_per_cu();
  if (forced >= 0) cap = forced;
  if (cap == 0) return 0;
  const DeviceLds d = device_lds();
  if (d.lds_per_cu <= 0) return 0;
  if (cap <= 8) {
    const int bytes = (d.lds_per_cu / cap - 1024) / 256 * 256;
    return bytes > 0 ? (size_t)bytes : 0;
  }
  const int bytes = d.lds_per_cu / cap / 1024 * 1024;
  if (bytes <= 0 || (cap + 1) * bytes <= d.lds_per_cu) return 0;
  return (size_t)bytes;
}

/* Launch of one fused-kernel instance with `lds` bytes of (unused) dynamic
 * LDS; above the default 64 KB limit the instance's limit is raised once
 * per device (a bit per device id; ids past 63 raise it at every launch). */
template <int V, int U, bool L, bool A, int G, int P, int W, int F, int T, bool GR>
void launch_fused(dim3 grid, dim3 block, size_t lds, hipStream_t s, const FusedArgs &p) {
  if (lds > 65536) {
    static std::atomic<uint64_t> raised{0};
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0;
    if (!bit || !(raised.load(std::memory_order_relaxed) & bit)) {
      /* a refusal surfaces as the launch's error */
      if (hipFuncSetAttribute(reinterpret_cast<const void *>(&fused_kernel<V, U, L, A, G, P, W, F, T, GR>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)device_lds().lds_per_cu) == hipSuccess)
        raised.fetch_or(bit, std::memory_order_relaxed);
    }
  }
  hipLaunchKernelGGL((fused_kernel<V, U, L, A, G, P, W, F, T, GR>), grid, block, lds, s, p);
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

/* Tiled kernels: floor(n / tile) full tiles plus one block per `threads`
 * elements of the remainder. */
uint64_t tiled_blocks(uint64_t n, int per_thread, int threads = kBlock) {
  uint64_t tile = (uint64_t)threads * (uint64_t)per_thread;
  return n / tile + ((n % tile) + threads - 1) / threads;
}

unsigned tiled_grid(uint64_t n, int per_thread, int threads = kBlock) {
  return (unsigned)tiled_blocks(n, per_thread, threads);
}

bool tiled_ok(uint64_t n, int per_thread, int threads = kBlock) {
  return tiled_blocks(n, per_thread, threads) <= 0x7fffffffull;
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

/* ------------------------------------------------------------------------
 * Pipelined ZeRO-Offload step: the events of one call and the hooks the
 * host update calls from its pool threads (each makes the caller's device
 * current on that thread before its HIP call).
 * ---------------------------------------------------------------------- */

constexpr int kMaxOffloadPieces = 1024;

/* The events of one call. Each is complete (or its stream synchronized)
 * before the call returns, so none is released while pending. */
struct OffloadEvents {
  hipEvent_t flag = nullptr;
  std::vector<hipEvent_t> piece;

  int create(int pieces) {
    piece.assign((size_t)pieces, nullptr);
    if (hipEventCreateWithFlags(&flag, hipEventDisableTiming) != hipSuccess)
      return fail(ZS_ERR_HIP, "zs_offload_step: hipEventCreate failed%s");
    for (hipEvent_t &ev : piece)
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess)
        return fail(ZS_ERR_HIP, "zs_offload_step: hipEventCreate failed%s");
    return ZS_OK;
  }

  ~OffloadEvents() {
    if (flag) (void)hipEventDestroy(flag);
    for (hipEvent_t ev : piece)
      if (ev) (void)hipEventDestroy(ev);
  }
};

struct OffloadHooks {
  int device = 0;
  const hipEvent_t *ev_piece = nullptr;
  const uint64_t *cuts = nullptr;
  uint16_t *params_dev = nullptr;
  const uint16_t *params_host = nullptr;
  hipStream_t stream = nullptr;
  std::atomic<int> error{0};  /* first HIP error of a hook */

  void note(hipError_t e) {
    int none = 0;
    if (e != hipSuccess) error.compare_exchange_strong(none, (int)e);
  }
};

/* piece k's gradient is in host memory once its event has completed */
int offload_arrived(void *c, int k) {
  OffloadHooks *h = static_cast<OffloadHooks *>(c);
  hipError_t e = hipSetDevice(h->device);
  if (e == hipSuccess) e = hipEventSynchronize(h->ev_piece[k]);
  h->note(e);
  return e == hipSuccess ? 0 : 1;
}

/* piece k's parameters are final: send them back (same stream, so after
 * every gradient piece) */
void offload_updated(void *c, int k) {
  OffloadHooks *h = static_cast<OffloadHooks *>(c);
  const uint64_t lo = h->cuts[k], hi = h->cuts[k + 1];
  if (hi == lo) return;
  hipError_t e = hipSetDevice(h->device);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->params_dev + lo, h->params_host + lo, 2 * (hi - lo),
                       hipMemcpyHostToDevice, h->stream);
  h->note(e);
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
                          int wire_dtype, uint32_t world, uint32_t rank,
                          uint64_t n, float *grad_part, int accumulate,
                          uint32_t *overflow_flag, float loss_scale,
                          void *stream) {
  if (!worker_grads || !grad_part)
    return fail(ZS_ERR_INVALID_ARG, "null worker_grads or grad_part%s");
  if (world == 0 || world > ZS_MAX_WORLD || rank >= world)
    return fail(ZS_ERR_INVALID_ARG, "need 0 < world <= 64 and rank < world%s");
  if (!valid_dtype(grad_dtype)) return fail(ZS_ERR_INVALID_ARG, "bad grad dtype%s");
  if (!valid_wire(wire_dtype)) return fail(ZS_ERR_INVALID_ARG, "bad wire dtype%s");
  if (too_big(n)) return fail(ZS_ERR_UNSUPPORTED, "n exceeds 2^48 elements%s");
  ReduceArgs a;
  a.wire = wire_dtype;
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
  /* A first (non-accumulating) reduction of aligned operands takes four
   * 4-element vectors per thread and stores whole lines non-temporally;
   * measured on MI355X at W = 4: 4 % faster than two 8-element vectors with
   * plain stores, while an accumulating one, which reads its output first,
   * was 3 % slower that way and keeps the plain shape. */
  const bool nt = !accumulate && vec >= 4;
  if (nt) vec = 4;
  const int per_thread = vec * (nt ? 4 : kTileVecs);
  if (!tiled_ok(n, per_thread)) return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(tiled_grid(n, per_thread)), block(kBlock);
#define ZS_REDUCE_K(V, U, D, W, NT) \
  hipLaunchKernelGGL((reduce_kernel<V, U, D, W, NT>), grid, block, 0, s, a)
#define ZS_REDUCE_W(V, U, D, NT)                                          \
  do {                                                                    \
    if (wire_dtype == ZS_WIRE_BF16) ZS_REDUCE_K(V, U, D, ZS_WIRE_BF16, NT);      \
    else if (wire_dtype == ZS_WIRE_FP16) ZS_REDUCE_K(V, U, D, ZS_WIRE_FP16, NT); \
    else ZS_REDUCE_K(V, U, D, ZS_WIRE_FP32, NT);                          \
  } while (0)
#define ZS_LAUNCH_REDUCE(D)                                   \
  do {                                                        \
    if (nt) {                                                 \
      ZS_REDUCE_W(4, 4, D, true);                             \
    } else {                                                  \
      switch (vec) {                                          \
        case 8: ZS_REDUCE_W(8, kTileVecs, D, false); break;   \
        case 4: ZS_REDUCE_W(4, kTileVecs, D, false); break;   \
        case 2: ZS_REDUCE_W(2, kTileVecs, D, false); break;   \
        default: ZS_REDUCE_W(1, kTileVecs, D, false); break;  \
      }                                                       \
    }                                                         \
  } while (0)
  if (grad_dtype == ZS_BF16) ZS_LAUNCH_REDUCE(ZS_BF16);
  else ZS_LAUNCH_REDUCE(ZS_FP16);
#undef ZS_LAUNCH_REDUCE
#undef ZS_REDUCE_W
#undef ZS_REDUCE_K
  return launch_result();
}

int zs_check_overflow(const float *grad_part, uint64_t n, float loss_scale,
                      uint32_t *overflow_flag, void *stream) {
  if (!grad_part || !overflow_flag)
    return fail(ZS_ERR_INVALID_ARG, "null grad_part or overflow_flag%s");
  if (too_big(n)) return fail(ZS_ERR_UNSUPPORTED, "n exceeds 2^48 elements%s");
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
  if (too_big(n)) return fail(ZS_ERR_UNSUPPORTED, "n exceeds 2^48 elements%s");
  AdamArgs p;
  if (!make_scales(1, hp->loss_scale, &p.k))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (const char *bad = zs_host::hparams_problem(hp)) return fail(ZS_ERR_INVALID_ARG, "%s", bad);
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
  if (too_big(n) || too_big(offset))
    return fail(ZS_ERR_UNSUPPORTED, "n or offset exceeds 2^48 elements%s");
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

/* zs_step_fused, with optional start/stop events recorded on the stream
 * immediately before and after the kernel launch; with `dev`, the scale,
 * bias corrections and flag of the device-resident flow (a->hp.loss_scale,
 * a->hp.step_t and a->overflow_flag unused). */
/* clear_first: NULL, or a device word that a one-thread kernel zeroes on
 * `stream` after every check has passed and before the fused kernel (and
 * ev_start), so a refused call enqueues nothing. */
static int step_fused_impl(const zs_step_args *a, void *stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop, zs_device_scaler *dev,
                           uint32_t *clear_first = nullptr) {
  if (!a) return fail(ZS_ERR_INVALID_ARG, "null args%s");
  if (a->state_layout != ZS_STATE_SPLIT && a->state_layout != ZS_STATE_GROUPED)
    return fail(ZS_ERR_INVALID_ARG, "unknown state layout%s");
  const bool grouped = a->state_layout == ZS_STATE_GROUPED;
  if (!a->worker_grads || !a->master_in || !a->master_out || !a->gather_buf ||
      (!a->overflow_flag && !dev))
    return fail(ZS_ERR_INVALID_ARG, "null pointer in zs_step_args%s");
  if (grouped ? (a->m_in || a->v_in || a->m_out || a->v_out)
              : (!a->m_in || !a->v_in || !a->m_out || !a->v_out))
    return fail(ZS_ERR_INVALID_ARG,
                grouped ? "grouped state: m and v pointers must be NULL%s"
                        : "null pointer in zs_step_args%s");
  if (a->world == 0 || a->world > ZS_MAX_WORLD || a->rank >= a->world)
    return fail(ZS_ERR_INVALID_ARG, "need 0 < world <= 64 and rank < world%s");
  if (!valid_dtype(a->grad_dtype) || !valid_dtype(a->param_dtype))
    return fail(ZS_ERR_INVALID_ARG, "bad grad or param dtype%s");
  if (!valid_wire(a->wire_dtype)) return fail(ZS_ERR_INVALID_ARG, "bad wire dtype%s");
  if (too_big(a->n) || too_big(a->gather_offset))
    return fail(ZS_ERR_UNSUPPORTED, "n or gather_offset exceeds 2^48 elements%s");
  FusedArgs p{};
  p.wire = a->wire_dtype;
  zs_adamw_hparams hp = a->hp;
  if (dev) {
    /* placeholders: the kernel replaces the scale and the bias corrections */
    hp.loss_scale = 1.0f;
    hp.step_t = 1;
  }
  if (!make_scales(a->world, hp.loss_scale, &p.k))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (const char *bad = zs_host::hparams_problem(&hp)) return fail(ZS_ERR_INVALID_ARG, "%s", bad);
  if (!make_adam(&hp, &p.h)) return fail(ZS_ERR_INVALID_ARG, "step_t must be >= 1%s");
  p.dev = dev;
  p.lr = (double)a->hp.lr;
  const uint64_t n = a->n;
  if (n == 0) return ZS_OK;
  int rc = fill_ring(a->worker_grads, a->world, a->rank, &p.g);
  if (rc != ZS_OK) return rc;

  uint16_t *param_out = static_cast<uint16_t *>(a->gather_buf) + a->gather_offset;
  /* The output set must not overlap any input (the skip relies on the
   * input set being untouched) nor itself. Null entries (m and v with the
   * grouped layout, no acc_in) take no part. */
  const uint64_t b4 = 4 * n, b2 = 2 * n;
  const uint64_t bs = grouped ? grouped_state_bytes(n) : b4; /* master_in / master_out */
  const void *outs[] = {a->master_out, a->m_out, a->v_out, param_out};
  const uint64_t out_bytes[] = {bs, b4, b4, b2};
  const void *ins[] = {a->master_in, a->m_in, a->v_in, a->acc_in};
  const uint64_t in_bytes[] = {bs, b4, b4, b4};
  for (int i = 0; i < 4; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 4; ++j)
      if (ins[j] && overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return fail(ZS_ERR_ALIAS, "zs_step_fused: an output overlaps an input%s");
    for (uint32_t w = 0; w < a->world; ++w)
      if (overlaps(outs[i], out_bytes[i], p.g.p[w], b2))
        return fail(ZS_ERR_ALIAS, "zs_step_fused: an output overlaps a gradient buffer%s");
    for (int j = i + 1; j < 4; ++j)
      if (outs[j] && overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return fail(ZS_ERR_ALIAS, "zs_step_fused: two outputs overlap%s");
    if (dev && overlaps(outs[i], out_bytes[i], dev, sizeof(zs_device_scaler)))
      return fail(ZS_ERR_ALIAS, "zs_step_device: an output overlaps the device scaler%s");
  }
  /* The fused pass and the commit kernel write the device scaler while
   * other blocks still read the input set; a scaler inside an input would
   * corrupt the set a skipped step restores from. */
  if (dev) {
    for (int j = 0; j < 4; ++j)
      if (ins[j] && overlaps(dev, sizeof(zs_device_scaler), ins[j], in_bytes[j]))
        return fail(ZS_ERR_ALIAS, "zs_step_device: the device scaler overlaps an input%s");
    for (uint32_t w = 0; w < a->world; ++w)
      if (overlaps(dev, sizeof(zs_device_scaler), p.g.p[w], b2))
        return fail(ZS_ERR_ALIAS,
                    "zs_step_device: the device scaler overlaps a gradient buffer%s");
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
  p.flag = dev ? nullptr : a->overflow_flag;  /* the device flow marks dev->flag_epoch */

  const void *p16[ZS_MAX_WORLD + 1];
  for (uint32_t w = 0; w < a->world; ++w) p16[w] = p.g.p[w];
  p16[a->world] = param_out;
  const void *f32[] = {a->master_in, a->m_in, a->v_in, a->master_out, a->m_out,
                       a->v_out, a->acc_in ? a->acc_in : a->master_in};
  const int vec = fused_vec_of(pick_vec(p16, (int)a->world + 1, f32, 7));
  const bool multi = a->world > 1, acc = a->acc_in != nullptr;
  if (grouped && vec != 4)
    return fail(ZS_ERR_UNSUPPORTED,
                "grouped state needs operands aligned for 4-element vectors%s");
  FusedShape fs = grouped ? fused_shape_grouped(a->world) : fused_shape(vec, a->world, n);
  if (fs.access == kShapeR4NtL && env_batched_sum()) fs.access = kShapeB8NtL;
  const WriteWindow win = write_window(fs, a->world, n, acc);
  p.win_period = win.period;
  p.win_open = win.open_at;
  if (win.period) fs.cap = 0;
  const int per_thread = vec * fs.tile_vecs;
  if (!tiled_ok(n, per_thread, fs.threads))
    return fail(ZS_ERR_UNSUPPORTED, "n too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(tiled_grid(n, per_thread, fs.threads)), block(fs.threads);
  const size_t lds = fused_lds_bytes(fs.cap);
#define ZS_KF(V, U, L, A, G, P, W, S, T) \
  launch_fused<V, U, L, A, G, P, W, S, T, false>(grid, block, lds, s, p)
#define ZS_KG(U, L, A, G, P, W, S) \
  launch_fused<4, U, L, A, G, P, W, S, kFusedWaveBlock, true>(grid, block, lds, s, p)
#define ZS_K4(V, A, G, P, W)                                                             \
  do {                                                                                   \
    if (grouped) {                                                                       \
      if (!multi) ZS_KG(1, false, A, G, P, W, kShapeB8NtL);                              \
      else if (fs.tile_vecs == 1) ZS_KG(1, true, A, G, P, W, kShapeB8NtL);               \
      else if (fs.access == kShapeR4NtL) ZS_KG(2, true, A, G, P, W, kShapeR4NtL);        \
      else ZS_KG(2, true, A, G, P, W, kShapeB8NtL);                                      \
    } else if (!multi && fs.threads == kFusedWaveBlock)                                  \
      ZS_KF(4, 1, false, A, G, P, W, kShapeB8NtL, kFusedWaveBlock);                      \
    else if (!multi) ZS_KF(4, 2, false, A, G, P, W, kShapeB8NtL, kBlock);                \
    else if (fs.threads == kFusedWaveBlock && fs.tile_vecs == 1)                         \
      ZS_KF(4, 1, true, A, G, P, W, kShapeB8NtL, kFusedWaveBlock);                       \
    else if (fs.threads == kFusedWaveBlock && fs.access == kShapeR4NtL)                  \
      ZS_KF(4, 2, true, A, G, P, W, kShapeR4NtL, kFusedWaveBlock);                       \
    else if (fs.threads == kFusedWaveBlock) ZS_KF(4, 2, true, A, G, P, W, kShapeB8NtL,   \
                                                  kFusedWaveBlock);                      \
    else ZS_KF(4, 2, true, A, G, P, W, kShapeB8NtL, kBlock);                             \
  } while (0)
#define ZS_KNARROW(V, A, G, P, W)                                   \
  do {                                                              \
    if (!multi) ZS_KF(V, 1, false, A, G, P, W, kShapeB8, kBlock);   \
    else ZS_KF(V, 2, true, A, G, P, W, kShapeB8, kBlock);           \
  } while (0)
#define ZS_KWIRE(KM, V, A, G, P)                                   \
  do {                                                             \
    if (p.wire == ZS_WIRE_BF16) KM(V, A, G, P, ZS_WIRE_BF16);      \
    else if (p.wire == ZS_WIRE_FP16) KM(V, A, G, P, ZS_WIRE_FP16); \
    else KM(V, A, G, P, ZS_WIRE_FP32);                             \
  } while (0)
#define ZS_KACC(KM, V, G, P)                        \
  do {                                              \
    if (acc) ZS_KWIRE(KM, V, true, G, P);           \
    else ZS_KWIRE(KM, V, false, G, P);              \
  } while (0)
#define ZS_FUSED_VEC(G, P)                              \
  switch (vec) {                                        \
    case 4: ZS_KACC(ZS_K4, 4, G, P); break;             \
    case 2: ZS_KACC(ZS_KNARROW, 2, G, P); break;        \
    default: ZS_KACC(ZS_KNARROW, 1, G, P); break;       \
  }
  if (clear_first) {
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, s, clear_first);
    int rc = launch_result();
    if (rc != ZS_OK) return rc;
  }
  if (ev_start) {
    hipError_t e = hipEventRecord(ev_start, s);
    if (e != hipSuccess) return fail(ZS_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
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
#undef ZS_KACC
#undef ZS_KWIRE
#undef ZS_KNARROW
#undef ZS_K4
#undef ZS_KG
#undef ZS_KF
  int launched = launch_result();
  if (launched == ZS_OK && ev_stop) {
    hipError_t e = hipEventRecord(ev_stop, s);
    if (e != hipSuccess) return fail(ZS_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  }
  return launched;
}

/* The commit-or-skip step of zs_step_commit and zs_step_commit_noalloc:
 * the fused pass with `flag` (device memory; zeroed first on the stream when
 * clear is true) as its overflow word, the word's readback to host_flag, and
 * the scaler rule. */
static int step_commit_impl(const zs_step_args *a, uint32_t *flag, bool clear,
                            zs_loss_scaler *scaler, uint32_t *host_flag, hipStream_t s,
                            hipEvent_t ev_start, hipEvent_t ev_stop, int *committed) {
  if (!(scaler->scale > 0.0f) || !isfinite(scaler->scale))
    return fail(ZS_ERR_INVALID_ARG, "scaler->scale must be finite and > 0%s");
  if (scaler->step_t >= 0xffffffffull)
    return fail(ZS_ERR_UNSUPPORTED, "step count exceeds 32 bits%s");
  zs_step_args local = *a;
  local.hp.loss_scale = scaler->scale;
  local.hp.step_t = (uint32_t)(scaler->step_t + 1);
  local.overflow_flag = flag;
  int rc = step_fused_impl(&local, s, ev_start, ev_stop, nullptr, clear ? flag : nullptr);
  if (rc != ZS_OK) return rc;
  if (a->n == 0) {
    *committed = 1;
    return zs_scaler_update(scaler, 0);
  }
  /* The flag is only ever 0 or 1, so a sentinel in host memory shows when
   * the 4-byte copy (stream-ordered after the kernel) has landed: the call
   * spins on that word, which returns sooner than a blocking stream
   * synchronization, and queries the stream once per kQueryMicros so that
   * a failed stream ends the wait with an error instead of a hang. */
  volatile uint32_t *hf = host_flag;
  const uint32_t kSentinel = 0xffffffffu;
  *hf = kSentinel;
  hipError_t e = hipMemcpyAsync(host_flag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return fail(ZS_ERR_HIP, "flag readback failed: %s", hipGetErrorString(e));
  auto last = std::chrono::steady_clock::now();
  const auto every = std::chrono::microseconds(kQueryMicros);
  for (uint32_t spins = 1; *hf == kSentinel; ++spins) {
    if ((spins & 1023u) != 0) continue;
    auto now = std::chrono::steady_clock::now();
    if (now - last < every) continue;
    last = now;
    hipError_t q = hipStreamQuery(s);
    if (q == hipErrorNotReady) continue;
    if (q != hipSuccess)
      return fail(ZS_ERR_HIP, "stream failed before the flag arrived: %s", hipGetErrorString(q));
    if (*hf == kSentinel) return fail(ZS_ERR_HIP, "flag readback did not arrive%s");
  }
  uint32_t got = *hf;
  *committed = got == 0;
  return zs_scaler_update(scaler, got);
}

int zs_step_fused(const zs_step_args *a, void *stream) {
  return step_fused_impl(a, stream, nullptr, nullptr, nullptr);
}

int zs_device_scaler_make(const zs_loss_scaler *s, float beta1, float beta2,
                          zs_device_scaler *out) {
  if (!s || !out) return fail(ZS_ERR_INVALID_ARG, "null scaler or output%s");
  if (!(s->scale > 0.0f) || !isfinite(s->scale))
    return fail(ZS_ERR_INVALID_ARG, "scale must be finite and > 0%s");
  if (!zs_host::beta_ok(beta1) || !zs_host::beta_ok(beta2))
    return fail(ZS_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)%s");
  zs_device_scaler d;
  memset(&d, 0, sizeof d);
  d.scale = s->scale;
  d.clean_steps = s->clean_steps;
  d.growth_interval = s->growth_interval;
  d.dynamic = s->dynamic;
  d.step_t = s->step_t;
  d.skipped = s->skipped;
  /* beta^(t+1) by t+1 repeated multiplications, as make_adam forms it */
  double b1t, b2t;
  zs_host::beta_powers(beta1, beta2, s->step_t + 1, &b1t, &b2t);
  d.beta1_t = b1t;
  d.beta2_t = b2t;
  *out = d;
  g_err[0] = 0;
  return ZS_OK;
}

int zs_step_device(const zs_step_args *a, zs_device_scaler *dev, void *stream, void *ev_start,
                   void *ev_stop) {
  if (!dev || (uintptr_t)dev % alignof(zs_device_scaler) != 0)
    return fail(ZS_ERR_INVALID_ARG, "device scaler must be non-null and 8-byte aligned%s");
  int rc = step_fused_impl(a, stream, static_cast<hipEvent_t>(ev_start),
                           static_cast<hipEvent_t>(ev_stop), dev);
  if (rc != ZS_OK) return rc;
  CommitArgs c;
  c.dev = dev;
  c.master_in = a->master_in;
  c.m_in = a->m_in;
  c.v_in = a->v_in;
  c.master_out = a->master_out;
  c.m_out = a->m_out;
  c.v_out = a->v_out;
  c.param_out = static_cast<uint16_t *>(a->gather_buf) + a->gather_offset;
  c.n = a->n;
  c.beta1 = (double)a->hp.beta1;
  c.beta2 = (double)a->hp.beta2;
  const void *p16[] = {c.param_out};
  const void *f32[] = {c.master_in, c.m_in, c.v_in, c.master_out, c.m_out, c.v_out};
  const int vec = pick_vec(p16, 1, f32, 6);
  /* a few large blocks: they only copy on a skipped step (grid-stride) */
  const uint64_t per_block = (uint64_t)kCommitBlock * (uint64_t)vec;
  const uint64_t want = (a->n + per_block - 1) / per_block;
  const unsigned blocks =
      (unsigned)(want < 1 ? 1 : (want > (uint64_t)kCommitBlocks ? kCommitBlocks : want));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool grouped = a->state_layout == ZS_STATE_GROUPED;
#define ZS_COMMIT_K(V, P)                                                                   \
  do {                                                                                      \
    if (grouped)                                                                            \
      hipLaunchKernelGGL((commit_kernel<V, P, true>), dim3(blocks), dim3(kCommitBlock), 0, s, c); \
    else                                                                                    \
      hipLaunchKernelGGL((commit_kernel<V, P, false>), dim3(blocks), dim3(kCommitBlock), 0, s, c); \
  } while (0)
#define ZS_COMMIT_VEC(P)                      \
  switch (vec) {                              \
    case 8: ZS_COMMIT_K(8, P); break;         \
    case 4: ZS_COMMIT_K(4, P); break;         \
    case 2: ZS_COMMIT_K(2, P); break;         \
    default: ZS_COMMIT_K(1, P); break;        \
  }
  if (a->param_dtype == ZS_BF16) {
    ZS_COMMIT_VEC(ZS_BF16)
  } else {
    ZS_COMMIT_VEC(ZS_FP16)
  }
#undef ZS_COMMIT_VEC
#undef ZS_COMMIT_K
  return launch_result();
}

int zs_step_commit(const zs_step_args *a, zs_loss_scaler *scaler, uint32_t *host_flag,
                   void *stream, void *ev_start, void *ev_stop, int *committed) {
  if (!a || !scaler || !host_flag || !committed)
    return fail(ZS_ERR_INVALID_ARG, "null args, scaler, host_flag or committed%s");
  return step_commit_impl(a, a->overflow_flag, false, scaler, host_flag,
                          static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_start),
                          static_cast<hipEvent_t>(ev_stop), committed);
}

int zs_step_commit_noalloc(const zs_step_args *a, zs_loss_scaler *scaler, uint32_t *host_flag,
                           void *stream, void *ev_start, void *ev_stop, int *committed) {
  if (!a || !scaler || !host_flag || !committed)
    return fail(ZS_ERR_INVALID_ARG, "null args, scaler, host_flag or committed%s");
  uint32_t *word = nullptr;
  int rc = scratch_word(&word);
  if (rc != ZS_OK) return rc;
  return step_commit_impl(a, word, true, scaler, host_flag, static_cast<hipStream_t>(stream),
                          static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop),
                          committed);
}

int zs_all_gather_step(void *const *replicas, uint32_t world, uint64_t phi, uint32_t sigma,
                       uint32_t step, void *stream) {
  if (!replicas) return fail(ZS_ERR_INVALID_ARG, "null replicas%s");
  if (world == 0 || world > ZS_MAX_WORLD)
    return fail(ZS_ERR_INVALID_ARG, "need 0 < world <= 64%s");
  if (sigma >= world || step == 0 || step >= world)
    return fail(ZS_ERR_INVALID_ARG, "need sigma < world and 1 <= step < world%s");
  if (too_big(phi)) return fail(ZS_ERR_UNSUPPORTED, "phi exceeds 2^48 elements%s");
  GatherArgs g;
  for (uint32_t k = 0; k < world; ++k) {
    if (!replicas[k]) return fail(ZS_ERR_INVALID_ARG, "replicas has a null pointer%s");
    g.r[k] = static_cast<uint16_t *>(replicas[k]);
  }
  for (uint32_t k = world; k < ZS_MAX_WORLD; ++k) g.r[k] = nullptr;
  for (uint32_t i = 0; i < world; ++i)
    for (uint32_t j = i + 1; j < world; ++j)
      if (overlaps(g.r[i], 2 * phi, g.r[j], 2 * phi))
        return fail(ZS_ERR_ALIAS, "zs_all_gather_step: replicas overlap%s");
  g.world = world;
  g.sigma = sigma;
  g.step = step;
  g.phi = phi;
  g.chunk = phi / world + (phi % world != 0);
  if (phi == 0) return ZS_OK;
  /* 16-byte copies need every replica 16-byte aligned and chunk starts at
   * multiples of 8 elements. */
  bool wide = g.chunk % 8 == 0;
  for (uint32_t k = 0; k < world && wide; ++k) wide = ((uintptr_t)g.r[k] % 16) == 0;
  const int vec = wide ? 8 : 1;
  const uint64_t blocks = (g.chunk + (uint64_t)kBlock * vec - 1) / ((uint64_t)kBlock * vec);
  if (blocks > 0x7fffffffull) return fail(ZS_ERR_UNSUPPORTED, "chunk too large for one launch%s");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)blocks, world), block(kBlock);
  if (wide) hipLaunchKernelGGL(gather_step_kernel<8>, grid, block, 0, s, g);
  else hipLaunchKernelGGL(gather_step_kernel<1>, grid, block, 0, s, g);
  return launch_result();
}

int zs_offload_step(const float *grad_dev, float *grad_host, float *master, float *m, float *v,
                    void *params_host, void *params_dev, uint64_t n, const zs_adamw_hparams *hp,
                    int param_dtype, uint32_t *flag_dev, uint32_t *flag_host, int threads,
                    int pieces, void *stream, int *committed) {
  if (!grad_dev || !grad_host || !master || !m || !v || !params_host || !params_dev || !hp ||
      !flag_dev || !flag_host || !committed)
    return fail(ZS_ERR_INVALID_ARG, "zs_offload_step: null pointer%s");
  if (!valid_dtype(param_dtype)) return fail(ZS_ERR_INVALID_ARG, "bad param dtype%s");
  if (too_big(n)) return fail(ZS_ERR_UNSUPPORTED, "n exceeds 2^48 elements%s");
  if (pieces < 1 || pieces > kMaxOffloadPieces)
    return fail(ZS_ERR_INVALID_ARG, "pieces must lie in [1, 1024]%s");
  if (!(hp->loss_scale > 0.0f) || !isfinite(hp->loss_scale))
    return fail(ZS_ERR_INVALID_ARG, "loss_scale must be finite and > 0%s");
  if (hp->step_t == 0) return fail(ZS_ERR_INVALID_ARG, "step_t must be >= 1%s");
  if (const char *bad = zs_host::hparams_problem(hp)) return fail(ZS_ERR_INVALID_ARG, "%s", bad);
  {
    const void *host[] = {grad_host, master, m, v, params_host};
    const uint64_t bytes[] = {4 * n, 4 * n, 4 * n, 4 * n, 2 * n};
    for (int i = 0; i < 5; ++i)
      for (int j = i + 1; j < 5; ++j)
        if (overlaps(host[i], bytes[i], host[j], bytes[j]))
          return fail(ZS_ERR_INVALID_ARG, "zs_offload_step: host buffers overlap%s");
  }
  *committed = 0;
  if (n == 0) {
    *committed = 1;
    g_err[0] = 0;
    return ZS_OK;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  OffloadEvents ev;
  int rc = ev.create(pieces);
  if (rc != ZS_OK) return rc;
  /* the check, then the flag to the host */
  hipError_t e = hipMemsetAsync(flag_dev, 0, sizeof(uint32_t), s);
  if (e != hipSuccess) return fail(ZS_ERR_HIP, "zs_offload_step: %s", hipGetErrorString(e));
  rc = zs_check_overflow(grad_dev, n, hp->loss_scale, flag_dev, stream);
  if (rc != ZS_OK) return rc;
  e = hipMemcpyAsync(flag_host, flag_dev, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipEventRecord(ev.flag, s);
  if (e == hipSuccess) e = hipEventSynchronize(ev.flag);
  if (e != hipSuccess) return fail(ZS_ERR_HIP, "zs_offload_step: %s", hipGetErrorString(e));
  if (*static_cast<volatile uint32_t *>(flag_host) != 0) {
    g_err[0] = 0;
    return ZS_OK;  /* skipped: nothing copied or written */
  }
  /* the gradient in pieces, each announced by its event; the parameter
   * copies that the host update enqueues follow on the same stream */
  std::vector<uint64_t> cuts((size_t)pieces + 1);
  for (int k = 0; k < pieces; ++k) cuts[(size_t)k] = n * (uint64_t)k / (uint64_t)pieces / 64 * 64;
  cuts[(size_t)pieces] = n;
  for (int k = 0; k < pieces && e == hipSuccess; ++k) {
    const uint64_t lo = cuts[(size_t)k], hi = cuts[(size_t)k + 1];
    if (hi > lo)
      e = hipMemcpyAsync(grad_host + lo, grad_dev + lo, 4 * (hi - lo), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(ev.piece[(size_t)k], s);
  }
  if (e != hipSuccess) {
    /* wait for what was enqueued before the events are released */
    (void)hipStreamSynchronize(s);
    return fail(ZS_ERR_HIP, "zs_offload_step: %s", hipGetErrorString(e));
  }
  OffloadHooks ctx;
  ctx.ev_piece = ev.piece.data();
  ctx.cuts = cuts.data();
  ctx.params_dev = static_cast<uint16_t *>(params_dev);
  ctx.params_host = static_cast<const uint16_t *>(params_host);
  ctx.stream = s;
  if (hipGetDevice(&ctx.device) != hipSuccess) ctx.device = 0;
  zs_host::PieceHooks hooks{&ctx, &offload_arrived, &offload_updated};
  rc = zs_host::update_in_pieces(master, m, v, grad_host, n, hp, params_host, param_dtype,
                                 threads, cuts.data(), pieces, hooks);
  const int herr = ctx.error.load();
  if (herr != 0 || rc != ZS_OK) {
    (void)hipStreamSynchronize(s);
    if (herr != 0)
      return fail(ZS_ERR_HIP, "zs_offload_step: %s", hipGetErrorString((hipError_t)herr));
    return fail(rc, "zs_offload_step: the host update refused its arguments%s");
  }
  *committed = 1;
  g_err[0] = 0;
  return ZS_OK;
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
