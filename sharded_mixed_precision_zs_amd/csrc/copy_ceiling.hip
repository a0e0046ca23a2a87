/*
 * copy_ceiling.hip -- libzscopy: measurement kernels that the benchmark times
 * beside the shard step, as the practical HBM ceilings of the part it runs
 * on. Measurement only: no step of the method runs here, and the shard-step
 * library does not use it.
 *
 * zs_copy_ceiling: every lane moves one 16-byte vector (a non-temporal load,
 * then a plain store), so each 64-lane wave reads 1 KB and writes 1 KB. On
 * MI355X copies with 1-2 KB per wave streamed fastest (about 6.45 TB/s for
 * read plus write); wider bursts per wave and persistent grids were slower,
 * and the runtime's device-to-device memcpy reaches 4.6-5.2 TB/s.
 * zs_copy_shape runs the same copy in the other shapes of a small catalogue
 * (vectors per lane, vector width, non-temporal loads and stores, block
 * size, persistent grids, residency caps), so the benchmark can show which
 * read-plus-write rate any copy shape reaches on the part.
 *
 * zs_wave_probe: the shard step's streams in the fused kernel's present
 * access shape (one-wave blocks, 4-element vectors, non-temporal loads and
 * stores, four 16-bit loads in flight, the grouped fp32 state, the same
 * residency caps and write windows), with the arithmetic replaced by
 * integer folds, for any mix of 16-bit input streams (the W gradients), an
 * fp32 input and output state (master / m / v) and a 16-bit output stream
 * (the parameters). With no outputs it is a read-only stream, with no
 * inputs a write-only one, and with the step's streams it gives the rate of
 * that exact mix of reads and writes without the arithmetic.
 *
 * zs_stream_probe: the same idea in an earlier shape of the fused kernel
 * (256-thread blocks, 8-element vectors, batches of eight 16-bit loads,
 * plain stores, three separate fp32 arrays), kept for the phase sweep that
 * separates a shard's reads from its writes in time.
 */
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kCopyBlock = 256;

thread_local const char *g_copy_err = "";

using f4 = float __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kCopyBlock)
copy_kernel(const f4 *__restrict__ src, f4 *__restrict__ dst, uint64_t nvec) {
  const uint64_t i = (uint64_t)blockIdx.x * kCopyBlock + threadIdx.x;
  if (i < nvec) dst[i] = __builtin_nontemporal_load(src + i);
}

/* ------------------------------------------------------------------------
 * Stream probe. Thread t of block b owns kProbeVecs-element vectors u < U at
 * element ((b * U + u) * kCopyBlock + t) * 8: the fused step's tile. Per
 * vector, in the fused step's order:
 *   - the 16-bit inputs, one non-temporal 16-byte load per stream: stream
 *     0, then batches of kProbeBatch streams loaded ahead of their use,
 *     folded by integer adds;
 *   - the fp32 inputs, two 16-byte loads each: after the 16-bit inputs when
 *     there are several of them, before the single one otherwise;
 *   - fp32 output k = fp32 input k XOR the fold (the fold alone when there
 *     is no input k), the 16-bit output = the fold XOR every fp32 input that
 *     no fp32 output carries.
 * Loads that no output carries are kept live by a store of `magic` to
 * `sink` taken only when the folded values equal it (a data-dependent
 * branch the compiler cannot remove; with random inputs it is practically
 * never taken).
 * ---------------------------------------------------------------------- */

constexpr int kProbeMaxIn16 = 64;
constexpr int kProbeBatch = 8;   /* 16-bit loads in flight per thread */

using u4 = uint32_t __attribute__((ext_vector_type(4)));

struct ProbeArgs {
  const u4 *in16[kProbeMaxIn16];
  uint32_t n_in16;
  const u4 *in32[3];
  u4 *out32[3];
  u4 *out16;
  uint32_t *sink;
  uint32_t magic;
};

template <int U, bool MULTI, int NIN, int NOUT, bool P16>
__global__ void __launch_bounds__(kCopyBlock) stream_probe(ProbeArgs a) {
  /* in 16-byte units: a 16-bit vector of 8 elements is one unit, an fp32
   * vector two */
  uint64_t v16[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    v16[u] = ((uint64_t)blockIdx.x * U + u) * kCopyBlock + threadIdx.x;
  u4 fold[U], st[U][3][2];
  auto load_state = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < NIN; ++k) {
        st[u][k][0] = a.in32[k][2 * v16[u]];
        st[u][k][1] = a.in32[k][2 * v16[u] + 1];
      }
  };
  if constexpr (!MULTI) load_state();
  /* stream 0 first, then batches from stream 1, as the fused step's sum */
#pragma unroll
  for (int u = 0; u < U; ++u)
    fold[u] = a.n_in16 ? __builtin_nontemporal_load(a.in16[0] + v16[u]) : u4{0u, 0u, 0u, 0u};
  uint32_t j = 1;
  for (; j + kProbeBatch <= a.n_in16; j += kProbeBatch) {
    u4 r[kProbeBatch][U];
#pragma unroll
    for (int b = 0; b < kProbeBatch; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) r[b][u] = __builtin_nontemporal_load(a.in16[j + b] + v16[u]);
#pragma unroll
    for (int b = 0; b < kProbeBatch; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) fold[u] += r[b][u];
  }
  for (; j < a.n_in16; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) fold[u] += __builtin_nontemporal_load(a.in16[j] + v16[u]);
  if constexpr (MULTI) load_state();
  bool hit = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int k = 0; k < NOUT; ++k) {
      const u4 x0 = k < NIN ? st[u][k][0] ^ fold[u] : fold[u];
      const u4 x1 = k < NIN ? st[u][k][1] ^ fold[u] : fold[u];
      a.out32[k][2 * v16[u]] = x0;
      a.out32[k][2 * v16[u] + 1] = x1;
    }
    /* inputs no fp32 output carries go into the 16-bit output or the sink */
    u4 rest = fold[u];
#pragma unroll
    for (int k = NOUT; k < NIN; ++k) rest ^= st[u][k][0] ^ st[u][k][1];
    if constexpr (P16) a.out16[v16[u]] = rest;
    if constexpr (!P16 && (NOUT == 0 || NIN > NOUT))
      hit |= (rest.x ^ rest.y ^ rest.z ^ rest.w) == a.magic;
  }
  if constexpr (!P16 && (NOUT == 0 || NIN > NOUT))
    if (hit) *a.sink = a.magic;
}

/* Dynamic LDS (never touched) that caps residency at `cap` blocks per CU,
 * as the fused step's launch does; 0 = no cap. */
size_t probe_lds_bytes(uint32_t cap, int *lds_per_cu) {
  *lds_per_cu = 0;
  if (cap == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                            dev) != hipSuccess)
    return 0;
  const int bytes = (*lds_per_cu / (int)cap - 1024) / 256 * 256;
  return bytes > 0 ? (size_t)bytes : 0;
}

template <int U, bool M, int NIN, int NOUT, bool P16>
hipError_t launch_probe(unsigned blocks, size_t lds, int lds_per_cu, hipStream_t s,
                        const ProbeArgs &a) {
  const void *fn = reinterpret_cast<const void *>(&stream_probe<U, M, NIN, NOUT, P16>);
  if (lds > 65536) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_per_cu);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((stream_probe<U, M, NIN, NOUT, P16>), dim3(blocks), dim3(kCopyBlock), lds,
                     s, a);
  return hipGetLastError();
}

template <int U, int NIN, int NOUT>
hipError_t launch_probe_p(bool p16, unsigned blocks, size_t lds, int lds_per_cu, hipStream_t s,
                          const ProbeArgs &a) {
  const bool m = a.n_in16 > 1;
  if (p16)
    return m ? launch_probe<U, true, NIN, NOUT, true>(blocks, lds, lds_per_cu, s, a)
             : launch_probe<U, false, NIN, NOUT, true>(blocks, lds, lds_per_cu, s, a);
  return m ? launch_probe<U, true, NIN, NOUT, false>(blocks, lds, lds_per_cu, s, a)
           : launch_probe<U, false, NIN, NOUT, false>(blocks, lds, lds_per_cu, s, a);
}

template <int U, int NIN>
hipError_t launch_probe_o(uint32_t nout, bool p16, unsigned blocks, size_t lds, int lds_per_cu,
                          hipStream_t s, const ProbeArgs &a) {
  switch (nout) {
    case 0: return launch_probe_p<U, NIN, 0>(p16, blocks, lds, lds_per_cu, s, a);
    case 1: return launch_probe_p<U, NIN, 1>(p16, blocks, lds, lds_per_cu, s, a);
    default: return launch_probe_p<U, NIN, 3>(p16, blocks, lds, lds_per_cu, s, a);
  }
}

template <int U>
hipError_t launch_probe_i(uint32_t nin, uint32_t nout, bool p16, unsigned blocks, size_t lds,
                          int lds_per_cu, hipStream_t s, const ProbeArgs &a) {
  switch (nin) {
    case 0: return launch_probe_o<U, 0>(nout, p16, blocks, lds, lds_per_cu, s, a);
    case 1: return launch_probe_o<U, 1>(nout, p16, blocks, lds, lds_per_cu, s, a);
    default: return launch_probe_o<U, 3>(nout, p16, blocks, lds, lds_per_cu, s, a);
  }
}

bool span_overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

/* ------------------------------------------------------------------------
 * Copy shapes. Lane t of block b moves U vectors of VB bytes (8 or 16):
 * vector u at vector index (b * U + u) * T + t, so each vector of a wave
 * covers whole lines; loads and stores are optionally non-temporal.
 * PERSIST blocks walk the tiles with a grid stride; the others take one
 * tile each (the grid is the tile count).
 * ---------------------------------------------------------------------- */
using u2 = uint32_t __attribute__((ext_vector_type(2)));
template <int VB> struct CopyVec { using T = u4; };
template <> struct CopyVec<8> { using T = u2; };

template <int T, int U, int VB, bool NTL, bool NTS, bool PERSIST>
__global__ void __launch_bounds__(T)
copy_shape_kernel(const void *__restrict__ src, void *__restrict__ dst, uint64_t tiles) {
  using V = typename CopyVec<VB>::T;
  const V *s = static_cast<const V *>(src);
  V *d = static_cast<V *>(dst);
  const uint64_t stride = PERSIST ? (uint64_t)gridDim.x : tiles;
  for (uint64_t tile = blockIdx.x; tile < tiles; tile += stride) {
    V r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t i = (tile * U + u) * T + threadIdx.x;
      if constexpr (NTL) r[u] = __builtin_nontemporal_load(s + i);
      else r[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t i = (tile * U + u) * T + threadIdx.x;
      if constexpr (NTS) __builtin_nontemporal_store(r[u], d + i);
      else d[i] = r[u];
    }
  }
}

struct CopyShape {
  const char *name;
  const void *fn;
  int threads, vecs, vec_bytes;
  bool persistent;
};

template <int T, int U, int VB, bool NTL, bool NTS, bool P>
constexpr CopyShape mk_copy(const char *name) {
  return CopyShape{name, reinterpret_cast<const void *>(&copy_shape_kernel<T, U, VB, NTL, NTS, P>),
                   T, U, VB, P};
}

const CopyShape kCopyShapes[] = {
    mk_copy<256, 1, 16, true, false, false>("16 B per lane, nt load, plain store (the ceiling copy)"),
    mk_copy<256, 1, 16, false, false, false>("16 B per lane, plain load and store"),
    mk_copy<256, 1, 16, true, true, false>("16 B per lane, nt load and store"),
    mk_copy<256, 1, 16, false, true, false>("16 B per lane, plain load, nt store"),
    mk_copy<256, 1, 8, true, false, false>("8 B per lane, nt load, plain store"),
    mk_copy<256, 2, 16, true, false, false>("2 x 16 B per lane, nt load, plain store"),
    mk_copy<256, 4, 16, true, false, false>("4 x 16 B per lane, nt load, plain store"),
    mk_copy<256, 2, 16, true, true, false>("2 x 16 B per lane, nt load and store"),
    mk_copy<64, 1, 16, true, false, false>("16 B per lane, 64-thread blocks"),
    mk_copy<1024, 1, 16, true, false, false>("16 B per lane, 1024-thread blocks"),
    mk_copy<256, 1, 16, true, false, true>("16 B per lane, persistent grid"),
    mk_copy<256, 4, 16, true, false, true>("4 x 16 B per lane, persistent grid"),
};
constexpr int kCopyShapeCount = (int)(sizeof kCopyShapes / sizeof kCopyShapes[0]);

/* ------------------------------------------------------------------------
 * Wave probe: the shard step's streams in the fused kernel's present access
 * shape, with integer folds in place of the arithmetic. One-wave blocks;
 * thread t of block b owns the 4-element vectors at elements
 * e = (b * U + u) * 256 + 4t, u < U. Per vector:
 *   - each 16-bit input stream is one non-temporal 8-byte load, folded in
 *     stream order as two 32-bit words (fold = rotl(fold, 1) + words, see
 *     wave_fold). With more than four streams four loads
 *     stay in flight: the first four are issued together, every add is
 *     followed by the load four streams ahead, and the streams left after
 *     the last full round are loaded with the state; with four or fewer all
 *     are loaded, then added;
 *   - the fp32 input state, in 1024-element groups of three arrays (the
 *     grouped state layout), is one non-temporal 16-byte load per array:
 *     issued first when there is at most one 16-bit stream, else together
 *     with the last 16-bit loads;
 *   - every output value is formed before the first store: base = the fold
 *     XOR (low 32 bits of e, magic); each output state array = the input
 *     array XOR (base, base), or (base, base) with no input state; the
 *     16-bit output = base, XOR the input state's words folded to 8 bytes
 *     when no output state carries them;
 *   - with write windows, the wave then waits until the wall clock's phase
 *     in the period reaches the open part, as the fused kernel's rolling
 *     shape does; all stores are non-temporal.
 * A probe whose loads reach no output stores `magic` to `sink` when the
 * folded words equal it (a data-dependent branch the compiler keeps).
 * ---------------------------------------------------------------------- */
constexpr int kWaveBlock = 64;
constexpr uint64_t kWaveGroup = 1024;
constexpr int kWaveAhead = 4;

struct WaveArgs {
  const u2 *in16[kProbeMaxIn16];
  uint32_t n_in16;
  const u4 *state_in;
  u4 *state_out;
  u2 *out16;
  uint32_t *sink;
  uint32_t magic;
  uint32_t win_period, win_open;   /* wall-clock ticks; period 0: no windows */
};

/* One step of the 16-bit streams' fold: the running fold rotated left by
 * one bit, plus the stream's words. Unlike a plain sum the compiler cannot
 * reassociate it, so, as in the fused kernel's fp32 sum, each add waits for
 * its own stream's load only. */
__device__ __forceinline__ u2 wave_fold(u2 s, u2 x) { return ((s << 1u) | (s >> 31u)) + x; }

/* The last round of the rolling sum: the R (< 4) streams left after the
 * last full refill are loaded together with the state, then everything in
 * flight is added. Picked by wave_tail_pick so that every load count is
 * fixed at compile time: the compiler then waits for exactly the load an
 * add needs (a run-time guard on the loads would make it wait for all). */
template <int U, int R, typename F>
__device__ __forceinline__ void wave_tail(const WaveArgs &a, uint32_t j, const uint64_t (&v)[U],
                                          u2 (&r)[kWaveAhead][U], u2 (&sum)[U], F &state) {
  u2 t[R > 0 ? R : 1][U];
#pragma unroll
  for (int b = 0; b < R; ++b)
#pragma unroll
    for (int u = 0; u < U; ++u) t[b][u] = __builtin_nontemporal_load(a.in16[j + kWaveAhead + b] + v[u]);
  state();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < kWaveAhead; ++b) {
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = wave_fold(sum[u], r[b][u]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int b = 0; b < R; ++b) {
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = wave_fold(sum[u], t[b][u]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int U, int R, typename F>
__device__ __forceinline__ void wave_tail_pick(const WaveArgs &a, uint32_t j,
                                               const uint64_t (&v)[U], u2 (&r)[kWaveAhead][U],
                                               u2 (&sum)[U], F &state, uint32_t left) {
  if constexpr (R == 0) {
    wave_tail<U, 0>(a, j, v, r, sum, state);
  } else {
    if (left == (uint32_t)R) wave_tail<U, R>(a, j, v, r, sum, state);
    else wave_tail_pick<U, R - 1>(a, j, v, r, sum, state, left);
  }
}

template <int U, bool SIN, bool SOUT, bool P16>
__global__ void __launch_bounds__(kWaveBlock) wave_probe(WaveArgs a) {
  uint64_t e[U], v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    e[u] = ((uint64_t)blockIdx.x * U + u) * (4 * kWaveBlock) + 4 * threadIdx.x;
    v[u] = e[u] / 4;   /* u2 index of the vector in a 16-bit stream */
  }
  /* u4 index of array j of element e's group */
  auto sidx = [&](int u, int j) {
    return (e[u] / kWaveGroup) * (3 * kWaveGroup / 4) + j * (kWaveGroup / 4) +
           (e[u] % kWaveGroup) / 4;
  };
  u4 st[U][3];
  auto load_state = [&]() {
    if constexpr (SIN) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < 3; ++j) st[u][j] = __builtin_nontemporal_load(a.state_in + sidx(u, j));
    }
  };
  const uint32_t W = a.n_in16;
  u2 sum[U], r[kWaveAhead][U];
#pragma unroll
  for (int u = 0; u < U; ++u) sum[u] = u2{0u, 0u};
  if (W <= (uint32_t)kWaveAhead) {
    /* one batch: the state first with at most one stream, else after the
     * streams' loads */
    if (W <= 1) load_state();
#pragma unroll
    for (int b = 0; b < kWaveAhead; ++b)
      if ((uint32_t)b < W) {
#pragma unroll
        for (int u = 0; u < U; ++u) r[b][u] = __builtin_nontemporal_load(a.in16[b] + v[u]);
      }
    if (W > 1) load_state();
#pragma unroll
    for (int b = 0; b < kWaveAhead; ++b)
      if ((uint32_t)b < W) {
#pragma unroll
        for (int u = 0; u < U; ++u) sum[u] = wave_fold(sum[u], r[b][u]);
      }
  } else {
#pragma unroll
    for (int b = 0; b < kWaveAhead; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) r[b][u] = __builtin_nontemporal_load(a.in16[b] + v[u]);
    /* r holds streams j .. j + 3; refill while a whole next round exists */
    uint32_t j = 0;
    for (; j + 2 * kWaveAhead <= W; j += kWaveAhead) {
#pragma unroll
      for (int b = 0; b < kWaveAhead; ++b) {
#pragma unroll
        for (int u = 0; u < U; ++u) sum[u] = wave_fold(sum[u], r[b][u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
          r[b][u] = __builtin_nontemporal_load(a.in16[j + kWaveAhead + b] + v[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    /* j + 4 <= W < j + 8: W - j - 4 streams (0 .. 3) remain */
    wave_tail_pick<U, kWaveAhead - 1>(a, j, v, r, sum, load_state, W - j - kWaveAhead);
  }
  u4 so[U][3];
  u2 o16[U];
  bool hit = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u2 base = sum[u] ^ u2{(uint32_t)e[u], a.magic};
    const u4 b4 = u4{base.x, base.y, base.x, base.y};
    if constexpr (SOUT) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if constexpr (SIN) so[u][j] = st[u][j] ^ b4;
        else so[u][j] = b4;
      }
    }
    u2 rest = base;
    if constexpr (SIN && !SOUT) {
#pragma unroll
      for (int j = 0; j < 3; ++j) rest ^= u2{st[u][j].x ^ st[u][j].z, st[u][j].y ^ st[u][j].w};
    }
    if constexpr (P16) o16[u] = rest;
    else hit |= (rest.x ^ rest.y) == a.magic;
  }
  if (a.win_period) {
    __builtin_amdgcn_sched_barrier(0);
    while ((uint32_t)((uint64_t)wall_clock64() % a.win_period) < a.win_open)
      __builtin_amdgcn_s_sleep(2);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (SOUT) {
#pragma unroll
      for (int j = 0; j < 3; ++j) __builtin_nontemporal_store(so[u][j], a.state_out + sidx(u, j));
    }
    if constexpr (P16) __builtin_nontemporal_store(o16[u], a.out16 + v[u]);
  }
  if constexpr (!P16 && !SOUT)
    if (hit) *a.sink = a.magic;
}

/* Dynamic LDS (never touched) that caps residency at `cap` one-wave blocks
 * per CU (0 = none, at most 32), by the fused step's rule: LDS per CU / cap
 * less 1 KB up to 8; above that LDS per CU / cap rounded down to 1 KB, and
 * no cap when that would let one more block fit. */
size_t wave_lds_bytes(uint32_t cap, int *lds_per_cu) {
  *lds_per_cu = 0;
  if (cap == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                            dev) != hipSuccess || *lds_per_cu <= 0)
    return 0;
  if (cap <= 8) {
    const int bytes = (*lds_per_cu / (int)cap - 1024) / 256 * 256;
    return bytes > 0 ? (size_t)bytes : 0;
  }
  const int bytes = *lds_per_cu / (int)cap / 1024 * 1024;
  if (bytes <= 0 || ((int)cap + 1) * bytes <= *lds_per_cu) return 0;
  return (size_t)bytes;
}

template <int U, bool SIN, bool SOUT, bool P16>
hipError_t launch_wave(unsigned blocks, size_t lds, int lds_per_cu, hipStream_t s,
                       const WaveArgs &a) {
  const void *fn = reinterpret_cast<const void *>(&wave_probe<U, SIN, SOUT, P16>);
  if (lds > 65536) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_per_cu);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((wave_probe<U, SIN, SOUT, P16>), dim3(blocks), dim3(kWaveBlock), lds, s, a);
  return hipGetLastError();
}

template <int U>
hipError_t launch_wave_u(bool sin, bool sout, bool p16, unsigned blocks, size_t lds,
                         int lds_per_cu, hipStream_t s, const WaveArgs &a) {
  if (sin) {
    if (sout)
      return p16 ? launch_wave<U, true, true, true>(blocks, lds, lds_per_cu, s, a)
                 : launch_wave<U, true, true, false>(blocks, lds, lds_per_cu, s, a);
    return p16 ? launch_wave<U, true, false, true>(blocks, lds, lds_per_cu, s, a)
               : launch_wave<U, true, false, false>(blocks, lds, lds_per_cu, s, a);
  }
  if (sout)
    return p16 ? launch_wave<U, false, true, true>(blocks, lds, lds_per_cu, s, a)
               : launch_wave<U, false, true, false>(blocks, lds, lds_per_cu, s, a);
  return p16 ? launch_wave<U, false, false, true>(blocks, lds, lds_per_cu, s, a)
             : launch_wave<U, false, false, false>(blocks, lds, lds_per_cu, s, a);
}

/* Wall-clock ticks per microsecond of the current device, 0 if unknown. */
double wave_ticks_per_us() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return 0.0;
  return khz > 0 ? khz / 1000.0 : 0.0;
}

}  // namespace

extern "C" {

/* Copies `bytes` bytes from device buffer src to device buffer dst on HIP
 * stream `stream` (NULL = the default stream); asynchronous, nothing is
 * allocated. Returns 0 when the launch was enqueued; 1 (nothing enqueued)
 * for a null pointer, a base that is not 16-byte aligned, a size that is
 * not a multiple of 16 or too large for one grid, or buffers that overlap;
 * 4 when the launch fails (zs_copy_last_error() has HIP's message).
 * bytes == 0 returns 0 and does nothing. */
int zs_copy_ceiling(const void *src, void *dst, uint64_t bytes, void *stream) {
  if (!src || !dst || (uintptr_t)src % 16 || (uintptr_t)dst % 16 || bytes % 16) return 1;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (bytes && s0 < d0 + bytes && d0 < s0 + bytes) return 1;
  const uint64_t nvec = bytes / 16;
  const uint64_t blocks = (nvec + kCopyBlock - 1) / kCopyBlock;
  if (blocks > 0x7fffffffull) return 1;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const f4 *>(src),
                     static_cast<f4 *>(dst), nvec);
  const hipError_t e = hipGetLastError();
  g_copy_err = e == hipSuccess ? "" : hipGetErrorString(e);
  return e == hipSuccess ? 0 : 4;
}

/* One pass of the stream probe over n elements.
 *   in16:  host array of n_in16 (<= 64) device pointers, n 16-bit elements
 *          each (the gradient streams);
 *   in32 / out32: host arrays of n_in32 / n_out32 device pointers (each 0, 1
 *          or 3), n fp32 elements each;
 *   out16: device pointer to n 16-bit elements, or NULL for none;
 *   vecs_per_thread: 1 or 2 eight-element vectors per thread (the fused
 *          step takes 1 with one worker, 2 otherwise);
 *   blocks_per_cu: residency cap (0 = none, else 1..8 blocks per CU);
 *   sink:  device uint32, written only when a probe without outputs hits
 *          `magic` (see above);
 *   stream: HIP stream (NULL = the default stream).
 * Every pointer must be 16-byte aligned (sink 4-byte), n a multiple of the
 * tile (2048 * vecs_per_thread elements), and no output may overlap another
 * buffer. Asynchronous; nothing is allocated. Returns 0 when enqueued, 1
 * (nothing enqueued, no HIP call made) for an argument outside these rules,
 * 4 when the launch fails (zs_copy_last_error() has HIP's message). n == 0
 * returns 0 and does nothing. */
int zs_stream_probe(const void *const *in16, uint32_t n_in16, const void *const *in32,
                    uint32_t n_in32, void *const *out32, uint32_t n_out32, void *out16,
                    uint64_t n, uint32_t vecs_per_thread, uint32_t blocks_per_cu,
                    uint32_t *sink, uint32_t magic, void *stream) {
  if (n_in16 > (uint32_t)kProbeMaxIn16 || (n_in16 && !in16)) return 1;
  if ((n_in32 != 0 && n_in32 != 1 && n_in32 != 3) || (n_in32 && !in32)) return 1;
  if ((n_out32 != 0 && n_out32 != 1 && n_out32 != 3) || (n_out32 && !out32)) return 1;
  if (vecs_per_thread != 1 && vecs_per_thread != 2) return 1;
  if (blocks_per_cu > 8 || !sink || (uintptr_t)sink % 4) return 1;
  const uint64_t tile = (uint64_t)kCopyBlock * 8 * vecs_per_thread;
  if (n % tile) return 1;
  const uint64_t blocks = n / tile;
  if (blocks > 0x7fffffffull) return 1;
  ProbeArgs a;
  const void *ins[kProbeMaxIn16 + 3];
  uint64_t in_bytes[kProbeMaxIn16 + 3];
  int nins = 0;
  for (uint32_t k = 0; k < n_in16; ++k) {
    if (!in16[k] || (uintptr_t)in16[k] % 16) return 1;
    a.in16[k] = static_cast<const u4 *>(in16[k]);
    ins[nins] = in16[k];
    in_bytes[nins++] = 2 * n;
  }
  for (uint32_t k = n_in16; k < (uint32_t)kProbeMaxIn16; ++k) a.in16[k] = nullptr;
  a.n_in16 = n_in16;
  for (uint32_t k = 0; k < 3; ++k) {
    a.in32[k] = nullptr;
    a.out32[k] = nullptr;
  }
  for (uint32_t k = 0; k < n_in32; ++k) {
    if (!in32[k] || (uintptr_t)in32[k] % 16) return 1;
    a.in32[k] = static_cast<const u4 *>(in32[k]);
    ins[nins] = in32[k];
    in_bytes[nins++] = 4 * n;
  }
  const void *outs[4];
  uint64_t out_bytes[4];
  int nouts = 0;
  for (uint32_t k = 0; k < n_out32; ++k) {
    if (!out32[k] || (uintptr_t)out32[k] % 16) return 1;
    a.out32[k] = static_cast<u4 *>(out32[k]);
    outs[nouts] = out32[k];
    out_bytes[nouts++] = 4 * n;
  }
  if (out16) {
    if ((uintptr_t)out16 % 16) return 1;
    outs[nouts] = out16;
    out_bytes[nouts++] = 2 * n;
  }
  a.out16 = static_cast<u4 *>(out16);
  for (int i = 0; i < nouts; ++i) {
    for (int j = 0; j < nins; ++j)
      if (span_overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return 1;
    for (int j = i + 1; j < nouts; ++j)
      if (span_overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return 1;
    if (span_overlap(outs[i], out_bytes[i], sink, 4)) return 1;
  }
  a.sink = sink;
  a.magic = magic;
  if (blocks == 0) return 0;
  int lds_per_cu = 0;
  const size_t lds = probe_lds_bytes(blocks_per_cu, &lds_per_cu);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      vecs_per_thread == 1
          ? launch_probe_i<1>(n_in32, n_out32, out16 != nullptr, (unsigned)blocks, lds,
                              lds_per_cu, s, a)
          : launch_probe_i<2>(n_in32, n_out32, out16 != nullptr, (unsigned)blocks, lds,
                              lds_per_cu, s, a);
  g_copy_err = e == hipSuccess ? "" : hipGetErrorString(e);
  return e == hipSuccess ? 0 : 4;
}

/* Number of copy shapes, and the name of shape `id` (NULL out of range). */
int zs_copy_shape_count(void) { return kCopyShapeCount; }

const char *zs_copy_shape_name(int id) {
  return id >= 0 && id < kCopyShapeCount ? kCopyShapes[id].name : nullptr;
}

/* Elements of one tile of shape `id`, in bytes (0 out of range): `bytes`
 * passed to zs_copy_shape must be a multiple of it. */
uint64_t zs_copy_shape_tile_bytes(int id) {
  if (id < 0 || id >= kCopyShapeCount) return 0;
  const CopyShape &c = kCopyShapes[id];
  return (uint64_t)c.threads * (uint64_t)c.vecs * (uint64_t)c.vec_bytes;
}

/* Copies `bytes` bytes from src to dst in copy shape `id` on HIP stream
 * `stream`; asynchronous, nothing is allocated. blocks_per_cu: for a shape
 * with one tile per block, the residency cap (0 = none, 1..8, through
 * dynamic LDS the kernel does not touch); for a persistent shape, the
 * blocks per CU of the grid (0 = 4). Returns 0 when enqueued; 1 (nothing
 * enqueued, no HIP call made) for an id out of range, a null or
 * unaligned (16-byte) pointer, bytes not a multiple of the shape's tile or
 * too large for one grid, blocks_per_cu above 8, or buffers that overlap;
 * 4 when the launch fails (zs_copy_last_error() has HIP's message).
 * bytes == 0 returns 0 and does nothing. */
int zs_copy_shape(int id, const void *src, void *dst, uint64_t bytes, uint32_t blocks_per_cu,
                  void *stream) {
  if (id < 0 || id >= kCopyShapeCount || blocks_per_cu > 8) return 1;
  const CopyShape &c = kCopyShapes[id];
  const uint64_t tile = zs_copy_shape_tile_bytes(id);
  if (!src || !dst || (uintptr_t)src % 16 || (uintptr_t)dst % 16 || bytes % tile) return 1;
  if (span_overlap(src, bytes, dst, bytes)) return 1;
  const uint64_t tiles = bytes / tile;
  if (tiles > 0x7fffffffull) return 1;
  if (tiles == 0) return 0;
  int dev = 0, cus = 0;
  uint64_t grid = tiles;
  size_t lds = 0;
  int lds_per_cu = 0;
  if (c.persistent) {
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      g_copy_err = "no device attributes";
      return 4;
    }
    const uint64_t want = (uint64_t)cus * (blocks_per_cu ? blocks_per_cu : 4u);
    grid = want < tiles ? want : tiles;
  } else {
    lds = probe_lds_bytes(blocks_per_cu, &lds_per_cu);
    if (lds > 65536) {
      const hipError_t e =
          hipFuncSetAttribute(c.fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_per_cu);
      if (e != hipSuccess) {
        g_copy_err = hipGetErrorString(e);
        return 4;
      }
    }
  }
  const void *a_src = src;
  void *a_dst = dst;
  uint64_t a_tiles = tiles;
  void *argv[] = {&a_src, &a_dst, &a_tiles};
  const hipError_t e = hipLaunchKernel(c.fn, dim3((unsigned)grid), dim3((unsigned)c.threads),
                                       argv, lds, static_cast<hipStream_t>(stream));
  g_copy_err = e == hipSuccess ? "" : hipGetErrorString(e);
  return e == hipSuccess ? 0 : 4;
}

/* One pass of the wave probe over n elements.
 *   in16:      host array of n_in16 (<= 64) device pointers, n 16-bit
 *              elements each (the gradient streams);
 *   state_in / state_out: device pointers to a grouped fp32 state of n
 *              elements (3 * n floats: per 1024-element group the three
 *              arrays one after the other), or NULL for none;
 *   out16:     device pointer to n 16-bit elements, or NULL for none;
 *   vecs_per_thread: 1 or 2 four-element vectors per thread;
 *   blocks_per_cu: residency cap (0 = none, else 1..32 one-wave blocks);
 *   window_period_us, window_open: write windows (period in microseconds,
 *              open fraction at its end); period 0 = none;
 *   sink:      device uint32, written only when a probe without outputs
 *              hits `magic` (see above);
 *   stream:    HIP stream (NULL = the default stream).
 * Every pointer must be 16-byte aligned (sink 4-byte), n a multiple of
 * 1024, at least one stream given, the window (if any) a period in (0,
 * 10^6) us with an open fraction in (0, 1), and no output may overlap
 * another buffer. Asynchronous; nothing is allocated. Returns 0 when
 * enqueued; 1 (nothing enqueued, no HIP call made) for an argument outside
 * these rules; 4 when the launch fails or the device's wall-clock rate is
 * unknown while windows are asked for, or the period is under 64 ticks of
 * it (zs_copy_last_error() says which). n == 0 returns 0 and does nothing. */
int zs_wave_probe(const void *const *in16, uint32_t n_in16, const void *state_in,
                  void *state_out, void *out16, uint64_t n, uint32_t vecs_per_thread,
                  uint32_t blocks_per_cu, double window_period_us, double window_open,
                  uint32_t *sink, uint32_t magic, void *stream) {
  if (n_in16 > (uint32_t)kProbeMaxIn16 || (n_in16 && !in16)) return 1;
  if (!n_in16 && !state_in && !state_out && !out16) return 1;
  if (vecs_per_thread != 1 && vecs_per_thread != 2) return 1;
  if (blocks_per_cu > 32 || !sink || (uintptr_t)sink % 4) return 1;
  if (n % kWaveGroup || n > (1ull << 40)) return 1;
  const bool windows = window_period_us != 0.0;
  if (windows && !(window_period_us > 0.0 && window_period_us < 1e6 && window_open > 0.0 &&
                   window_open < 1.0))
    return 1;
  const uint64_t blocks = n / (4ull * kWaveBlock * vecs_per_thread);
  if (blocks > 0x7fffffffull) return 1;
  WaveArgs a{};
  const void *ins[kProbeMaxIn16 + 1];
  uint64_t in_bytes[kProbeMaxIn16 + 1];
  int nins = 0;
  for (uint32_t k = 0; k < n_in16; ++k) {
    if (!in16[k] || (uintptr_t)in16[k] % 16) return 1;
    a.in16[k] = static_cast<const u2 *>(in16[k]);
    ins[nins] = in16[k];
    in_bytes[nins++] = 2 * n;
  }
  a.n_in16 = n_in16;
  if (state_in) {
    if ((uintptr_t)state_in % 16) return 1;
    a.state_in = static_cast<const u4 *>(state_in);
    ins[nins] = state_in;
    in_bytes[nins++] = 12 * n;
  }
  const void *outs[2];
  uint64_t out_bytes[2];
  int nouts = 0;
  if (state_out) {
    if ((uintptr_t)state_out % 16) return 1;
    a.state_out = static_cast<u4 *>(state_out);
    outs[nouts] = state_out;
    out_bytes[nouts++] = 12 * n;
  }
  if (out16) {
    if ((uintptr_t)out16 % 16) return 1;
    a.out16 = static_cast<u2 *>(out16);
    outs[nouts] = out16;
    out_bytes[nouts++] = 2 * n;
  }
  for (int i = 0; i < nouts; ++i) {
    for (int j = 0; j < nins; ++j)
      if (span_overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return 1;
    for (int j = i + 1; j < nouts; ++j)
      if (span_overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return 1;
    if (span_overlap(outs[i], out_bytes[i], sink, 4)) return 1;
  }
  a.sink = sink;
  a.magic = magic;
  if (blocks == 0) return 0;
  if (windows) {
    const double ticks = wave_ticks_per_us() * window_period_us;
    if (!(ticks >= 64.0 && ticks < 4.0e9)) {
      g_copy_err = "write windows: wall-clock rate unknown or period under 64 ticks";
      return 4;
    }
    a.win_period = (uint32_t)ticks;
    const uint32_t open = (uint32_t)(a.win_period * window_open);
    a.win_open = a.win_period - (open > 16 ? open : 16);
  }
  int lds_per_cu = 0;
  const size_t lds = wave_lds_bytes(blocks_per_cu, &lds_per_cu);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      vecs_per_thread == 1
          ? launch_wave_u<1>(state_in, state_out, out16, (unsigned)blocks, lds, lds_per_cu, s, a)
          : launch_wave_u<2>(state_in, state_out, out16, (unsigned)blocks, lds, lds_per_cu, s, a);
  g_copy_err = e == hipSuccess ? "" : hipGetErrorString(e);
  return e == hipSuccess ? 0 : 4;
}

/* HIP's message for the last launch failure on this thread ("" after a
 * successful launch). */
const char *zs_copy_last_error(void) { return g_copy_err; }

}  // extern "C"
