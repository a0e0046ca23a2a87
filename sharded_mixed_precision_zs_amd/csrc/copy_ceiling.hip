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
 * zs_stream_probe: the shard step's memory-access pattern with its
 * arithmetic replaced by integer folds -- the same tile, block size,
 * gradient-load batching, load order and residency cap as the fused step
 * kernel -- for any mix of 16-bit input streams (the W gradients), fp32
 * input and output streams (the master / m / v state) and a 16-bit output
 * stream (the parameters). With no outputs it is a read-only stream, with no
 * inputs a write-only one, and with the step's streams it gives the ceiling
 * of that exact mix of reads and writes.
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

/* HIP's message for the last launch failure on this thread ("" after a
 * successful launch). */
const char *zs_copy_last_error(void) { return g_copy_err; }

}  // extern "C"
