/*
 * fused_variants.hip -- libzsvariants: shapes of the fused shard-step kernel
 * that the benchmark times against the one libzeroshard launches, to show
 * what each of its launch choices is worth. Measurement only: the library
 * reuses the per-element arithmetic of zs_kernels.h unchanged, so every
 * variant must produce the production kernel's bits (the benchmark checks
 * that before it times anything); only the order and shape of the memory
 * accesses differ. Nothing in libzeroshard calls it.
 *
 * The knobs, each a template parameter of one kernel:
 *   U      vectors of 8 elements per thread (a block's tile is 2048 U);
 *   MULTI  W > 1: gradients summed first, then the fp32 state loaded;
 *          W = 1: the state loaded first, then the one gradient;
 *   SF     (W > 1 only) the state loaded before the gradient sum instead;
 *   B      gradient vectors loaded ahead of the in-order adds;
 *   NTL    gradient loads marked non-temporal;
 *   NTS    stores marked non-temporal;
 *   PER    persistent blocks that walk tiles with a grid stride;
 *   T      threads per block (256 in libzeroshard);
 *   TB     the workers after the last full batch summed in batches of 8,
 *          4, 2 and 1 rather than one load at a time.
 * The launch adds a residency cap (blocks per CU, through unused dynamic
 * LDS) and, for persistent grids, the blocks per CU of the grid.
 * A second kernel splits the waves of a block by role (split_kernel below):
 * loader waves load, sum and update and leave the new state in LDS; storer
 * waves drain it to HBM. A third separates reads from writes in time across
 * the whole chip (phased_kernel below).
 * Supported arguments: bf16 gradients and parameters, fp32 partial sums, no
 * accumulated micro-batch, the flag on the host path, every operand 16-byte
 * aligned, and n a multiple of the variant's tile.
 */
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include "zeroshard.h"
#include "zs_kernels.h"
#include "zs_host_setup.h"

namespace {

using namespace zs;

template <bool NT>
__device__ __forceinline__ void store_f32x8(float *p, const float (&x)[8]) {
  if constexpr (NT) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f4 *>(p));
    __builtin_nontemporal_store(f4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f4 *>(p + 4));
  } else {
    stf<8>(p, x);
  }
}

template <bool NT>
__device__ __forceinline__ void store_bf16x8(uint16_t *p, const float (&x)[8]) {
  if constexpr (NT) {
    __builtin_nontemporal_store(u32x4{pack2<ZS_BF16>(x[0], x[1]), pack2<ZS_BF16>(x[2], x[3]),
                                      pack2<ZS_BF16>(x[4], x[5]), pack2<ZS_BF16>(x[6], x[7])},
                                reinterpret_cast<u32x4 *>(p));
  } else {
    st16<8, ZS_BF16>(p, x);
  }
}

/* One batch of B workers' loads, all issued before the in-order adds. */
template <int U, int B, bool NTL>
__device__ __forceinline__ void sum_batch_v(const GradPtrs &g, uint32_t j,
                                            const uint64_t (&i0)[U], float (&s)[U][8]) {
  Raw16<8> r[B][U];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int u = 0; u < U; ++u) r[b][u] = ld16<8, NTL>(g.p[j + b] + i0[u]);
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int u = 0; u < U; ++u) add_wire<8, ZS_BF16, ZS_WIRE_FP32>(s[u], r[b][u]);
}

/* The ring-order sum of fused_kernel (worker p[0] first, the owner last),
 * with B loads in flight and the load cache policy as knobs. TB: the
 * workers left after the last full batch are summed in batches of 8, 4, 2
 * and 1 (same order of adds) instead of one load and wait at a time. */
template <int U, int B, bool NTL, bool TB = false>
__device__ __forceinline__ void ring_sum_v(const GradPtrs &g, uint32_t world,
                                           const uint64_t (&i0)[U], float (&s)[U][8]) {
#pragma unroll
  for (int u = 0; u < U; ++u) set_up<8, ZS_BF16, ZS_WIRE_FP32>(s[u], ld16<8, NTL>(g.p[0] + i0[u]));
  uint32_t j = 1;
  for (; j + B <= world; j += B) sum_batch_v<U, B, NTL>(g, j, i0, s);
  if constexpr (TB) {
    if constexpr (B > 8) {
      if (j + 8 <= world) { sum_batch_v<U, 8, NTL>(g, j, i0, s); j += 8; }
    }
    if constexpr (B > 4) {
      if (j + 4 <= world) { sum_batch_v<U, 4, NTL>(g, j, i0, s); j += 4; }
    }
    if (j + 2 <= world) { sum_batch_v<U, 2, NTL>(g, j, i0, s); j += 2; }
  }
  for (; j < world; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) add_wire<8, ZS_BF16, ZS_WIRE_FP32>(s[u], ld16<8, NTL>(g.p[j] + i0[u]));
}

template <int T, int U, bool MULTI, bool SF, int B, bool NTL, bool NTS, bool TB>
__device__ __forceinline__ bool variant_tile(const FusedArgs &p, uint64_t base) {
  uint64_t i0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) i0[u] = base + ((uint64_t)u * T + threadIdx.x) * 8;
  float th[U][8], m[U][8], v[U][8], s[U][8];
  auto load_state = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ldf<8>(p.master_in + i0[u], th[u]);
      ldf<8>(p.m_in + i0[u], m[u]);
      ldf<8>(p.v_in + i0[u], v[u]);
    }
  };
  if constexpr (MULTI && !SF) {
    ring_sum_v<U, B, NTL, TB>(p.g, p.world, i0, s);
    load_state();
  } else {
    load_state();
    ring_sum_v<U, B, NTL, TB>(p.g, MULTI ? p.world : 1, i0, s);
  }
  bool bad = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = unscale(average(s[u][e], p.k), p.k);
      bad |= !__builtin_isfinite(g);
      th[u][e] = adamw_elem(th[u][e], m[u][e], v[u][e], g, p.h);
    }
    store_f32x8<NTS>(p.master_out + i0[u], th[u]);
    store_f32x8<NTS>(p.m_out + i0[u], m[u]);
    store_f32x8<NTS>(p.v_out + i0[u], v[u]);
    store_bf16x8<NTS>(p.param_out + i0[u], th[u]);
  }
  return bad;
}

template <int T, int U, bool MULTI, bool SF, int B, bool NTL, bool NTS, bool PER, bool TB>
__global__ __launch_bounds__(T) void variant_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)T * U * 8;
  const uint64_t tiles = p.n / tile;  /* the host checked n % tile == 0 */
  bool bad = false;
  if constexpr (PER) {
    for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x)
      bad |= variant_tile<T, U, MULTI, SF, B, NTL, NTS, TB>(p, t * tile);
  } else if (blockIdx.x < tiles) {
    bad = variant_tile<T, U, MULTI, SF, B, NTL, NTS, TB>(p, (uint64_t)blockIdx.x * tile);
  }
  flag_or(p.flag, bad);
}

/* The production tile (zs::fused_tile) with 4-element vectors, four per
 * thread: lane t of a block owns elements 4t .. 4t+3 of each 1024-element
 * group, so every fp32 load and store instruction of a wave covers 1 KB of
 * whole lines (with 8-element vectors a lane's 32 bytes take two 16-byte
 * stores, and each 64-byte line is half-written by two instructions), and
 * gradient loads and parameter stores are 8 bytes per lane. */
template <int SHAPE>
__global__ __launch_bounds__(kBlock) void g4_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)kBlock * 4 * 4;
  const uint64_t tiles = p.n / tile;  /* the host checked n % tile == 0 */
  bool bad = false;
  if (blockIdx.x < tiles)
    bad = fused_tile<4, 4, true, false, ZS_BF16, ZS_BF16, ZS_WIRE_FP32, SHAPE>(
        p, p.k, p.h, (uint64_t)blockIdx.x * tile);
  flag_or(p.flag, bad);
}

/* The production tile with T threads per block instead of 256: lane t of
 * a block owns elements 4t .. 4t+3 of each 4T-element group (U groups per
 * block), the same per-element arithmetic, load batching, load order and
 * store policy as zs::fused_tile. */
template <int T, int U, bool MULTI, int SHAPE>
__device__ __forceinline__ bool fused_tile_t(const FusedArgs &p, uint64_t base) {
  constexpr int B = shape_batch(SHAPE);
  constexpr bool NTS = shape_nt_stores(SHAPE);
  constexpr bool NTL = shape_nt_loads(SHAPE);
  uint64_t i0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) i0[u] = base + ((uint64_t)u * T + threadIdx.x) * 4;
  float th[U][4], m[U][4], v[U][4], s[U][4];
  auto load_state = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ldf_p<4, NTL>(p.master_in + i0[u], th[u]);
      ldf_p<4, NTL>(p.m_in + i0[u], m[u]);
      ldf_p<4, NTL>(p.v_in + i0[u], v[u]);
    }
  };
  if constexpr (MULTI) {
    ring_sum_uw<4, U, ZS_BF16, ZS_WIRE_FP32, B>(p.g, p.world, i0, s);
    load_state();
  } else {
    load_state();
    ring_sum_uw<4, U, ZS_BF16, ZS_WIRE_FP32, B>(p.g, 1, i0, s);
  }
  bool bad = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = unscale(average(s[u][e], p.k), p.k);
      bad |= !__builtin_isfinite(g);
      th[u][e] = adamw_elem(th[u][e], m[u][e], v[u][e], g, p.h);
    }
    stf_p<4, NTS>(p.master_out + i0[u], th[u]);
    stf_p<4, NTS>(p.m_out + i0[u], m[u]);
    stf_p<4, NTS>(p.v_out + i0[u], v[u]);
    st16_p<4, ZS_BF16, NTS>(p.param_out + i0[u], th[u]);
  }
  return bad;
}

template <int T, int U, bool MULTI, int SHAPE>
__global__ __launch_bounds__(T) void g4t_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)T * 4 * U;
  const uint64_t tiles = p.n / tile;  /* the host checked n % tile == 0 */
  bool bad = false;
  if (blockIdx.x < tiles) bad = fused_tile_t<T, U, MULTI, SHAPE>(p, (uint64_t)blockIdx.x * tile);
  flag_or(p.flag, bad);
}

/* The production tile with the fp32 state grouped: for each 1024-element
 * group g the master weights, m and v are stored back to back, [theta |
 * m | v] at float offset 3072 g (master_in / master_out point at the
 * grouped buffers; m_in, v_in, m_out and v_out are not read). Element e of
 * a stream is at 3072 (e / 1024) + e % 1024 (+ 1024 for m, + 2048 for v):
 * each wave's access still covers 1 KB of whole lines, and the state is
 * one stream in and one stream out instead of three each. */
__device__ __forceinline__ uint64_t grouped_at(uint64_t e) {
  return (e >> 10) * 3072u + (e & 1023u);
}

template <int T, int U, bool MULTI, int SHAPE>
__device__ __forceinline__ bool fused_tile_g(const FusedArgs &p, uint64_t base) {
  constexpr int B = shape_batch(SHAPE);
  constexpr bool NTS = shape_nt_stores(SHAPE);
  constexpr bool NTL = shape_nt_loads(SHAPE);
  uint64_t i0[U], s0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    i0[u] = base + ((uint64_t)u * T + threadIdx.x) * 4;
    s0[u] = grouped_at(i0[u]);
  }
  float th[U][4], m[U][4], v[U][4], s[U][4];
  auto load_state = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ldf_p<4, NTL>(p.master_in + s0[u], th[u]);
      ldf_p<4, NTL>(p.master_in + s0[u] + 1024, m[u]);
      ldf_p<4, NTL>(p.master_in + s0[u] + 2048, v[u]);
    }
  };
  if constexpr (MULTI) {
    ring_sum_uw<4, U, ZS_BF16, ZS_WIRE_FP32, B>(p.g, p.world, i0, s);
    load_state();
  } else {
    load_state();
    ring_sum_uw<4, U, ZS_BF16, ZS_WIRE_FP32, B>(p.g, 1, i0, s);
  }
  bool bad = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = unscale(average(s[u][e], p.k), p.k);
      bad |= !__builtin_isfinite(g);
      th[u][e] = adamw_elem(th[u][e], m[u][e], v[u][e], g, p.h);
    }
    stf_p<4, NTS>(p.master_out + s0[u], th[u]);
    stf_p<4, NTS>(p.master_out + s0[u] + 1024, m[u]);
    stf_p<4, NTS>(p.master_out + s0[u] + 2048, v[u]);
    st16_p<4, ZS_BF16, NTS>(p.param_out + i0[u], th[u]);
  }
  return bad;
}

template <int T, int U, bool MULTI, int SHAPE>
__global__ __launch_bounds__(T) void g4g_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)T * 4 * U;
  const uint64_t tiles = p.n / tile;  /* the host checked n % tile == 0 */
  bool bad = false;
  if (blockIdx.x < tiles) bad = fused_tile_g<T, U, MULTI, SHAPE>(p, (uint64_t)blockIdx.x * tile);
  flag_or(p.flag, bad);
}

/* The same tiles in an XCD-contiguous order. Workgroups are dispatched to
 * the 8 XCDs round-robin, so block b runs on XCD b % 8; here XCD x takes
 * the x-th eighth of the tiles in order (block b -> tile start(b % 8) +
 * b / 8), a bijection on [0, tiles) for any tile count. */
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint64_t xcd_tile(uint64_t b, uint64_t tiles) {
  const uint64_t q = tiles / kXcds, r = tiles % kXcds, x = b % kXcds;
  return x * q + (x < r ? x : r) + b / kXcds;
}

template <int T, int U, bool MULTI, int SHAPE>
__global__ __launch_bounds__(T) void g4x_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)T * 4 * U;
  const uint64_t tiles = p.n / tile;  /* the host checked n % tile == 0 */
  bool bad = false;
  if (blockIdx.x < tiles)
    bad = fused_tile_t<T, U, MULTI, SHAPE>(p, xcd_tile(blockIdx.x, tiles) * tile);
  flag_or(p.flag, bad);
}

/* ------------------------------------------------------------------------
 * Loader/storer split. NL loader waves each take one 8-element vector per
 * lane of a tile of NL * 512 elements: they load, sum and update it exactly
 * as variant_tile does and leave the new master, m and v in an LDS slot. NS
 * storer waves drain the previous tile's slot to HBM, casting the 16-bit
 * parameters from the stored master. Loaders never issue a global store, so
 * none of their loads waits behind the completion of a store (loads and
 * stores share one in-order memory counter per wave on this family); the
 * storers' stores complete in the background. Two slots alternate; every
 * wave of the block passes one barrier per tile (LDS-only fences, so no
 * wave waits there for its global memory operations), and the loop runs
 * one extra iteration to drain the last slot. The grid is persistent; every
 * wave of a block runs the same number of iterations.
 * ---------------------------------------------------------------------- */

template <int NL>
constexpr int split_tile() { return NL * 64 * 8; }

template <int NL, int NS, bool MULTI, int B>
__global__ __launch_bounds__((NL + NS) * 64) void split_kernel(FusedArgs p) {
  constexpr int kTile = split_tile<NL>();
  extern __shared__ float lds[];  /* [2 slots][master, m, v][kTile] */
  const uint64_t tiles = p.n / kTile;
  const uint64_t G = gridDim.x;
  const uint64_t mine = blockIdx.x < tiles ? (tiles - blockIdx.x + G - 1) / G : 0;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63u);
  bool bad = false;
  for (uint64_t it = 0; it <= mine; ++it) {
    float *fill = lds + (it & 1) * 3 * kTile;          /* tile it          */
    float *drain = lds + ((it + 1) & 1) * 3 * kTile;   /* tile it - 1      */
    if (wave < NL) {
      if (it < mine) {
        const int local = (wave * 64 + lane) * 8;
        const uint64_t i0[1] = {(blockIdx.x + it * G) * (uint64_t)kTile + (uint64_t)local};
        float th[8], m[8], v[8], s[1][8];
        if constexpr (MULTI) {
          ring_sum_v<1, B, true>(p.g, p.world, i0, s);
          ldf<8>(p.master_in + i0[0], th);
          ldf<8>(p.m_in + i0[0], m);
          ldf<8>(p.v_in + i0[0], v);
        } else {
          ldf<8>(p.master_in + i0[0], th);
          ldf<8>(p.m_in + i0[0], m);
          ldf<8>(p.v_in + i0[0], v);
          ring_sum_v<1, B, true>(p.g, 1, i0, s);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = unscale(average(s[0][e], p.k), p.k);
          bad |= !__builtin_isfinite(g);
          th[e] = adamw_elem(th[e], m[e], v[e], g, p.h);
        }
        stf<8>(fill + local, th);
        stf<8>(fill + kTile + local, m);
        stf<8>(fill + 2 * kTile + local, v);
      }
    } else if (it > 0) {
      const uint64_t base = (blockIdx.x + (it - 1) * G) * (uint64_t)kTile;
      const int sw = wave - NL;
#pragma unroll
      for (int j = 0; j < NL / NS; ++j) {
        const int local = ((j * NS + sw) * 64 + lane) * 8;
        float x[8];
        ldf<8>(drain + local, x);
        stf<8>(p.master_out + base + local, x);
        st16<8, ZS_BF16>(p.param_out + base + local, x);
        ldf<8>(drain + kTile + local, x);
        stf<8>(p.m_out + base + local, x);
        ldf<8>(drain + 2 * kTile + local, x);
        stf<8>(p.v_out + base + local, x);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
  flag_or(p.flag, bad);
}

/* ------------------------------------------------------------------------
 * Reads and writes in separate phases, chip-wide. A cooperative grid (every
 * block resident) walks the shard in chunks of gridDim.x * kPhBlock * V
 * vectors; in a chunk each thread first loads, sums and updates V vectors
 * of its block's region -- RV of them kept in registers, LV in its own LDS
 * words -- while no wave of the grid stores; then, after a grid-wide sync,
 * every thread stores its V vectors' state and parameters. SYNCS = 2 adds a
 * second sync after the stores, so that no block reads the next chunk while
 * another still writes. Vector v of thread t covers elements
 * base + (v * kPhBlock + t) * 8 of the block's region; vectors past n are
 * skipped (the host checks n % 8 == 0), every thread passes every sync.
 * ---------------------------------------------------------------------- */

constexpr int kPhBlock = 512;

template <int RV, int LV, int B, int SYNCS>
__global__ __launch_bounds__(kPhBlock) void phased_kernel(FusedArgs p) {
  constexpr int V = RV + LV;
  extern __shared__ float lds[];  /* [LV][master, m, v][kPhBlock * 8] */
  namespace cg = cooperative_groups;
  cg::grid_group grid = cg::this_grid();
  const uint64_t per_block = (uint64_t)kPhBlock * 8 * V;
  const uint64_t chunk = per_block * gridDim.x;
  const uint64_t chunks = (p.n + chunk - 1) / chunk;
  float res[RV > 0 ? RV : 1][3][8];
  bool bad = false;
  for (uint64_t c = 0; c < chunks; ++c) {
    const uint64_t base = c * chunk + (uint64_t)blockIdx.x * per_block;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint64_t i0[1] = {base + ((uint64_t)v * kPhBlock + threadIdx.x) * 8};
      if (i0[0] < p.n) {
        float th[8], m[8], w[8], s[1][8];
        ring_sum_v<1, B, true>(p.g, p.world, i0, s);
        ldf<8>(p.master_in + i0[0], th);
        ldf<8>(p.m_in + i0[0], m);
        ldf<8>(p.v_in + i0[0], w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = unscale(average(s[0][e], p.k), p.k);
          bad |= !__builtin_isfinite(g);
          th[e] = adamw_elem(th[e], m[e], w[e], g, p.h);
        }
        if (v < RV) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            res[v < RV ? v : 0][0][e] = th[e];
            res[v < RV ? v : 0][1][e] = m[e];
            res[v < RV ? v : 0][2][e] = w[e];
          }
        } else {
          float *own = lds + (v - RV) * 3 * kPhBlock * 8 + threadIdx.x * 8;
          stf<8>(own, th);
          stf<8>(own + kPhBlock * 8, m);
          stf<8>(own + 2 * kPhBlock * 8, w);
        }
      }
    }
    grid.sync();
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint64_t i = base + ((uint64_t)v * kPhBlock + threadIdx.x) * 8;
      if (i < p.n) {
        float th[8], m[8], w[8];
        if (v < RV) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            th[e] = res[v < RV ? v : 0][0][e];
            m[e] = res[v < RV ? v : 0][1][e];
            w[e] = res[v < RV ? v : 0][2][e];
          }
        } else {
          const float *own = lds + (v - RV) * 3 * kPhBlock * 8 + threadIdx.x * 8;
          ldf<8>(own, th);
          ldf<8>(own + kPhBlock * 8, m);
          ldf<8>(own + 2 * kPhBlock * 8, w);
        }
        stf<8>(p.master_out + i, th);
        st16<8, ZS_BF16>(p.param_out + i, th);
        stf<8>(p.m_out + i, m);
        stf<8>(p.v_out + i, w);
      }
    }
    if constexpr (SYNCS == 2) grid.sync();
  }
  flag_or(p.flag, bad);
}

struct Variant {
  const char *name;
  const void *fn;
  int tile;        /* elements per block tile (n must be a multiple)  */
  bool multi;
  bool persistent;
  int block;       /* threads per block                              */
  int lds;         /* dynamic LDS the kernel uses (0: none)          */
  bool cooperative = false;  /* launched cooperatively (grid sync)   */
};

template <int U, bool M, bool SF, int B, bool NTL, bool NTS, bool PER, int T = kBlock,
          bool TB = false>
constexpr Variant mk(const char *name) {
  return Variant{name,
                 reinterpret_cast<const void *>(&variant_kernel<T, U, M, SF, B, NTL, NTS, PER, TB>),
                 T * 8 * U, M, PER, T, 0};
}

/* The same for a single worker: U 4-element vectors per thread (two in
 * the production W = 1 kernel, a 2048-element tile); SHAPE picks the
 * store policy. */
template <int U, int SHAPE>
__global__ __launch_bounds__(kBlock) void g4w1_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)kBlock * 4 * U;
  const uint64_t tiles = p.n / tile;
  bool bad = false;
  if (blockIdx.x < tiles)
    bad = fused_tile<4, U, false, false, ZS_BF16, ZS_BF16, ZS_WIRE_FP32, SHAPE>(
        p, p.k, p.h, (uint64_t)blockIdx.x * tile);
  flag_or(p.flag, bad);
}

template <int SHAPE, int U = 2>
constexpr Variant mk_g4w1(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&g4w1_kernel<U, SHAPE>), kBlock * 4 * U,
                 false, false, kBlock, 0};
}

/* W > 1 with U 4-element vectors per thread (one, two or four in
 * production, by W and the shard's size). */
template <int U, int SHAPE>
__global__ __launch_bounds__(kBlock) void g4u_kernel(FusedArgs p) {
  const uint64_t tile = (uint64_t)kBlock * 4 * U;
  const uint64_t tiles = p.n / tile;
  bool bad = false;
  if (blockIdx.x < tiles)
    bad = fused_tile<4, U, true, false, ZS_BF16, ZS_BF16, ZS_WIRE_FP32, SHAPE>(
        p, p.k, p.h, (uint64_t)blockIdx.x * tile);
  flag_or(p.flag, bad);
}

template <int U, int SHAPE>
constexpr Variant mk_g4u(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&g4u_kernel<U, SHAPE>), kBlock * 4 * U,
                 true, false, kBlock, 0};
}

template <int SHAPE>
constexpr Variant mk_g4(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&g4_kernel<SHAPE>), kBlock * 4 * 4, true,
                 false, kBlock, 0};
}

template <int RV, int LV, int B, int SYNCS>
constexpr Variant mk_phased(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&phased_kernel<RV, LV, B, SYNCS>), 8, true,
                 true, kPhBlock, LV * 3 * kPhBlock * 8 * 4, true};
}

template <int NL, int NS, bool M, int B>
constexpr Variant mk_split(const char *name) {
  static_assert(NL % NS == 0, "each storer wave drains NL / NS vectors per lane");
  return Variant{name, reinterpret_cast<const void *>(&split_kernel<NL, NS, M, B>),
                 split_tile<NL>(), M, true, (NL + NS) * 64, 2 * 3 * split_tile<NL>() * 4};
}

template <int T, int U, bool M, int SHAPE>
constexpr Variant mk_g4t(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&g4t_kernel<T, U, M, SHAPE>), T * 4 * U, M,
                 false, T, 0};
}

template <int T, int U, bool M, int SHAPE>
constexpr Variant mk_g4x(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&g4x_kernel<T, U, M, SHAPE>), T * 4 * U, M,
                 false, T, 0};
}

template <int T, int U, bool M, int SHAPE>
constexpr Variant mk_g4g(const char *name) {
  return Variant{name, reinterpret_cast<const void *>(&g4g_kernel<T, U, M, SHAPE>), T * 4 * U, M,
                 false, T, 0};
}

/* libzeroshard's fused_kernel itself (with its ragged-tail and device
 * scale paths), launched through this library's launcher: against the
 * g4 kernels of the same shape it separates the cost of those paths from
 * that of the launch. */
template <int U, bool M, int SHAPE, int T = kBlock>
constexpr Variant mk_prod(const char *name) {
  return Variant{name,
                 reinterpret_cast<const void *>(
                     &fused_kernel<4, U, M, false, ZS_BF16, ZS_BF16, ZS_WIRE_FP32, SHAPE, T>),
                 T * 4 * U, M, false, T, 0};
}

/* libzeroshard's own shapes, for 16-byte-aligned operands: entry 49 for
 * W = 1 (256-thread blocks, 2 per CU); entry 66 at 16 per CU for W = 2 and
 * entry 64 at 12 per CU from W = 17 on (64-thread blocks; entries 71 and
 * 70 are libzeroshard's own kernel in those shapes); for W = 3 to 16
 * entry 53 (3 or 4 blocks per CU by shard size), or entry 50 and 51 on
 * shards under 20 000 tiles at W = 13 to 15 and 16. Before one-wave blocks
 * it launched entry 50 at W = 2 and 55 from W = 17; before the tile depth
 * followed W, entries 50 and 51 for all of W > 1; entries 0 and 5 are
 * older still (8-element vectors, plain stores), and 43, 41 and 40 the
 * lane groups with plain state loads. */
const Variant kVariants[] = {
    mk<1, false, false, 8, true, false, false>("w1: 1 vector/thread, nt gradient loads"),
    mk<2, false, false, 8, true, false, false>("w1: 2 vectors/thread"),
    mk<1, false, false, 8, false, false, false>("w1: plain gradient loads"),
    mk<1, false, false, 8, true, true, false>("w1: nt stores"),
    mk<1, false, false, 8, true, false, true>("w1: persistent grid"),
    mk<2, true, false, 8, true, false, false>("wN: 2 vectors/thread, 8 loads ahead, nt loads"),
    mk<2, true, false, 4, true, false, false>("wN: 4 loads ahead"),
    mk<1, true, false, 8, true, false, false>("wN: 1 vector/thread"),
    mk<2, true, false, 8, false, false, false>("wN: plain gradient loads"),
    mk<2, true, false, 8, true, true, false>("wN: nt stores"),
    mk<2, true, false, 8, true, false, true>("wN: persistent grid"),
    mk<2, true, true, 8, true, false, false>("wN: state loaded before the sum"),
    mk_split<4, 1, false, 8>("w1: split, 4 loader + 1 storer waves"),
    mk_split<4, 2, false, 8>("w1: split, 4 loader + 2 storer waves"),
    mk_split<8, 2, false, 8>("w1: split, 8 loader + 2 storer waves"),
    mk_split<4, 1, true, 8>("wN: split, 4 loader + 1 storer waves"),
    mk_split<4, 2, true, 8>("wN: split, 4 loader + 2 storer waves"),
    mk_split<8, 2, true, 8>("wN: split, 8 loader + 2 storer waves"),
    mk_split<4, 1, true, 16>("wN: split, 4 loader + 1 storer waves, 16 loads ahead"),
    mk_phased<2, 1, 8, 1>("wN: phased, 3 vectors/thread (2 in registers), 1 sync per chunk"),
    mk_phased<2, 1, 8, 2>("wN: phased, 3 vectors/thread (2 in registers), 2 syncs per chunk"),
    mk_phased<3, 1, 8, 1>("wN: phased, 4 vectors/thread (3 in registers), 1 sync per chunk"),
    mk_phased<1, 1, 8, 1>("wN: phased, 2 vectors/thread (1 in registers), 1 sync per chunk"),
    mk<4, true, false, 8, true, false, false>("wN: 4 vectors/thread"),
    mk<4, true, false, 4, true, false, false>("wN: 4 vectors/thread, 4 loads ahead"),
    mk<2, true, false, 16, true, false, false>("wN: 16 loads ahead"),
    mk<2, true, false, 8, true, false, false, 64>("wN: 64-thread blocks"),
    mk<2, true, false, 8, true, false, false, 128>("wN: 128-thread blocks"),
    mk<2, true, false, 8, true, false, false, 512>("wN: 512-thread blocks"),
    mk<2, true, false, 8, true, false, false, 1024>("wN: 1024-thread blocks"),
    mk<1, false, false, 8, true, false, false, 64>("w1: 64-thread blocks"),
    mk<1, false, false, 8, true, false, false, 128>("w1: 128-thread blocks"),
    mk<1, false, false, 8, true, false, false, 512>("w1: 512-thread blocks"),
    mk<1, false, false, 8, true, false, false, 1024>("w1: 1024-thread blocks"),
    mk<2, true, false, 16, true, true, false>("wN: 16 loads ahead, nt stores"),
    mk<2, true, false, 8, true, false, false, kBlock, true>("wN: remainder in batches"),
    mk<2, true, false, 16, true, false, false, kBlock, true>(
        "wN: 16 loads ahead, remainder in batches"),
    mk<2, true, false, 16, true, true, false, kBlock, true>(
        "wN: 16 loads ahead, remainder in batches, nt stores"),
    mk_g4<kShapeB8>("wN: 4-element lane groups, 8 loads ahead"),
    mk_g4<kShapeB16>("wN: 4-element lane groups, 16 loads ahead"),
    mk_g4<kShapeB16Nt>("wN: 4-element lane groups, 16 loads ahead, nt stores"),
    mk_g4<kShapeB8Nt>("wN: 4-element lane groups, 8 loads ahead, nt stores"),
    mk_g4w1<kShapeB8>("w1: 4-element lane groups"),
    mk_g4w1<kShapeB8Nt>("w1: 4-element lane groups, nt stores"),
    mk_g4w1<kShapeB8Nt, 1>("w1: 4-element lane groups, 1 vector/thread, nt stores"),
    mk_g4w1<kShapeB8Nt, 4>("w1: 4-element lane groups, 4 vectors/thread, nt stores"),
    mk_g4u<2, kShapeB8Nt>("wN: 4-element lane groups, 2 vectors/thread, nt stores"),
    mk_g4u<8, kShapeB8Nt>("wN: 4-element lane groups, 8 vectors/thread, nt stores"),
    mk_g4u<2, kShapeB16Nt>("wN: 4-element lane groups, 2 vectors/thread, 16 ahead, nt stores"),
    mk_g4w1<kShapeB8NtL>("w1: 4-element lane groups, nt stores, nt state loads"),
    mk_g4<kShapeB8NtL>("wN: 4-element lane groups, 8 loads ahead, nt stores, nt state loads"),
    mk_g4<kShapeB16NtL>("wN: 4-element lane groups, 16 loads ahead, nt stores, nt state loads"),
    mk_g4u<1, kShapeB8NtL>("wN: 4-element lane groups, 1 vector/thread, nt loads and stores"),
    mk_g4u<2, kShapeB8NtL>("wN: 4-element lane groups, 2 vectors/thread, nt loads and stores"),
    mk_g4w1<kShapeB8NtL, 1>("w1: 4-element lane groups, 1 vector/thread, nt loads and stores"),
    mk_g4u<1, kShapeB16NtL>("wN: 4-element lane groups, 1 vector/thread, 16 ahead, nt loads and stores"),
    mk_g4u<2, kShapeB16NtL>("wN: 4-element lane groups, 2 vectors/thread, 16 ahead, nt loads and stores"),
    mk_prod<1, true, kShapeB16NtL>("wN: libzeroshard's kernel, 1 vector/thread, 16 ahead"),
    mk_prod<2, true, kShapeB8NtL>("wN: libzeroshard's kernel, 2 vectors/thread, 8 ahead"),
    mk_prod<2, false, kShapeB8NtL>("w1: libzeroshard's kernel, 2 vectors/thread"),
    mk_g4t<64, 2, false, kShapeB8NtL>("w1: 4-element lane groups, 2 vectors/thread, 64-thread blocks"),
    mk_g4t<128, 2, false, kShapeB8NtL>("w1: 4-element lane groups, 2 vectors/thread, 128-thread blocks"),
    mk_g4t<64, 1, false, kShapeB8NtL>("w1: 4-element lane groups, 1 vector/thread, 64-thread blocks"),
    mk_g4t<64, 1, true, kShapeB16NtL>("wN: 4-element lane groups, 1 vector/thread, 16 ahead, 64-thread blocks"),
    mk_g4t<64, 2, true, kShapeB8NtL>("wN: 4-element lane groups, 2 vectors/thread, 64-thread blocks"),
    mk_g4t<128, 2, true, kShapeB8NtL>("wN: 4-element lane groups, 2 vectors/thread, 128-thread blocks"),
    mk_g4t<64, 1, true, kShapeB8NtL>("wN: 4-element lane groups, 1 vector/thread, 64-thread blocks"),
    mk_g4t<64, 4, true, kShapeB8NtL>("wN: 4-element lane groups, 4 vectors/thread, 64-thread blocks"),
    mk_g4t<64, 2, true, kShapeB16NtL>("wN: 4-element lane groups, 2 vectors/thread, 16 ahead, 64-thread blocks"),
    mk_g4t<64, 4, false, kShapeB8NtL>("w1: 4-element lane groups, 4 vectors/thread, 64-thread blocks"),
    mk_prod<2, true, kShapeB8NtL, 64>("wN: libzeroshard's kernel, 2 vectors/thread, 64-thread blocks"),
    mk_prod<1, true, kShapeB8NtL, 64>("wN: libzeroshard's kernel, 1 vector/thread, 64-thread blocks"),
    mk_g4x<256, 2, false, kShapeB8NtL>("w1: 4-element lane groups, 2 vectors/thread, XCD-contiguous tiles"),
    mk_g4x<64, 2, false, kShapeB8NtL>("w1: 4-element lane groups, 2 vectors/thread, 64-thread blocks, XCD-contiguous tiles"),
    mk_g4x<64, 2, true, kShapeB8NtL>("wN: 4-element lane groups, 2 vectors/thread, 64-thread blocks, XCD-contiguous tiles"),
    mk_g4x<256, 2, true, kShapeB8NtL>("wN: 4-element lane groups, 2 vectors/thread, XCD-contiguous tiles"),
    mk_g4g<256, 2, false, kShapeB8NtL>("w1: grouped state, 2 vectors/thread"),
    mk_g4g<256, 1, false, kShapeB8NtL>("w1: grouped state, 1 vector/thread"),
    mk_g4g<64, 1, false, kShapeB8NtL>("w1: grouped state, 1 vector/thread, 64-thread blocks"),
    mk_g4g<64, 2, false, kShapeB8NtL>("w1: grouped state, 2 vectors/thread, 64-thread blocks"),
    mk_g4g<64, 2, true, kShapeB8NtL>("wN: grouped state, 2 vectors/thread, 64-thread blocks"),
    mk_g4g<256, 2, true, kShapeB8NtL>("wN: grouped state, 2 vectors/thread"),
    mk_g4g<64, 1, true, kShapeB8NtL>("wN: grouped state, 1 vector/thread, 64-thread blocks"),
};
constexpr int kCount = (int)(sizeof kVariants / sizeof kVariants[0]);

thread_local char g_verr[256] = "";

int vfail(const char *msg) {
  snprintf(g_verr, sizeof g_verr, "%s", msg);
  return ZS_ERR_INVALID_ARG;
}

bool aligned16(const void *p) { return ((uintptr_t)p % 16) == 0; }

}  // namespace

extern "C" {

/* Number of variants; ids are 0 .. count-1. */
int zs_variant_count(void) { return kCount; }

/* Static description of variant `id` (NULL for an id out of range). */
const char *zs_variant_name(int id) { return id >= 0 && id < kCount ? kVariants[id].name : nullptr; }

/* Elements per block tile of variant `id` (0 for an id out of range). */
int zs_variant_tile(int id) { return id >= 0 && id < kCount ? kVariants[id].tile : 0; }

/* 1 if variant `id` is for W > 1, 0 if for W = 1, -1 for an id out of range. */
int zs_variant_multi(int id) { return id >= 0 && id < kCount ? (kVariants[id].multi ? 1 : 0) : -1; }

/* Detail of this thread's last refusal ("" after a launch). */
const char *zs_variant_last_error(void) { return g_verr; }

/* One launch of variant `id` on the arguments of zs_step_fused (same
 * meaning; the flag is OR-ed into a->overflow_flag), on `stream`.
 *   blocks_per_cu: residency cap, 0 = none, 1..32;
 *   persist_per_cu: blocks per CU of a persistent variant's grid (1..8;
 *                   ignored by the others).
 * Returns ZS_OK when enqueued; ZS_ERR_INVALID_ARG, before any launch, for an
 * id out of range, a world that does not suit the variant, a dtype, wire or
 * accumulated input it does not support, a null or unaligned pointer, n not
 * a multiple of its tile, or a cap out of range; ZS_ERR_HIP when the launch
 * fails. Asynchronous; nothing is allocated. */
int zs_variant_launch(int id, const zs_step_args *a, uint32_t blocks_per_cu,
                      uint32_t persist_per_cu, void *stream) {
  if (id < 0 || id >= kCount) return vfail("variant id out of range");
  const Variant &v = kVariants[id];
  if (!a || !a->worker_grads || !a->master_in || !a->m_in || !a->v_in || !a->master_out ||
      !a->m_out || !a->v_out || !a->gather_buf || !a->overflow_flag)
    return vfail("null argument");
  if (a->world == 0 || a->world > ZS_MAX_WORLD || a->rank >= a->world)
    return vfail("need 0 < world <= 64 and rank < world");
  if (v.multi != (a->world > 1)) return vfail("variant does not suit this world size");
  if (a->grad_dtype != ZS_BF16 || a->param_dtype != ZS_BF16 || a->wire_dtype != ZS_WIRE_FP32 ||
      a->acc_in)
    return vfail("variants take bf16 gradients and parameters, fp32 sums, no acc_in");
  if (blocks_per_cu > 32 || (v.persistent && (persist_per_cu < 1 || persist_per_cu > 8)))
    return vfail("cap or persistent blocks per CU out of range");
  const uint64_t tile = (uint64_t)v.tile;
  if (a->n == 0 || a->n % tile != 0 || a->n / tile > 0x7fffffffull)
    return vfail("n must be a positive multiple of the variant's tile");
  FusedArgs p{};
  p.world = a->world;
  p.wire = ZS_WIRE_FP32;
  p.n = a->n;
  for (uint32_t j = 0; j < a->world; ++j) {
    const void *g = a->worker_grads[(a->rank + 1 + j) % a->world];
    if (!g || !aligned16(g)) return vfail("null or unaligned gradient buffer");
    p.g.p[j] = static_cast<const uint16_t *>(g);
  }
  for (uint32_t j = a->world; j < ZS_MAX_WORLD; ++j) p.g.p[j] = nullptr;
  p.acc_in = nullptr;
  p.master_in = a->master_in;
  p.m_in = a->m_in;
  p.v_in = a->v_in;
  p.master_out = a->master_out;
  p.m_out = a->m_out;
  p.v_out = a->v_out;
  p.param_out = static_cast<uint16_t *>(a->gather_buf) + a->gather_offset;
  p.flag = a->overflow_flag;
  p.dev = nullptr;
  p.lr = a->hp.lr;
  const void *ptrs[] = {p.master_in, p.m_in, p.v_in, p.master_out, p.m_out, p.v_out, p.param_out};
  for (const void *q : ptrs)
    if (!aligned16(q)) return vfail("operands must be 16-byte aligned");
  if (!zs_host::make_scales(a->world, a->hp.loss_scale, &p.k)) return vfail("bad loss scale");
  if (!zs_host::make_adam(&a->hp, &p.h)) return vfail("step_t must be >= 1");
  int dev = 0, cus = 0, lds_per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess)
    return ZS_ERR_HIP;
  size_t lds = (size_t)v.lds;
  if (blocks_per_cu) {
    /* up to 8: the production launch's rule; above 8 the largest multiple
     * of 1 KB with which exactly `blocks_per_cu` blocks fit a CU */
    int bytes = blocks_per_cu <= 8 ? (lds_per_cu / (int)blocks_per_cu - 1024) / 256 * 256
                                   : lds_per_cu / (int)blocks_per_cu / 1024 * 1024;
    if (blocks_per_cu > 8 && (int)(blocks_per_cu + 1) * bytes <= lds_per_cu)
      return vfail("no LDS size caps residency at that many blocks per CU");
    if (bytes > v.lds) lds = (size_t)bytes;
  }
  if (lds > (size_t)lds_per_cu) return vfail("the variant's LDS exceeds the CU's");
  if (lds > 65536 &&
      hipFuncSetAttribute(v.fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_per_cu) != hipSuccess)
    return ZS_ERR_HIP;
  const uint64_t tiles = a->n / tile;
  uint64_t grid = tiles;
  if (v.persistent) {
    const uint64_t want = (uint64_t)cus * persist_per_cu;
    grid = want < tiles ? want : tiles;
  }
  void *args[] = {&p};
  /* a cooperative launch is refused, not run, unless every block of its
   * grid can be resident at once */
  const hipError_t e =
      v.cooperative
          ? hipLaunchCooperativeKernel(v.fn, dim3((unsigned)grid), dim3((unsigned)v.block), args,
                                       (unsigned)lds, static_cast<hipStream_t>(stream))
          : hipLaunchKernel(v.fn, dim3((unsigned)grid), dim3((unsigned)v.block), args, lds,
                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    snprintf(g_verr, sizeof g_verr, "launch failed: %s", hipGetErrorString(e));
    return ZS_ERR_HIP;
  }
  g_verr[0] = 0;
  return ZS_OK;
}

}  // extern "C"
