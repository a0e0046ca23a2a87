/*
 * synth_dev.hip -- device side of the seeded input generator (see
 * synth_core.h). Writes the same bits as synth_host.c, straight into HBM, so
 * inputs too large for host memory never cross PCIe. Launches are
 * grid-stride loops over 64-bit indices; every thread exits after its last
 * element.
 */
#include <hip/hip_runtime.h>

#include "synth_core.h"

namespace {

constexpr int kBlock = 256;

unsigned grid_for(uint64_t n) {
  uint64_t blocks = (n + kBlock - 1) / kBlock;
  const uint64_t cap = 256ull * 64ull;  /* enough waves to stream HBM */
  return (unsigned)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

__global__ void fill_normal_f32(uint64_t key, uint64_t first, uint64_t n,
                                float ks, float *out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = zsg_normal(zsg_hash(key, first + j), ks);
}

__global__ void fill_uniform_f32(uint64_t key, uint64_t first, uint64_t n,
                                 float ku, float *out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = zsg_uniform(zsg_hash(key, first + j), ku);
}

__global__ void fill_grad16(uint64_t key, uint64_t kinj, uint32_t threshold,
                            uint64_t first, uint64_t n, float ks, int dtype,
                            uint16_t *out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = zsg_grad16(key, kinj, threshold, first + j, ks, dtype);
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : -1; }

}  // namespace

extern "C" {

int zsg_dev_fill_normal_f32(uint64_t key, uint64_t first, uint64_t n, float ks,
                            float *out, void *stream) {
  if (n == 0) return 0;
  if (!out) return -1;
  hipLaunchKernelGGL(fill_normal_f32, dim3(grid_for(n)), dim3(kBlock), 0,
                     (hipStream_t)stream, key, first, n, ks, out);
  return launch_status();
}

int zsg_dev_fill_uniform_f32(uint64_t key, uint64_t first, uint64_t n,
                             float ku, float *out, void *stream) {
  if (n == 0) return 0;
  if (!out) return -1;
  hipLaunchKernelGGL(fill_uniform_f32, dim3(grid_for(n)), dim3(kBlock), 0,
                     (hipStream_t)stream, key, first, n, ku, out);
  return launch_status();
}

int zsg_dev_fill_grad16(uint64_t key, uint64_t kinj, uint32_t threshold,
                        uint64_t first, uint64_t n, float ks, int dtype,
                        uint16_t *out, void *stream) {
  if (n == 0) return 0;
  if (!out || (dtype != ZSG_BF16 && dtype != ZSG_FP16)) return -1;
  hipLaunchKernelGGL(fill_grad16, dim3(grid_for(n)), dim3(kBlock), 0,
                     (hipStream_t)stream, key, kinj, threshold, first, n, ks,
                     dtype, out);
  return launch_status();
}

}  // extern "C"
