/*
 * synth_host.c -- host side of the seeded input generator (see synth_core.h).
 * Fills arrays with the values that synth_dev.hip writes on the device.
 */
#include "synth_core.h"

uint64_t zsg_key_host(uint64_t seed, uint32_t stream, uint32_t worker,
                      uint32_t step, uint32_t micro) {
  return zsg_key(seed, stream, worker, step, micro);
}

void zsg_fill_normal_f32(uint64_t key, uint64_t first, uint64_t n, float ks,
                         float *out) {
  for (uint64_t j = 0; j < n; ++j) out[j] = zsg_normal(zsg_hash(key, first + j), ks);
}

void zsg_fill_uniform_f32(uint64_t key, uint64_t first, uint64_t n, float ku,
                          float *out) {
  for (uint64_t j = 0; j < n; ++j) out[j] = zsg_uniform(zsg_hash(key, first + j), ku);
}

void zsg_fill_grad16(uint64_t key, uint64_t kinj, uint32_t threshold,
                     uint64_t first, uint64_t n, float ks, int dtype,
                     uint16_t *out) {
  for (uint64_t j = 0; j < n; ++j)
    out[j] = zsg_grad16(key, kinj, threshold, first + j, ks, dtype);
}
