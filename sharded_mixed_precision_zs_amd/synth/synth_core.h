/*
 * synth_core.h -- counter-based synthetic inputs, identical on host and device.
 *
 * Seeded input generation only: this file holds none of the shard step's
 * arithmetic (no sums, no casts by rounding, no optimizer math). It is
 * compiled twice, by gcc for the host library and by hipcc for the device
 * library, and both produce the same bits for the same (key, index).
 *
 * Definition.
 *   sm(x)      = SplitMix64 output function (Steele, Lea and Flood, "Fast
 *                splittable pseudorandom number generators", OOPSLA 2014):
 *                z = x + G; z = (z ^ z>>30) * C1; z = (z ^ z>>27) * C2;
 *                return z ^ z>>31.
 *   key        = sm(sm(sm(sm(seed) ^ stream) ^ worker) ^ (step<<32 | micro))
 *   hash(k, i) = sm(k + i*G), the (i+1)-th output of SplitMix64 seeded at k.
 *   normal     = (float)(u0+u1+u2+u3 - 131070) * ks, with u0..u3 the four
 *                16-bit fields of the hash (Irwin-Hall, exact in fp32) and
 *                ks = sigma / sqrt((2^32-1)/3) rounded to fp32 by the caller;
 *                a single fp32 multiply, so host and device agree bit for bit.
 *   uniform    = (float)(hash >> 40) * ku, ku = hi / 2^24 rounded to fp32.
 *   16-bit     = the fp32 value truncated toward zero to bf16 or fp16 (a bit
 *                selection, deliberately not the step's nearest-even rounding).
 *   injection  = if (hash(kinj, i) >> 32) < threshold the value is replaced by
 *                +inf, -inf or a quiet NaN (low two hash bits 0, 1, else).
 */
#ifndef ZS_SYNTH_CORE_H
#define ZS_SYNTH_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define ZSG_FN static inline __host__ __device__
#else
#define ZSG_FN static inline
#endif

#define ZSG_GOLDEN 0x9E3779B97F4A7C15ull
#define ZSG_C1 0xBF58476D1CE4E5B9ull
#define ZSG_C2 0x94D049BB133111EBull

enum { ZSG_BF16 = 0, ZSG_FP16 = 1 };

ZSG_FN uint64_t zsg_sm(uint64_t x) {
  uint64_t z = x + ZSG_GOLDEN;
  z = (z ^ (z >> 30)) * ZSG_C1;
  z = (z ^ (z >> 27)) * ZSG_C2;
  return z ^ (z >> 31);
}

ZSG_FN uint64_t zsg_key(uint64_t seed, uint32_t stream, uint32_t worker,
                        uint32_t step, uint32_t micro) {
  uint64_t k = zsg_sm(seed);
  k = zsg_sm(k ^ (uint64_t)stream);
  k = zsg_sm(k ^ (uint64_t)worker);
  return zsg_sm(k ^ (((uint64_t)step << 32) | (uint64_t)micro));
}

ZSG_FN uint64_t zsg_hash(uint64_t key, uint64_t i) {
  return zsg_sm(key + i * ZSG_GOLDEN);
}

ZSG_FN float zsg_normal(uint64_t h, float ks) {
  int32_t s = (int32_t)(h & 0xffffu) + (int32_t)((h >> 16) & 0xffffu) +
              (int32_t)((h >> 32) & 0xffffu) + (int32_t)(h >> 48);
  return (float)(s - 131070) * ks;
}

ZSG_FN float zsg_uniform(uint64_t h, float ku) {
  return (float)(uint32_t)(h >> 40) * ku;
}

ZSG_FN uint32_t zsg_bits(float x) {
  union { float f; uint32_t u; } c;
  c.f = x;
  return c.u;
}

/* Truncate toward zero to a 16-bit float (bit selection, no rounding). */
ZSG_FN uint16_t zsg_trunc16(float x, int dtype) {
  uint32_t u = zsg_bits(x);
  if (dtype == ZSG_BF16) return (uint16_t)(u >> 16);
  uint32_t sign = (u >> 16) & 0x8000u;
  int32_t e = (int32_t)((u >> 23) & 0xffu) - 127;
  uint32_t m = (u & 0x7fffffu) | 0x800000u;
  if (((u >> 23) & 0xffu) == 0xffu)
    return (uint16_t)(sign | ((u & 0x7fffffu) ? 0x7e00u : 0x7c00u));
  if (e > 15) return (uint16_t)(sign | 0x7bffu);          /* clamp to max  */
  if (e >= -14)                                              /* normal        */
    return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | ((u >> 13) & 0x3ffu));
  if (e < -24) return (uint16_t)sign;                        /* below 2^-24   */
  return (uint16_t)(sign | (m >> (uint32_t)(-1 - e)));       /* subnormal     */
}

ZSG_FN uint16_t zsg_special16(uint64_t h, int dtype) {
  uint32_t kind = (uint32_t)(h & 3u);
  if (dtype == ZSG_BF16) return kind == 0 ? 0x7f80u : kind == 1 ? 0xff80u : 0x7fc0u;
  return kind == 0 ? 0x7c00u : kind == 1 ? 0xfc00u : 0x7e00u;
}

/* One 16-bit gradient value at flat index i. */
ZSG_FN uint16_t zsg_grad16(uint64_t key, uint64_t kinj, uint32_t threshold,
                           uint64_t i, float ks, int dtype) {
  if (threshold) {
    uint64_t hi = zsg_hash(kinj, i);
    if ((uint32_t)(hi >> 32) < threshold) return zsg_special16(hi, dtype);
  }
  return zsg_trunc16(zsg_normal(zsg_hash(key, i), ks), dtype);
}

#endif /* ZS_SYNTH_CORE_H */
