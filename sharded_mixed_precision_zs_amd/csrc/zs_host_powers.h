/*
 * zs_host_powers.h -- beta1^t and beta2^t for the bias corrections, formed in
 * binary64 by t repeated multiplications starting from 1 (the reading the
 * library and its tests use). A per-thread cache continues the product from
 * the last (beta1, beta2, t) asked for when t has not decreased: the same
 * multiplications in the same order, so the same bits, but O(1) per step
 * when t grows by one (a training loop at t = 10^6 would otherwise spend
 * milliseconds per step on the host). Host code only.
 */
#ifndef ZS_HOST_POWERS_H
#define ZS_HOST_POWERS_H

#include <stdint.h>

namespace zs_host {

inline void beta_powers(float beta1, float beta2, uint64_t t, double *b1t, double *b2t) {
  struct Cache {
    float beta1 = 0.0f, beta2 = 0.0f;
    uint64_t t = 0;
    double p1 = 1.0, p2 = 1.0;
    bool valid = false;
  };
  static thread_local Cache c;
  if (!c.valid || c.beta1 != beta1 || c.beta2 != beta2 || c.t > t) {
    c.beta1 = beta1;
    c.beta2 = beta2;
    c.t = 0;
    c.p1 = 1.0;
    c.p2 = 1.0;
    c.valid = true;
  }
  const double d1 = beta1, d2 = beta2;
  for (; c.t < t; ++c.t) {
    c.p1 *= d1;
    c.p2 *= d2;
  }
  *b1t = c.p1;
  *b2t = c.p2;
}

}  // namespace zs_host

#endif /* ZS_HOST_POWERS_H */
