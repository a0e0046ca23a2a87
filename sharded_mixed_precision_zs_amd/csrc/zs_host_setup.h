/*
 * zs_host_setup.h -- the per-step scalars every launch of the fused step
 * needs, formed on the host: the reciprocals of the world size and the loss
 * scale when they are exact powers of two, and the AdamW constants (formed
 * in binary64 from the fp32 hyper-parameters and rounded once to fp32; beta^t
 * by t repeated products). Shared by libzeroshard and the measurement
 * library of kernel variants, so both launch the same arithmetic. Host code
 * only; include after zs_kernels.h.
 */
#ifndef ZS_HOST_SETUP_H
#define ZS_HOST_SETUP_H

#include <math.h>
#include <stdint.h>

#include "zs_host_powers.h"
#include "zs_kernels.h"

namespace zs_host {

/* Exact power of two with a normal reciprocal: then x * (1/p) == x / p. */
inline bool exact_pow2(float p, float *inv) {
  if (!(p > 0.0f) || !isfinite(p)) return false;
  int e;
  float m = frexpf(p, &e);         /* p = m * 2^e, m in [0.5, 1) */
  if (m != 0.5f) return false;
  int k = e - 1;                   /* p = 2^k */
  if (k < -126 || k > 126) return false;
  *inv = ldexpf(1.0f, -k);
  return true;
}

/* The world and loss-scale half of a launch's constants; false for a loss
 * scale that is not finite and > 0. */
inline bool make_scales(uint32_t world, float loss_scale, zs::Scales *k) {
  if (!(loss_scale > 0.0f) || !isfinite(loss_scale)) return false;
  k->wf = (float)world;
  k->w_pow2 = exact_pow2(k->wf, &k->inv_w) ? 1 : 0;
  if (!k->w_pow2) k->inv_w = 0.0f;
  k->sf = loss_scale;
  k->s_pow2 = exact_pow2(loss_scale, &k->inv_s) ? 1 : 0;
  if (!k->s_pow2) k->inv_s = 0.0f;
  return true;
}

/* Per-step AdamW scalars in double, rounded once to fp32; false for
 * step_t == 0. */
inline bool make_adam(const zs_adamw_hparams *hp, zs::AdamK *k) {
  if (hp->step_t == 0) return false;
  double b1 = hp->beta1, b2 = hp->beta2, lr = hp->lr, wd = hp->weight_decay;
  double b1t, b2t;
  beta_powers(hp->beta1, hp->beta2, hp->step_t, &b1t, &b2t);
  k->alpha = (float)(lr / (1.0 - b1t));
  k->b2 = (float)sqrt(1.0 - b2t);
  k->delta = (float)(1.0 - lr * wd);
  k->c1 = (float)(1.0 - b1);
  k->c2 = (float)(1.0 - b2);
  k->beta1 = hp->beta1;
  k->beta2 = hp->beta2;
  k->eps = hp->eps;
  return true;
}

}  // namespace zs_host

#endif /* ZS_HOST_SETUP_H */
