/*
 * zs_hparams.h -- range check of the AdamW hyper-parameters, shared by the
 * GPU entry points and the host update. The accepted ranges are those of
 * the AdamW parameterisation the library follows (decoupled decay, bias
 * correction): 0 <= beta < 1 keeps 1 - beta^t positive for every t >= 1,
 * and lr, eps and weight_decay are finite and non-negative. Anything else
 * would turn every parameter into inf or NaN without an overflow being
 * reported. Host code only.
 */
#ifndef ZS_HPARAMS_H
#define ZS_HPARAMS_H

#include <math.h>

#include "zeroshard.h"

namespace zs_host {

inline bool beta_ok(float b) { return b >= 0.0f && b < 1.0f; }

inline bool nonneg_finite(float x) { return x >= 0.0f && isfinite(x); }

/* nullptr when the settings are usable, else what is wrong with them. */
inline const char *hparams_problem(const zs_adamw_hparams *hp) {
  if (!nonneg_finite(hp->lr)) return "lr must be finite and >= 0";
  if (!beta_ok(hp->beta1) || !beta_ok(hp->beta2)) return "beta1 and beta2 must lie in [0, 1)";
  if (!nonneg_finite(hp->eps)) return "eps must be finite and >= 0";
  if (!nonneg_finite(hp->weight_decay)) return "weight_decay must be finite and >= 0";
  return nullptr;
}

}  // namespace zs_host

#endif /* ZS_HPARAMS_H */
