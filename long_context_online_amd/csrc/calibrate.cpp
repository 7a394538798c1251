// Host-only threshold calibration: quantile inversion of critical values and the least-squares
// fit of the calibration model lambda * L = alpha * exp(beta * s) (pages: xllm-io review,
// 核心公式 threshold calibration lambda = a / L and calibration model; 模型组件 calibration
// module, one forward pass over a sample).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <vector>

#include "../../include/blasst.h"
#include "host.hpp"

using blasst::fail;
using blasst::ok;

extern "C" {

blasst_status blasst_calib_quantile(const float *crit, int64_t n, double target_s, double *ln_lambda) {
  if (!crit || !ln_lambda) return fail(BLASST_ERR_INVALID_ARG, "crit and ln_lambda must be non-NULL");
  if (n < 1) return fail(BLASST_ERR_INVALID_ARG, "n must be >= 1");
  if (!(target_s >= 0.0 && target_s <= 1.0)) return fail(BLASST_ERR_INVALID_ARG, "target_s must lie in [0, 1]");
  std::vector<double> c;
  c.reserve((size_t)n);
  for (int64_t i = 0; i < n; ++i)
    if (!std::isnan(crit[i])) c.push_back((double)crit[i]);
  if (c.empty()) return fail(BLASST_ERR_INVALID_ARG, "every critical value is NaN");
  std::sort(c.begin(), c.end());
  const int64_t N = (int64_t)c.size();
  const int64_t k = (int64_t)std::ceil(target_s * (double)N);
  if (k <= 0) {
    *ln_lambda = -INFINITY;
    return ok();
  }
  const double lo = c[(size_t)(k - 1)];
  const double hi = k < N ? c[(size_t)k] : INFINITY;
  double mid;
  if (std::isinf(lo) && lo > 0) {
    mid = 0.0;
  } else if (lo == hi) {
    mid = hi;
  } else if (std::isfinite(hi)) {
    mid = 0.5 * (lo + hi);
  } else {
    mid = lo + 1.0;
  }
  *ln_lambda = std::min(0.0, mid);
  return ok();
}

blasst_status blasst_calibrate(const double *L, const double *s, const double *lambda, int32_t n, double *alpha,
                               double *beta, double *rmse) {
  if (!L || !s || !lambda || !alpha || !beta) return fail(BLASST_ERR_INVALID_ARG, "L, s, lambda, alpha and beta must be non-NULL");
  if (n < 2) return fail(BLASST_ERR_INVALID_ARG, "at least two points are needed, got %d", (int)n);
  double xm = 0, ym = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (!(lambda[i] > 0.0) || !(L[i] > 0.0) || !std::isfinite(s[i]) || !std::isfinite(lambda[i]) ||
        !std::isfinite(L[i]))
      return fail(BLASST_ERR_INVALID_ARG, "point %d: lambda and L must be finite and > 0, s finite", (int)i);
    xm += s[i];
    ym += std::log(lambda[i] * L[i]);
  }
  xm /= n;
  ym /= n;
  double sxx = 0, sxy = 0;
  for (int32_t i = 0; i < n; ++i) {
    const double dx = s[i] - xm;
    sxx += dx * dx;
    sxy += dx * (std::log(lambda[i] * L[i]) - ym);
  }
  if (sxx == 0.0) return fail(BLASST_ERR_INVALID_ARG, "the points need at least two distinct s values");
  const double b = sxy / sxx;
  const double la = ym - b * xm;
  double sse = 0;
  for (int32_t i = 0; i < n; ++i) {
    const double r = std::log(lambda[i] * L[i]) - (la + b * s[i]);
    sse += r * r;
  }
  *alpha = std::exp(la);
  *beta = b;
  if (rmse) *rmse = std::sqrt(sse / n);
  return ok();
}

double blasst_lambda_for(double alpha, double beta, double s, double L) {
  if (!(L > 0.0)) return NAN;
  return std::min(1.0, alpha * std::exp(beta * s) / L);
}

}  // extern "C"
