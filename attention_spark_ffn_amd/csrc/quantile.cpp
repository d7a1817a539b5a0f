// Standard-normal quantile for the statistical top-k threshold
// theta = mean + std * Q(1 - k/d) (Spark Transformer reading notes, section
// "方法详解 / 关键设计", item "Statistical Top-k").
//
// Computed on the host in fp64 by solving the upper-tail equation
//     P(Z > z) = erfc(z / sqrt 2) / 2 = k / d
// with bisection on a bracket followed by Newton steps, using the C library's
// erfc.  The kernels receive z as a scalar.
#include <cmath>
#include <cstdint>

#include "spark_ffn.h"

namespace {

double upper_tail(double z) { return 0.5 * std::erfc(z / std::sqrt(2.0)); }

// z >= 0 with P(Z > z) = t, for 0 < t <= 1/2.
double solve_upper(double t) {
  double lo = 0.0, hi = 1.0;
  while (upper_tail(hi) > t && hi < 64.0) hi *= 2.0;
  for (int i = 0; i < 200 && hi - lo > 1e-15 * (1.0 + hi); ++i) {
    const double mid = 0.5 * (lo + hi);
    if (upper_tail(mid) > t) lo = mid; else hi = mid;
  }
  double z = 0.5 * (lo + hi);
  const double inv_sqrt_2pi = 0.3989422804014327;
  for (int i = 0; i < 3; ++i) {
    const double pdf = inv_sqrt_2pi * std::exp(-0.5 * z * z);
    if (!(pdf > 0.0)) break;
    z += (upper_tail(z) - t) / pdf;  // Newton on P(Z > z) - t, derivative -pdf
  }
  return z;
}

}  // namespace

extern "C" double spark_threshold_z(int64_t k, int64_t d) {
  if (d <= 0 || k <= 0 || k >= d) return std::nan("");
  if (2 * k == d) return 0.0;
  if (2 * k < d) return solve_upper((double)k / (double)d);
  return -solve_upper((double)(d - k) / (double)d);
}
