// Host construction of the NF4 levels and decision thresholds (and of the
// evenly spaced 4-bit levels of the format variants).
//
// The levels sit at quantiles of the standard normal distribution ([P1] "The
// mechanism in brief"; [P4] "NF4 and double quantisation"): 8 positive
// quantiles at probabilities 0.5 + (d - 0.5) * j / 8 (j = 1..8), 7 negative at
// 0.5 + (d - 0.5) * j / 7 (j = 1..7) mirrored, and an exact zero; everything is
// divided by the quantile at d, so the extremes are exactly -1 and +1.  The
// tail offset d = ((1 - 1/30) + (1 - 1/32)) / 2 is not given by the pages; it
// is the offset of the construction in the paper they cite.
//
// The inverse normal here is bisection on Phi(x) = erfc(-x / sqrt 2) / 2 in
// double precision, to adjacent doubles: accurate to ~1e-15 relative, far
// inside the smallest fp32 rounding margin of any level.
#include <cmath>
#include <limits>
#include <mutex>
#include <stdexcept>

#include "common.h"

namespace qlora {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 4000; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double elo = std::fabs(normal_cdf(lo) - p), ehi = std::fabs(normal_cdf(hi) - p);
  return elo < ehi ? lo : hi;
}

float round_down_f32(double x) {
  float f = (float)x;  // round to nearest even
  if ((double)f > x) f = std::nextafterf(f, -INFINITY);
  return f;
}

void set_thresholds(Nf4Consts& c) {
  for (int i = 0; i < 15; ++i) {
    double mid = ((double)c.level[i] + (double)c.level[i + 1]) * 0.5;  // exact
    c.thr[i] = round_down_f32(mid);
  }
}

// Evenly spaced levels over [-1, 1] ("plain int4", the alternative NF4 is
// compared with in [P2] "Follow-up questions to expect"): fp32 of
// -1 + 2 i / 15.
Nf4Consts build_uniform() {
  Nf4Consts c;
  for (int i = 0; i < 16; ++i) c.level[i] = (float)(-1.0 + 2.0 * i / 15.0);
  set_thresholds(c);
  return c;
}

QuantSearch build_search(const Nf4Consts& c) {
  QuantSearch qs;
  for (int i = 0; i < 14; ++i)  // the search needs thresholds > 3 cells apart
    if ((double)c.thr[i + 1] - (double)c.thr[i] <= 3.0 / 128.0) throw std::logic_error("thresholds too close");
  for (int i = 0; i < 256; ++i) {
    const double start = i == 0 ? -std::numeric_limits<double>::infinity() : (i - 1) / 128.0 - 1.0;
    int n = 0;
    for (int t = 0; t < 15; ++t) n += (double)c.thr[t] < start ? 1 : 0;
    qs.cand[i] = (uint8_t)n;
  }
  for (int t = 0; t < 15; ++t) qs.thr16[t] = c.thr[t];
  qs.thr16[15] = std::numeric_limits<float>::infinity();
  return qs;
}

Nf4Consts build() {
  const double d = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  const double step = d - 0.5;
  const double top = normal_quantile(d);
  double lv[16];
  // ascending: 7 negatives (most negative first), zero, 8 positives
  for (int j = 7; j >= 1; --j) lv[7 - j] = -normal_quantile(0.5 + step * (j / 7.0)) / top;
  lv[7] = 0.0;
  for (int j = 1; j <= 8; ++j) lv[7 + j] = normal_quantile(0.5 + step * (j / 8.0)) / top;
  Nf4Consts c;
  for (int i = 0; i < 16; ++i) c.level[i] = (float)lv[i];
  set_thresholds(c);
  return c;
}

}  // namespace

const Nf4Consts& nf4_consts() {
  static std::once_flag once;
  static Nf4Consts consts;
  std::call_once(once, [] { consts = build(); });
  return consts;
}

const QuantSearch& quant_search() {
  static std::once_flag once;
  static QuantSearch qs;
  std::call_once(once, [] { qs = build_search(nf4_consts()); });
  return qs;
}

const Nf4Consts& int4_consts() {
  static std::once_flag once;
  static Nf4Consts consts;
  std::call_once(once, [] { consts = build_uniform(); });
  return consts;
}

const QuantSearch& quant_search_int4() {
  static std::once_flag once;
  static QuantSearch qs;
  std::call_once(once, [] { qs = build_search(int4_consts()); });
  return qs;
}

}  // namespace qlora
