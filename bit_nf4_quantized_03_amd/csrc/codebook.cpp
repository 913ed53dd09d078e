// Host-side derivation of the NF4 levels and decision thresholds.
//
// NF4 is built for normally distributed weights and is finer near zero
// (Guanaco topic page, "Technical Innovations: NormalFloat4"); a 4-bit type
// with an exact zero that uses all 16 values (ai-papercheck QLoRA review,
// finding on paper p.5 Section 3). The levels are quantiles of N(0, 1) at
// equally spaced probabilities: 8 on the positive side and 7 on the negative
// side between 1/2 and p_max = 1 - (1/32 + 1/30)/2 (the centre of the outermost
// equal-mass bin, averaged over the 16- and the 15-level views of the
// asymmetric type), plus 0, divided by the quantile at p_max so the ends are
// exactly -1 and +1.
//
// The quantile is found by bisection on the normal CDF written with erfcl in
// long double (64-bit significand), then rounded once to fp32.
#include <cmath>
#include <cfloat>
#include <mutex>
#include <algorithm>

#include "internal.h"

namespace qnf4 {
namespace {

long double normal_cdf(long double x) { return 0.5L * erfcl(-x / sqrtl(2.0L)); }

long double normal_quantile(long double p) {
  long double lo = -40.0L, hi = 40.0L;
  for (int it = 0; it < 200; ++it) {
    long double mid = 0.5L * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5L * (lo + hi);
}

// Largest fp32 <= v for a value v given exactly in double.
float round_down_f32(double v) {
  float f = static_cast<float>(v);
  if (static_cast<double>(f) > v) f = std::nextafterf(f, -INFINITY);
  return f;
}

void set_thresholds(Nf4Tables &t) {
  for (int i = 0; i < 15; ++i) {
    // the sum of two fp32 values of magnitude <= 1 is exact in double
    double mid = (static_cast<double>(t.lv[i]) + static_cast<double>(t.lv[i + 1])) * 0.5;
    t.thr[i] = round_down_f32(mid);
  }
}

// The 4-bit float with one sign bit, two exponent bits (bias 1, exponent
// field 0 subnormal) and one mantissa bit, divided by its largest magnitude
// (6) so that a block's absmax maps to +-1; the FP4 comparison format of the
// paper's Table 4 (QLoRA review, findings on paper p.8 Table 4), whose levels
// the pages leave open. The zero appears once (index 7) and +1 is repeated at
// index 15.
Nf4Tables derive_fp4() {
  long double mag[8];
  for (int e = 0; e < 4; ++e)
    for (int m = 0; m < 2; ++m)
      mag[2 * e + m] = e == 0 ? 0.5L * m : ldexpl(1.0L + 0.5L * m, e - 1);
  Nf4Tables t;
  for (int i = 0; i < 7; ++i) t.lv[i] = static_cast<float>(-mag[7 - i] / mag[7]);
  for (int i = 0; i < 8; ++i) t.lv[7 + i] = static_cast<float>(mag[i] / mag[7]);
  t.lv[15] = 1.0f;
  set_thresholds(t);
  // The threshold between the two +1 entries would sit at exactly 1, where
  // every block's absmax element lands; no scaled value exceeds 1, so any
  // threshold above 1 gives the same codes and keeps the quantizer's fast
  // path away from the exact-division fallback.
  t.thr[14] = 2.0f;
  return t;
}

Nf4Tables derive() {
  const long double p_max = 1.0L - (1.0L / 32.0L + 1.0L / 30.0L) / 2.0L;
  const long double z_max = normal_quantile(p_max);
  long double v[16];
  int k = 0;
  for (int i = 0; i < 7; ++i) {  // negative side, p = p_max ... towards 1/2
    long double p = p_max + (0.5L - p_max) * static_cast<long double>(i) / 7.0L;
    v[k++] = -normal_quantile(p) / z_max;
  }
  v[k++] = 0.0L;
  for (int i = 0; i < 8; ++i) {  // positive side
    long double p = p_max + (0.5L - p_max) * static_cast<long double>(i) / 8.0L;
    v[k++] = normal_quantile(p) / z_max;
  }
  std::sort(v, v + 16);
  Nf4Tables t;
  for (int i = 0; i < 16; ++i) t.lv[i] = static_cast<float>(v[i]);
  set_thresholds(t);
  return t;
}

}  // namespace

const Nf4Tables &nf4_tables() {
  static Nf4Tables tables;
  static std::once_flag once;
  std::call_once(once, [] { tables = derive(); });
  return tables;
}

const Nf4Tables &fp4_tables() {
  static Nf4Tables tables;
  static std::once_flag once;
  std::call_once(once, [] { tables = derive_fp4(); });
  return tables;
}

}  // namespace qnf4
