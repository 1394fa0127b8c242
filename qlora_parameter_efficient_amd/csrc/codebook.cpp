// NF4 codebook, built on the host in double precision.
//
// "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ..."
// (llms.blog), section "1. 4-bit NormalFloat (NF4) Quantization": the 2^4
// levels are quantiles of N(0, 1) normalised to [-1, 1].  The printed
// midpoint formula has infinite outer terms and no exact zero; the levels
// used here are the asymmetric quantile set with an exact zero: 8 positive
// quantiles at probabilities 1/2 + (p_top - 1/2) j / 8 (j = 1..8), 7 negative
// ones mirrored from 1/2 + (p_top - 1/2) j / 7 (j = 1..7), and 0, all divided
// by the quantile at p_top = 1 - (1/32 + 1/30) / 2 (half of a bin of the
// 16- and 15-bin grids the two sides use).
//
// The symmetric variant reads the midpoint formula literally: level i is the
// mean of the normal quantiles at i/16 and (i+1)/16 for i = 0..15, with the
// infinite end quantiles taken at probabilities delta and 1 - delta (the same
// half-bin delta), divided by the largest level; it is symmetric and holds no
// zero.  Its negative half is the exact mirror of the positive half.
//
// The inverse normal CDF is computed from the C library's erfc: bracketing
// bisection followed by Newton steps, which converges to double precision.
#include <cmath>
#include <cstring>
#include <mutex>

#include "common.h"

namespace lq {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int i = 0; i < 80; ++i) {
    double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int i = 0; i < 3; ++i) x -= (normal_cdf(x) - p) / normal_pdf(x);
  return x;
}

constexpr double kDelta = 0.5 * (1.0 / 32.0 + 1.0 / 30.0);

void fill_thresholds(NF4Table& t) {
  for (int i = 0; i < 15; ++i) {
    float s = t.cb[i] + t.cb[i + 1];  // float32 sum, then exact halving
    t.thr[i] = s * 0.5f;
  }
}

NF4Table build_symmetric_table() {
  NF4Table t;
  std::memset(&t, 0, sizeof(t));
  // quantiles at 8/16 .. 15/16 and 1 - delta; Q(1/2) = 0 exactly
  double q[9];
  q[0] = 0.0;
  for (int j = 9; j <= 15; ++j) q[j - 8] = normal_quantile(j / 16.0);
  q[8] = normal_quantile(1.0 - kDelta);
  double lv[8];  // levels 8..15
  for (int i = 0; i < 8; ++i) lv[i] = 0.5 * (q[i] + q[i + 1]);
  for (int i = 0; i < 8; ++i) {
    t.cb[8 + i] = (float)(lv[i] / lv[7]);
    t.cb[7 - i] = -t.cb[8 + i];
  }
  fill_thresholds(t);
  return t;
}

NF4Table build_table() {
  NF4Table t;
  std::memset(&t, 0, sizeof(t));
  const double p_top = 1.0 - kDelta;
  const double z_top = normal_quantile(p_top);
  double lv[16];
  // ascending: 7 negatives (most negative first), zero, 8 positives
  for (int j = 7; j >= 1; --j) lv[7 - j] = -normal_quantile(0.5 + (p_top - 0.5) * j / 7.0);
  lv[7] = 0.0;
  for (int j = 1; j <= 8; ++j) lv[7 + j] = normal_quantile(0.5 + (p_top - 0.5) * j / 8.0);
  for (int i = 0; i < 16; ++i) t.cb[i] = (float)(lv[i] / z_top);
  t.cb[7] = 0.0f;
  fill_thresholds(t);
  return t;
}

}  // namespace

const NF4Table& nf4_table(int32_t codebook) {
  static std::once_flag once;
  static NF4Table tables[2];
  std::call_once(once, [] {
    tables[LQ_CB_NF4] = build_table();
    tables[LQ_CB_NF4_SYMMETRIC] = build_symmetric_table();
  });
  return tables[codebook == LQ_CB_NF4_SYMMETRIC ? LQ_CB_NF4_SYMMETRIC : LQ_CB_NF4];
}

}  // namespace lq
