// The NF4 codebook used by the kernels, computed on the host once per process.
//
// Levels: standard-normal quantiles at evenly spaced probabilities between
// P = ((1 - 1/30) + (1 - 1/32)) / 2 and 1/2 (9 points for the positive side, 8 for the
// negative side, the point 1/2 dropped on both), an exact zero, all divided by the quantile at
// P ("Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @2:19: levels
// placed where normally distributed weights fall; the construction of QLoRA, arXiv
// 2305.14314, which "An 8B Fine-Tune Now Fits in 4 GB of VRAM" links).
//
// The quantile is found by bisection on the normal CDF written with erfc, then polished with
// Newton steps, in fp64; each level is then rounded to fp32, and each midpoint is the fp64
// mean of two adjacent fp32 levels rounded to fp32.

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.h"

namespace lsn {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200 && hi - lo > 0.0; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int i = 0; i < 2; ++i) x -= (normal_cdf(x) - p) / normal_pdf(x);
  return x;
}

std::vector<double> evenly_spaced(double start, double stop, int num) {
  std::vector<double> v(num);
  const double step = (stop - start) / (num - 1);
  for (int i = 0; i < num; ++i) v[i] = start + i * step;
  return v;
}

Nf4Table build_table() {
  const double p_max = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  const double z_max = normal_quantile(p_max);
  std::vector<double> levels;
  const std::vector<double> pos = evenly_spaced(p_max, 0.5, 9);
  const std::vector<double> neg = evenly_spaced(p_max, 0.5, 8);
  for (int i = 0; i < 8; ++i) levels.push_back(normal_quantile(pos[i]));
  for (int i = 0; i < 7; ++i) levels.push_back(-normal_quantile(neg[i]));
  levels.push_back(0.0);
  std::sort(levels.begin(), levels.end());
  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.q[i] = (float)(levels[i] / z_max);
  // the two end levels are the quantile at P divided by itself: exactly -1 and +1
  for (int i = 0; i < 15; ++i) t.m[i] = (float)(((double)t.q[i] + (double)t.q[i + 1]) / 2.0);
  return t;
}

}  // namespace

const Nf4Table &nf4_table() {
  static std::once_flag once;
  static Nf4Table table;
  std::call_once(once, [] { table = build_table(); });
  return table;
}

}  // namespace lsn
