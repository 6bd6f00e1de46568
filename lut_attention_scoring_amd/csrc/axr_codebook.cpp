// Host-side design-time codebook: the Lloyd-Max quantizer for N(0, 1/d).
//
// "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract:
// after the orthogonal transform each coordinate of a unit key is close to
// N(0, 1/d), so the optimal scalar quantizer depends only on d and b and is
// fixed at design time.  The quantizer is found by iterating the two
// Lloyd-Max conditions (Lloyd 1982; Max 1960) to their fixed point:
// midpoint thresholds and conditional-mean centroids.  The density is
// symmetric and log-concave, so the fixed point is unique and symmetric; the
// iteration here runs on the positive half of the unit-variance problem and
// mirrors and scales the result, which makes the middle threshold exactly 0.

#include <cmath>
#include <map>
#include <mutex>
#include <utility>

#include "axr_internal.h"

namespace axr {
namespace {

// Standard normal density and upper tail P(Z > x), accurate in the tails.
inline double npdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) * 0.39894228040143267794;  // 1/sqrt(2 pi)
}
inline double upper_tail(double x) { return 0.5 * std::erfc(x * 0.70710678118654752440); }

}  // namespace

void solve_codebook(int d, int b, Codebook* out) {
  const int levels = 1 << b;
  const int half = levels / 2;
  // Positive half: centroids pc[0..half), edges pe[0] = 0 < pe[1] < ... < pe[half] = inf.
  double pc[kMaxLevels / 2], pe[kMaxLevels / 2 + 1];
  for (int i = 0; i < half; ++i) pc[i] = 3.0 * (i + 0.5) / half;  // any start converges
  pe[0] = 0.0;
  pe[half] = INFINITY;
  for (int iter = 0; iter < 100000; ++iter) {
    for (int i = 1; i < half; ++i) pe[i] = 0.5 * (pc[i - 1] + pc[i]);
    double change = 0.0;
    for (int i = 0; i < half; ++i) {
      // E[Z | pe[i] < Z <= pe[i+1]] = (phi(lo) - phi(hi)) / (Q(lo) - Q(hi))
      const double mass = upper_tail(pe[i]) - upper_tail(pe[i + 1]);
      const double next = (npdf(pe[i]) - npdf(pe[i + 1])) / mass;
      change = std::fmax(change, std::fabs(next - pc[i]));
      pc[i] = next;
    }
    if (change == 0.0) break;
  }
  for (int i = 1; i < half; ++i) pe[i] = 0.5 * (pc[i - 1] + pc[i]);
  const double sigma = 1.0 / std::sqrt(static_cast<double>(d));
  out->d = d;
  out->b = b;
  for (int i = 0; i < half; ++i) {
    out->centroid[half + i] = sigma * pc[i];
    out->centroid[half - 1 - i] = -sigma * pc[i];
  }
  out->threshold[half - 1] = 0.0;
  for (int i = 1; i < half; ++i) {
    out->threshold[half - 1 + i] = sigma * pe[i];
    out->threshold[half - 1 - i] = -sigma * pe[i];
  }
}

const Codebook& cached_codebook(int d, int b) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, Codebook> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(d, b);
  auto it = cache.find(key);
  if (it == cache.end()) {
    Codebook cb;
    solve_codebook(d, b, &cb);
    it = cache.emplace(key, cb).first;
  }
  return it->second;
}

}  // namespace axr
