// Per-problem budget split from pilot MSEs (gist.science page, section 2,
// "Adaptive Budget Allocation": the total budget is redistributed in
// proportion to the square root of the pilot MSE).
//
// Pure host code in IEEE double.  Compiled with -ffp-contract=off so that no
// multiply-add is fused: every sum runs over problems in increasing order and
// every share is (R * w) / S, which makes the result reproducible bit for bit
// by any implementation that performs the same operations.
#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/kvsculpt.h"

extern "C" kvs_status kvs_allocate_budget(const double* mse, int32_t P, int64_t K_total, double alpha,
                                          int32_t k_min, int32_t k_max, int32_t* k_out) {
  if (!mse || !k_out || P < 1 || k_min < 1 || k_min > k_max) return KVS_ERR_INVALID;
  if (K_total < (int64_t)P * k_min || K_total > (int64_t)P * k_max) return KVS_ERR_INVALID;
  std::vector<double> w(P);
  for (int p = 0; p < P; ++p) {
    const double v = mse[p];
    if (!(v >= 0.0) || std::isinf(v)) return KVS_ERR_INVALID;
    w[p] = (alpha == 0.5) ? std::sqrt(v) : (alpha == 1.0 ? v : std::pow(v, alpha));
  }
  double total = 0.0;
  for (int p = 0; p < P; ++p) total += w[p];
  if (total == 0.0)
    for (int p = 0; p < P; ++p) w[p] = 1.0;

  // Bounded water-filling: x_p = clamp(t w_p, k_min, k_max), sum x = K_total.
  // Each round fixes the violators that the clamped total proves final.
  std::vector<int> fixed(P, 0);        // 0 = free, else the bound it sits at
  std::vector<double> x(P, 0.0);
  for (;;) {
    double R = (double)K_total;
    for (int p = 0; p < P; ++p)
      if (fixed[p]) R -= (double)fixed[p];
    double S = 0.0;
    int nfree = 0;
    for (int p = 0; p < P; ++p)
      if (!fixed[p]) {
        S += w[p];
        ++nfree;
      }
    if (nfree == 0) break;
    bool any_hi = false, any_lo = false;
    for (int p = 0; p < P; ++p) {
      if (fixed[p]) continue;
      x[p] = (S > 0.0) ? (R * w[p]) / S : R / (double)nfree;
      if (x[p] > (double)k_max) any_hi = true;
      if (x[p] < (double)k_min) any_lo = true;
    }
    if (!any_hi && !any_lo) break;
    double C = 0.0;
    for (int p = 0; p < P; ++p) {
      if (fixed[p]) continue;
      C += x[p] > (double)k_max ? (double)k_max : (x[p] < (double)k_min ? (double)k_min : x[p]);
    }
    const bool fix_lo = !(C < R);     // C > R or C == R
    const bool fix_hi = !(C > R);     // C < R or C == R
    for (int p = 0; p < P; ++p) {
      if (fixed[p]) continue;
      if (fix_hi && x[p] > (double)k_max) fixed[p] = k_max;
      else if (fix_lo && x[p] < (double)k_min) fixed[p] = k_min;
    }
  }

  // Floors, then the remaining units to the largest fractional parts
  // (ties: lower problem index first).
  int64_t used = 0;
  std::vector<int> order;
  std::vector<double> frac(P, 0.0);
  for (int p = 0; p < P; ++p) {
    if (fixed[p]) {
      k_out[p] = fixed[p];
    } else {
      const double fl = std::floor(x[p]);
      k_out[p] = (int32_t)fl;
      frac[p] = x[p] - fl;
      order.push_back(p);
    }
    used += k_out[p];
  }
  // stable insertion sort by descending fraction (P is small)
  for (size_t i = 1; i < order.size(); ++i) {
    const int v = order[i];
    size_t j = i;
    while (j > 0 && frac[order[j - 1]] < frac[v]) {
      order[j] = order[j - 1];
      --j;
    }
    order[j] = v;
  }
  int64_t left = K_total - used;
  for (size_t i = 0; i < order.size() && left > 0; ++i) {
    const int p = order[i];
    if (k_out[p] < k_max) {
      k_out[p] += 1;
      --left;
    }
  }
  return left == 0 ? KVS_OK : KVS_ERR_INVALID;
}

// Two-level split (the same page and section: allocation at the layer and
// the KV-head level): layer signal = mean of its heads' MSE (summed in head
// order, divided by the head count), layer budgets by the flat split with
// bounds [heads k_min, min(heads k_max, K_total)], then each layer's budget
// over its heads by the flat split on their own MSE.
extern "C" kvs_status kvs_allocate_budget_two_level(const double* mse, int32_t layers,
                                                    int32_t heads, int64_t K_total, double alpha,
                                                    int32_t k_min, int32_t k_max, int32_t* k_out) {
  if (!mse || !k_out || layers < 1 || heads < 1 || k_min < 1 || k_min > k_max) return KVS_ERR_INVALID;
  const int64_t P = (int64_t)layers * heads;
  if (P > 0x7fffffff || K_total < P * k_min || K_total > P * k_max) return KVS_ERR_INVALID;
  const int64_t lmax = std::min<int64_t>((int64_t)heads * k_max, K_total);
  if (lmax > 0x7fffffff || (int64_t)heads * k_min > 0x7fffffff) return KVS_ERR_INVALID;
  std::vector<double> lmse(layers);
  for (int l = 0; l < layers; ++l) {
    double acc = 0.0;
    for (int h = 0; h < heads; ++h) {
      const double v = mse[(int64_t)l * heads + h];
      if (!(v >= 0.0) || std::isinf(v)) return KVS_ERR_INVALID;
      acc += v;
    }
    lmse[l] = acc / (double)heads;
  }
  std::vector<int32_t> kl(layers);
  kvs_status s = kvs_allocate_budget(lmse.data(), layers, K_total, alpha, heads * k_min, (int32_t)lmax,
                                     kl.data());
  if (s != KVS_OK) return s;
  for (int l = 0; l < layers; ++l) {
    s = kvs_allocate_budget(mse + (int64_t)l * heads, heads, kl[l], alpha, k_min, k_max,
                            k_out + (int64_t)l * heads);
    if (s != KVS_OK) return s;
  }
  return KVS_OK;
}
