// Host-side dual-constraint batch scheduling and its cost model (AdaptiveLoad
// technical summary, section 2.A; load-balance measure, section 4).  See
// include/adaln_sched.h for the contract.  No device code, no HIP calls.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <numeric>
#include <vector>

#include "../../include/adaln_sched.h"

#define ADALN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool budgets_ok(int64_t m_mem, int64_t m_comp, double p) {
  return m_mem >= 0 && m_comp >= 0 && std::isfinite(p) && p > 0.0;
}

// S^k for integral k >= 0, or -1 when it exceeds INT64_MAX.
int64_t ipow_or_overflow(int64_t S, int64_t k) {
  int64_t r = 1;
  for (int64_t i = 0; i < k; ++i) {
    if (r > INT64_MAX / S) return -1;
    r *= S;
  }
  return r;
}

// The compute bound floor(m_comp / S^p).
int64_t compute_bound(int64_t S, int64_t m_comp, double p) {
  if (p == std::floor(p) && p <= 64.0) {
    const int64_t sp = ipow_or_overflow(S, static_cast<int64_t>(p));
    return sp < 0 ? 0 : m_comp / sp;        // S^p > INT64_MAX >= m_comp: bound 0
  }
  const double q = std::floor(static_cast<double>(m_comp) / std::pow(static_cast<double>(S), p));
  if (!(q >= 0.0)) return 0;
  if (q >= 9.2e18) return INT64_MAX;
  return static_cast<int64_t>(q);
}

int64_t batch_size(int64_t S, int64_t m_mem, int64_t m_comp, double p) {
  const int64_t by_mem = m_mem / S;
  const int64_t by_comp = compute_bound(S, m_comp, p);
  return std::max<int64_t>(1, std::min(by_mem, by_comp));
}

// Least squares of t ~ a + b*x for x = B*S^p at a fixed p.  x is scaled by its
// maximum for conditioning; sums are centred and accumulated in long double.
// Returns the residual sum of squares, or +inf when all x are equal.
double fit_linear(const double* B, const double* S, const double* t, int64_t n, double p,
                  double* a, double* b) {
  std::vector<long double> u(static_cast<size_t>(n));
  long double umax = 0.0L;
  for (int64_t i = 0; i < n; ++i) {
    u[i] = static_cast<long double>(B[i]) * std::pow(static_cast<long double>(S[i]), static_cast<long double>(p));
    umax = std::max(umax, u[i]);
  }
  if (!(umax > 0.0L) || !std::isfinite(static_cast<double>(umax))) return std::numeric_limits<double>::infinity();
  long double um = 0.0L, tm = 0.0L;
  for (int64_t i = 0; i < n; ++i) { u[i] /= umax; um += u[i]; tm += t[i]; }
  um /= n;
  tm /= n;
  long double sxx = 0.0L, sxt = 0.0L;
  for (int64_t i = 0; i < n; ++i) {
    const long double du = u[i] - um;
    sxx += du * du;
    sxt += du * (static_cast<long double>(t[i]) - tm);
  }
  if (!(sxx > 0.0L)) return std::numeric_limits<double>::infinity();
  const long double bu = sxt / sxx;
  const long double aa = tm - bu * um;
  long double rss = 0.0L;
  for (int64_t i = 0; i < n; ++i) {
    const long double r = aa + bu * u[i] - static_cast<long double>(t[i]);
    rss += r * r;
  }
  *a = static_cast<double>(aa);
  *b = static_cast<double>(bu / umax);
  return static_cast<double>(rss);
}

}  // namespace

ADALN_EXPORT int64_t adaln_sched_batch_size(int64_t S, int64_t m_mem, int64_t m_comp, double p) {
  if (S < 1 || !budgets_ok(m_mem, m_comp, p)) return -1;
  return batch_size(S, m_mem, m_comp, p);
}

ADALN_EXPORT adaln_status_t adaln_sched_plan(const int64_t* lengths, int64_t n, int64_t m_mem,
                                             int64_t m_comp, double p, int64_t* group_of,
                                             int64_t* n_groups) {
  if (n < 0 || !n_groups || !budgets_ok(m_mem, m_comp, p)) return ADALN_ERR_INVALID_ARG;
  if (n > 0 && (!lengths || !group_of)) return ADALN_ERR_INVALID_ARG;
  for (int64_t i = 0; i < n; ++i)
    if (lengths[i] < 1) return ADALN_ERR_INVALID_ARG;
  // samples by ascending length, input order among equal lengths
  std::vector<int64_t> order(static_cast<size_t>(n));
  std::iota(order.begin(), order.end(), int64_t{0});
  std::stable_sort(order.begin(), order.end(),
                   [lengths](int64_t x, int64_t y) { return lengths[x] < lengths[y]; });
  int64_t g = 0;
  for (int64_t i = 0; i < n;) {
    const int64_t S = lengths[order[i]];
    const int64_t size = batch_size(S, m_mem, m_comp, p);
    int64_t in_group = 0;
    for (; i < n && lengths[order[i]] == S; ++i) {
      if (in_group == size) { ++g; in_group = 0; }
      group_of[order[i]] = g;
      ++in_group;
    }
    ++g;                                  // the next length starts a new group
  }
  *n_groups = g;
  return ADALN_OK;
}

ADALN_EXPORT adaln_status_t adaln_cost_fit(const double* B, const double* S, const double* t,
                                           int64_t n, double p_lo, double p_hi, double* a,
                                           double* b, double* p, double* rss) {
  if (n < 3 || !B || !S || !t || !a || !b || !p || !rss) return ADALN_ERR_INVALID_ARG;
  if (!(std::isfinite(p_lo) && std::isfinite(p_hi) && p_lo > 0.0 && p_lo < p_hi && p_hi <= 16.0))
    return ADALN_ERR_INVALID_ARG;
  for (int64_t i = 0; i < n; ++i)
    if (!(std::isfinite(B[i]) && B[i] > 0.0 && std::isfinite(S[i]) && S[i] > 0.0 && std::isfinite(t[i])))
      return ADALN_ERR_INVALID_ARG;

  constexpr int kGrid = 256;
  double best_p = 0.0, best_r = std::numeric_limits<double>::infinity();
  int best_k = -1;
  double ta = 0.0, tb = 0.0;
  for (int k = 0; k < kGrid; ++k) {
    const double pk = p_lo + (p_hi - p_lo) * k / (kGrid - 1);
    const double r = fit_linear(B, S, t, n, pk, &ta, &tb);
    if (r < best_r) { best_r = r; best_p = pk; best_k = k; }
  }
  if (best_k < 0) return ADALN_ERR_INVALID_ARG;   // no p gives distinct B*S^p
  // golden-section search on the bracket around the best grid point
  const double step = (p_hi - p_lo) / (kGrid - 1);
  double lo = std::max(p_lo, best_p - step), hi = std::min(p_hi, best_p + step);
  const double invphi = (std::sqrt(5.0) - 1.0) / 2.0;
  double c = hi - invphi * (hi - lo), d = lo + invphi * (hi - lo);
  double fc = fit_linear(B, S, t, n, c, &ta, &tb), fd = fit_linear(B, S, t, n, d, &ta, &tb);
  for (int it = 0; it < 200 && (hi - lo) > 1e-14 * std::max(1.0, std::fabs(best_p)); ++it) {
    if (fc <= fd) { hi = d; d = c; fd = fc; c = hi - invphi * (hi - lo); fc = fit_linear(B, S, t, n, c, &ta, &tb); }
    else          { lo = c; c = d; fc = fd; d = lo + invphi * (hi - lo); fd = fit_linear(B, S, t, n, d, &ta, &tb); }
  }
  for (double cand : {c, d, 0.5 * (lo + hi)}) {
    const double r = fit_linear(B, S, t, n, cand, &ta, &tb);
    if (r < best_r) { best_r = r; best_p = cand; }
  }
  double fa = 0.0, fb = 0.0;
  const double r = fit_linear(B, S, t, n, best_p, &fa, &fb);
  *a = fa;
  *b = fb;
  *p = best_p;
  *rss = r;
  return ADALN_OK;
}

ADALN_EXPORT double adaln_load_cv(const double* load, int64_t n) {
  const double nan = std::numeric_limits<double>::quiet_NaN();
  if (!load || n < 1) return nan;
  long double mean = 0.0L;
  for (int64_t i = 0; i < n; ++i) mean += load[i];
  mean /= n;
  if (mean == 0.0L) return nan;
  long double var = 0.0L;
  for (int64_t i = 0; i < n; ++i) {
    const long double d = static_cast<long double>(load[i]) - mean;
    var += d * d;
  }
  var /= n;
  return static_cast<double>(std::sqrt(var) / mean);
}
