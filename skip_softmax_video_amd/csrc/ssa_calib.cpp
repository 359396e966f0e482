// Calibration variants on the host (C ABI): the linear-space fit of
// scale_factor = a * exp(b * sparsity) and pooling of calibration passes.
//
// ModelOpt pull request "skip-softmax ... via dedicated Triton kernels",
// sections "Calibration" and "Config & conversion": the calibrator fits the
// exponential model either in log space (recommended for diffusion, where
// scale factors span orders of magnitude) or, by default, in linear space.
// ModelOpt README "Skip-Softmax Sparse Attention for Diffusion Models",
// section "Known Issues": the sparsity curve depends on the resolution, so
// calibration samples are pooled per key length.
#include <math.h>

#include <vector>

#include "ssa.h"

namespace {

// Scan range and step of b around the log-space slope.
constexpr double kScanHalfWidth = 100.0;
constexpr int kScanPoints = 2001;

struct Points {
  std::vector<double> x, y;  // sparsity, scale factor
  double xmax = 0.0;
};

// H(b) = (sum y u)^2 / sum u^2 and g(b) ~ dH/db (same sign), u = e^{b (x - xmax)}
void h_and_slope(const Points& P, double b, double* h, double* g) {
  double n = 0.0, d = 0.0, n1 = 0.0, d1 = 0.0;
  for (size_t i = 0; i < P.x.size(); ++i) {
    const double xc = P.x[i] - P.xmax;
    const double u = exp(b * xc);
    n += P.y[i] * u;
    d += u * u;
    n1 += P.y[i] * xc * u;
    d1 += 2.0 * xc * u * u;
  }
  if (h) *h = n * n / d;
  if (g) *g = 2.0 * n1 * d - n * d1;
}

}  // namespace

extern "C" int ssa_calibration_fit_linear(const double* lambda, const double* sparsity, const double* seq_k,
                                          int32_t n, ssa_calib_result* out) {
  ssa_calib_result logfit;
  const int st = ssa_calibration_fit(lambda, sparsity, seq_k, n, &logfit);  // validates, b0, range
  if (st != SSA_OK) return st;
  Points P;
  for (int i = 0; i < n; ++i) {
    const double s = sparsity[i], lam = lambda[i], sk = seq_k[i];
    if (!(s > 0.0 && s < 1.0) || !(lam > 0.0) || !(sk > 0.0)) continue;
    P.x.push_back(s);
    P.y.push_back(lam * sk);
  }
  P.xmax = logfit.s_max;
  // coarse scan of H around the log-space slope
  const double step = 2.0 * kScanHalfWidth / (kScanPoints - 1);
  int best = 0;
  double hbest = -1.0;
  for (int k = 0; k < kScanPoints; ++k) {
    double h;
    h_and_slope(P, logfit.b - kScanHalfWidth + k * step, &h, nullptr);
    if (h > hbest) {
      hbest = h;
      best = k;
    }
  }
  if (best == 0 || best == kScanPoints - 1 || !(hbest > 0.0)) return SSA_ERR_FIT_DEGENERATE;
  // bisect dH/db = 0 inside the two cells around the best grid point
  double lo = logfit.b - kScanHalfWidth + (best - 1) * step;
  double hi = logfit.b - kScanHalfWidth + (best + 1) * step;
  double glo, ghi;
  h_and_slope(P, lo, nullptr, &glo);
  h_and_slope(P, hi, nullptr, &ghi);
  if (!(glo > 0.0 && ghi < 0.0)) return SSA_ERR_FIT_DEGENERATE;
  for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    double g;
    h_and_slope(P, mid, nullptr, &g);
    if (g > 0.0)
      lo = mid;
    else
      hi = mid;
  }
  const double b = 0.5 * (lo + hi);
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < P.x.size(); ++i) {
    const double u = exp(b * (P.x[i] - P.xmax));
    num += P.y[i] * u;
    den += u * u;
  }
  out->b = b;
  out->log_a = log(num / den) - b * P.xmax;
  out->a = exp(out->log_a);
  out->s_min = logfit.s_min;
  out->s_max = logfit.s_max;
  out->n_used = logfit.n_used;
  return SSA_OK;
}

extern "C" int ssa_calibration_pool_add(const ssa_problem* p, const int32_t* counts, const int32_t* tiles,
                                        int32_t n, ssa_calib_pool* pool) {
  if (p == nullptr || p->cu_seqlens == nullptr || counts == nullptr || tiles == nullptr || pool == nullptr ||
      n < 1 || p->batch < 1 || p->num_heads < 1 || p->block < 1 || pool->max_groups < 0 || pool->n_groups < 0 ||
      pool->n_groups > pool->max_groups)
    return SSA_ERR_INVALID_ARG;
  if (pool->n_lambda != 0 && pool->n_lambda != n) return SSA_ERR_INVALID_ARG;
  if (p->cu_seqlens[0] != 0) return SSA_ERR_INVALID_ARG;
  if (pool->max_groups > 0 && (pool->seq_k == nullptr || pool->skipped == nullptr || pool->visited == nullptr))
    return SSA_ERR_INVALID_ARG;
  // map every non-empty sequence to a group first, so a full pool leaves everything unchanged
  std::vector<int> group(p->batch, -1);
  int ng = pool->n_groups;
  std::vector<int64_t> new_keys;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t S = (int64_t)p->cu_seqlens[b + 1] - p->cu_seqlens[b];
    if (S < 0) return SSA_ERR_INVALID_ARG;
    if (S == 0) continue;
    int g = -1;
    for (int i = 0; i < pool->n_groups; ++i)
      if (pool->seq_k[i] == S) g = i;
    for (size_t i = 0; g < 0 && i < new_keys.size(); ++i)
      if (new_keys[i] == S) g = pool->n_groups + (int)i;
    if (g < 0) {
      if (ng >= pool->max_groups) return SSA_ERR_INVALID_ARG;
      new_keys.push_back(S);
      g = ng++;
    }
    group[b] = g;
  }
  pool->n_lambda = n;
  for (size_t i = 0; i < new_keys.size(); ++i) {
    const int g = pool->n_groups + (int)i;
    pool->seq_k[g] = new_keys[i];
    pool->visited[g] = 0;
    for (int k = 0; k < n; ++k) pool->skipped[(int64_t)g * n + k] = 0;
  }
  pool->n_groups = ng;
  int64_t w = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t S = (int64_t)p->cu_seqlens[b + 1] - p->cu_seqlens[b];
    const int64_t nwg = (S + p->block - 1) / p->block * p->num_heads;
    const int g = group[b];
    for (int64_t i = 0; i < nwg; ++i, ++w) {
      pool->visited[g] += tiles[w];
      for (int k = 0; k < n; ++k) pool->skipped[(int64_t)g * n + k] += counts[w * n + k];
    }
  }
  return SSA_OK;
}

extern "C" int ssa_calibration_pool_points(const ssa_calib_pool* pool, const double* lambdas, double* lambda_out,
                                           double* sparsity_out, double* seq_k_out, int32_t* n_points) {
  if (pool == nullptr || lambdas == nullptr || lambda_out == nullptr || sparsity_out == nullptr ||
      seq_k_out == nullptr || n_points == nullptr || pool->n_groups < 0 || pool->n_lambda < 0)
    return SSA_ERR_INVALID_ARG;
  const int n = pool->n_lambda;
  for (int g = 0; g < pool->n_groups; ++g)
    for (int k = 0; k < n; ++k) {
      const int64_t i = (int64_t)g * n + k;
      lambda_out[i] = lambdas[k];
      sparsity_out[i] = pool->visited[g] > 0 ? (double)pool->skipped[i] / (double)pool->visited[g] : NAN;
      seq_k_out[i] = (double)pool->seq_k[g];
    }
  *n_points = pool->n_groups * n;
  return SSA_OK;
}
