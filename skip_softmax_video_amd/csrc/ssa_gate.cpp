// Host-side timestep and layer gating of skip-softmax attention (C ABI).
//
// TensorRT-LLM docs "VisualGen Sparse Attention (Beta)", sections "Checkpoint
// Config", "User Configuration" and "Mapping disabled_until_timestep to
// Actual Denoising Steps": skip-softmax is off while the normalized timestep
// is at or above disabled_until_timestep, and ignore patterns disable
// matching layers. TensorRT-LLM pull request "Add SkipSoftmax sparse
// attention support for visual generation", section "Use Cases", case 1d:
// per-layer fnmatch overrides of threshold_scale_factor, where 0 means dense.
#include <fnmatch.h>
#include <math.h>
#include <string.h>

#include "ssa.h"

namespace {

bool finite_nonneg(double x) { return x == x && x >= 0.0 && !isinf(x); }

// fnmatch against the full module name or its component-relative name
// (everything after the first '.').
bool layer_matches(const char* layer, const char* pattern) {
  if (pattern == nullptr) return false;
  if (fnmatch(pattern, layer, FNM_NOESCAPE) == 0) return true;
  const char* dot = strchr(layer, '.');
  return dot != nullptr && fnmatch(pattern, dot + 1, FNM_NOESCAPE) == 0;
}

}  // namespace

extern "C" int ssa_gate_layer(const ssa_gate_spec* g, const char* layer, const double* timesteps,
                              int32_t n_timesteps, double base_scale_factor, double* scale_factor,
                              int32_t* rule) {
  if (g == nullptr || layer == nullptr || timesteps == nullptr || scale_factor == nullptr ||
      rule == nullptr || n_timesteps < 1)
    return SSA_ERR_INVALID_ARG;
  const double cut = g->disabled_until_timestep;
  if (cut == cut && !(cut >= 0.0 && cut <= 1.0)) return SSA_ERR_INVALID_ARG;
  if (!finite_nonneg(base_scale_factor)) return SSA_ERR_INVALID_ARG;
  if ((g->n_ignore > 0 && g->ignore == nullptr) || (g->n_overrides > 0 && g->overrides == nullptr) ||
      g->n_ignore < 0 || g->n_overrides < 0)
    return SSA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < g->n_overrides; ++i)
    if (g->overrides[i].pattern == nullptr || !finite_nonneg(g->overrides[i].scale_factor))
      return SSA_ERR_INVALID_ARG;
  double t = timesteps[0];
  for (int32_t i = 0; i < n_timesteps; ++i) {
    if (timesteps[i] != timesteps[i]) return SSA_ERR_INVALID_ARG;
    t = timesteps[i] > t ? timesteps[i] : t;
  }
  if (cut == cut && t >= cut) {
    *scale_factor = 0.0;
    *rule = SSA_GATE_TIMESTEP;
    return SSA_OK;
  }
  for (int32_t i = 0; i < g->n_ignore; ++i)
    if (layer_matches(layer, g->ignore[i])) {
      *scale_factor = 0.0;
      *rule = SSA_GATE_IGNORED;
      return SSA_OK;
    }
  for (int32_t i = 0; i < g->n_overrides; ++i)
    if (layer_matches(layer, g->overrides[i].pattern)) {
      *scale_factor = g->overrides[i].scale_factor;
      *rule = SSA_GATE_OVERRIDE;
      return SSA_OK;
    }
  *scale_factor = base_scale_factor;
  *rule = SSA_GATE_BASE;
  return SSA_OK;
}

extern "C" int ssa_flow_timesteps(int32_t n_steps, int32_t num_train_timesteps, double flow_shift, double* t) {
  if (t == nullptr || n_steps < 1 || num_train_timesteps < 1 || !(flow_shift > 0.0) || isinf(flow_shift))
    return SSA_ERR_INVALID_ARG;
  const double keep = 1.0 - 1.0 / (double)num_train_timesteps;
  for (int32_t i = 0; i < n_steps; ++i) {
    const double s = 1.0 - (double)i * keep / (double)n_steps;
    const double shifted = flow_shift * s / (1.0 + (flow_shift - 1.0) * s);
    t[i] = keep * shifted;
  }
  return SSA_OK;
}

extern "C" int ssa_gate_dense_steps(const double* t, int32_t n, double cutoff, int32_t* dense_steps) {
  if (dense_steps == nullptr || n < 0 || (n > 0 && t == nullptr)) return SSA_ERR_INVALID_ARG;
  if (cutoff == cutoff && !(cutoff >= 0.0 && cutoff <= 1.0)) return SSA_ERR_INVALID_ARG;
  int32_t c = 0;
  if (cutoff == cutoff)
    for (int32_t i = 0; i < n; ++i) c += t[i] >= cutoff ? 1 : 0;
  *dense_steps = c;
  return SSA_OK;
}
