// Host-side configuration of Skip-Softmax: the factor a layer hands to the
// kernel on a given denoising step.  No GPU work happens here.
//
// The rules: "Skip-Softmax" design document of vLLM-Omni, sections "From
// configuration to the kernel threshold" (two mutually exclusive controls,
// the one accepted calibration formula, ignore patterns matched against the
// full and the component-relative module name, layers without coefficients
// run dense) and "Timestep gating" (the cutoff, the 0 sentinel, dense while
// t is above the cutoff or unpublished, the dense-step count, the
// flow-shifted rectified-flow schedule).  The C ABI is declared in
// include/ssa.h.

#include <fnmatch.h>

#include <cmath>
#include <cstring>

#include "ssa.h"

namespace {

constexpr const char* kFormula = "a * exp(b * target_sparsity)";

bool glob(const char* pattern, const char* name) { return fnmatch(pattern, name, 0) == 0; }

}  // namespace

extern "C" {

int ssa_check_formula(const char* formula) {
  if (formula == nullptr) return SSA_ERR_INVALID_ARG;
  return std::strcmp(formula, kFormula) == 0 ? SSA_OK : SSA_ERR_BAD_CONFIG;
}

int ssa_check_spec(int has_threshold, double threshold, int has_target, double target_sparsity,
                   int has_calibration) {
  if ((has_threshold != 0) == (has_target != 0)) return SSA_ERR_INVALID_ARG;
  if (has_threshold) return std::isfinite(threshold) && threshold >= 0.0 ? SSA_OK : SSA_ERR_BAD_THRESHOLD;
  if (!std::isfinite(target_sparsity)) return SSA_ERR_BAD_THRESHOLD;
  return has_calibration ? SSA_OK : SSA_ERR_NO_CALIBRATION;
}

int ssa_ignore_match(const char* module_name, const char* component, const char* const* patterns, int npatterns,
                     int* matched) {
  if (module_name == nullptr || matched == nullptr || npatterns < 0 || (npatterns > 0 && patterns == nullptr))
    return SSA_ERR_INVALID_ARG;
  // The name relative to the component: what follows "<component>.".
  const char* rel = module_name;
  if (component != nullptr && component[0] != '\0') {
    const size_t n = std::strlen(component);
    if (std::strncmp(module_name, component, n) == 0 && module_name[n] == '.') rel = module_name + n + 1;
  }
  *matched = 0;
  for (int i = 0; i < npatterns; ++i) {
    if (patterns[i] == nullptr) return SSA_ERR_INVALID_ARG;
    if (glob(patterns[i], module_name) || glob(patterns[i], rel)) {
      *matched = 1;
      break;
    }
  }
  return SSA_OK;
}

int ssa_layer_factor(int has_threshold, double threshold, int has_target, double target_sparsity,
                     int ignored, int has_coefficients, double a, double b, int seqlen, int has_t, double t,
                     double disabled_until_timestep, double* factor_out) {
  if (factor_out == nullptr) return SSA_ERR_INVALID_ARG;
  if ((has_threshold != 0) == (has_target != 0)) return SSA_ERR_INVALID_ARG;
  if (seqlen <= 0) return SSA_ERR_BAD_THRESHOLD;
  if (!std::isfinite(disabled_until_timestep) || disabled_until_timestep < 0.0) return SSA_ERR_BAD_THRESHOLD;
  double factor = 0.0;
  if (has_threshold) {
    if (!std::isfinite(threshold) || threshold < 0.0) return SSA_ERR_BAD_THRESHOLD;
    factor = threshold * (double)seqlen;
  } else {
    if (!std::isfinite(target_sparsity)) return SSA_ERR_BAD_THRESHOLD;
    if (has_coefficients) {
      if (!std::isfinite(a) || !std::isfinite(b) || !(a > 0.0)) return SSA_ERR_NO_CALIBRATION;
      factor = a * std::exp(b * target_sparsity);
    }   // a layer without coefficients runs dense
  }
  // A layer matched by an ignore pattern stays dense whatever the control.
  if (ignored) factor = 0.0;
  // Timestep gate: 0 disables it (t is not read); otherwise dense while t is
  // above the cutoff or not published.
  if (disabled_until_timestep > 0.0 && (!has_t || !(t <= disabled_until_timestep))) factor = 0.0;
  *factor_out = factor;
  return SSA_OK;
}

int ssa_dense_steps(const double* t, int n, double disabled_until_timestep, int* count) {
  if (count == nullptr || n < 0 || (n > 0 && t == nullptr)) return SSA_ERR_INVALID_ARG;
  int c = 0;
  if (disabled_until_timestep > 0.0)
    for (int i = 0; i < n; ++i) c += t[i] > disabled_until_timestep ? 1 : 0;
  *count = c;
  return SSA_OK;
}

int ssa_flow_shift_schedule(double shift, int num_inference_steps, double* t_out) {
  if (t_out == nullptr || num_inference_steps < 2 || !std::isfinite(shift) || !(shift > 0.0))
    return SSA_ERR_INVALID_ARG;
  const int n = num_inference_steps;
  for (int i = 0; i + 1 < n; ++i) {
    const double u = 1.0 - (double)i / (double)(n - 1);
    t_out[i] = shift * u / (1.0 + (shift - 1.0) * u);
  }
  return SSA_OK;
}

}  // extern "C"
