// Driver for the sanitizer build of the host configuration functions
// (csrc/ssa_config.cpp; tests only): every entry point, its argument
// errors included, on the pages' worked values (the Wan 2.2 coefficients,
// the MiniMax-H3 flow-shift schedule and its dense-step table).  Exit status
// 0 = all checks passed; the sanitizers abort on the first error.
#include <cmath>
#include <cstdio>
#include <vector>

#include "ssa.h"

static int failures = 0;
static void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s\n", what);
    ++failures;
  }
}

int main() {
  check(ssa_check_formula("a * exp(b * target_sparsity)") == SSA_OK, "formula accepted");
  check(ssa_check_formula("a * b") == SSA_ERR_BAD_CONFIG, "formula rejected");
  check(ssa_check_formula(nullptr) == SSA_ERR_INVALID_ARG, "null formula");
  check(ssa_check_spec(1, 0.01, 0, 0.0, 0) == SSA_OK, "threshold control");
  check(ssa_check_spec(1, 0.01, 1, 0.7, 1) == SSA_ERR_INVALID_ARG, "both controls");
  check(ssa_check_spec(0, 0.0, 1, 0.7, 0) == SSA_ERR_NO_CALIBRATION, "target without calibration");
  check(ssa_check_spec(1, NAN, 0, 0.0, 0) == SSA_ERR_BAD_THRESHOLD, "NaN threshold");
  const char* pats[] = {"blocks.0.attn1", "*.attn2"};
  int m = -1;
  check(ssa_ignore_match("transformer.blocks.0.attn1", "transformer", pats, 2, &m) == SSA_OK && m == 1, "relative match");
  check(ssa_ignore_match("transformer.blocks.5.attn1", "transformer", pats, 2, &m) == SSA_OK && m == 0, "no match");
  check(ssa_ignore_match("x.attn2", nullptr, pats, 2, &m) == SSA_OK && m == 1, "full match, no component");
  check(ssa_ignore_match("transformer", "transformer", pats, 2, &m) == SSA_OK, "name equal to component");
  check(ssa_ignore_match("t", "", pats, 0, &m) == SSA_OK && m == 0, "no patterns");
  check(ssa_ignore_match(nullptr, "t", pats, 2, &m) == SSA_ERR_INVALID_ARG, "null name");
  const char* bad[] = {nullptr};
  check(ssa_ignore_match("t.x", "t", bad, 1, &m) == SSA_ERR_INVALID_ARG, "null pattern");
  double f = -1.0;
  const double a = 2822.6209952221557, b = 4.388250623520793;
  check(ssa_layer_factor(0, 0, 1, 0.7, 0, 1, a, b, 32760, 1, 0.9, 0.93, &f) == SSA_OK &&
            std::fabs(f - a * std::exp(b * 0.7)) <= 1e-9 * f, "calibrated factor");
  check(ssa_layer_factor(0, 0, 1, 0.7, 0, 1, a, b, 32760, 1, 0.95, 0.93, &f) == SSA_OK && f == 0.0, "gate closed");
  check(ssa_layer_factor(0, 0, 1, 0.7, 1, 1, a, b, 32760, 1, 0.5, 0.93, &f) == SSA_OK && f == 0.0, "ignored layer");
  check(ssa_layer_factor(0, 0, 1, 0.7, 0, 1, a, b, 32760, 0, 0.0, 0.93, &f) == SSA_OK && f == 0.0, "no t");
  check(ssa_layer_factor(1, 0.01, 0, 0, 0, 0, 0, 0, 4096, 0, 0.0, 0.0, &f) == SSA_OK && f == 0.01 * 4096, "threshold");
  check(ssa_layer_factor(1, 0.01, 0, 0, 0, 0, 0, 0, 0, 0, 0.0, 0.0, &f) == SSA_ERR_BAD_THRESHOLD, "seqlen 0");
  check(ssa_layer_factor(0, 0, 1, 0.7, 0, 1, -1.0, b, 10, 0, 0.0, 0.0, &f) == SSA_ERR_NO_CALIBRATION, "a <= 0");
  check(ssa_layer_factor(0, 0, 1, 0.7, 0, 1, a, b, 10, 0, 0.0, 0.0, nullptr) == SSA_ERR_INVALID_ARG, "null out");
  std::vector<double> ts(49);
  check(ssa_flow_shift_schedule(12.0, 50, ts.data()) == SSA_OK, "schedule");
  check(std::fabs(ts[0] - 1.0) < 1e-12 && std::fabs(ts[1] - 0.998) < 5e-4, "schedule values");
  const double cut[] = {1.0, 0.99, 0.97, 0.95, 0.90, 0.86};
  const int want[] = {0, 6, 14, 19, 28, 33};
  for (int i = 0; i < 6; ++i) {
    int c = -1;
    check(ssa_dense_steps(ts.data(), 49, cut[i], &c) == SSA_OK && c == want[i], "dense-step table");
  }
  int c = -1;
  check(ssa_dense_steps(ts.data(), 49, 0.0, &c) == SSA_OK && c == 0, "cutoff 0");
  check(ssa_dense_steps(nullptr, 3, 0.5, &c) == SSA_ERR_INVALID_ARG, "null schedule");
  check(ssa_flow_shift_schedule(12.0, 1, ts.data()) == SSA_ERR_INVALID_ARG, "too few steps");
  std::printf("config driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
