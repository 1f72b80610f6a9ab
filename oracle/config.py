"""CPU oracle for the host-side configuration of Skip-Softmax: which factor a
layer passes to the kernel on a given denoising step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests use it.  It shares no code with the
library's host functions.

Source: "Skip-Softmax" design document of vLLM-Omni, sections "From
configuration to the kernel threshold" (the two controls, the calibration
config and how it is consumed) and "Timestep gating" (the gate, where t comes
from, and the mapping of the cutoff to denoising steps).  Pinned by tests in
tests/test_config.py against the page's own worked table, its printed
coefficients and its ignore-matching example.
"""
from __future__ import annotations

import fnmatch
import math
from typing import Iterable, List, Optional, Sequence

# The one calibration curve the page accepts.
FORMULA = "a * exp(b * target_sparsity)"


class ConfigError(ValueError):
    """A configuration the page says must be rejected."""


def check_spec(threshold: Optional[float], target_sparsity: Optional[float]) -> None:
    """The two user controls are mutually exclusive; a threshold is a finite
    non-negative number."""
    if (threshold is None) == (target_sparsity is None):
        raise ConfigError("exactly one of threshold and target_sparsity must be given")
    if threshold is not None and not (math.isfinite(threshold) and threshold >= 0.0):
        raise ConfigError("threshold must be finite and non-negative")
    if target_sparsity is not None and not math.isfinite(target_sparsity):
        raise ConfigError("target_sparsity must be finite")


def check_formula(formula: str) -> None:
    """Only the exponential calibration curve is accepted at startup."""
    if formula != FORMULA:
        raise ConfigError(f"unsupported calibration formula {formula!r}")


def is_ignored(module_name: str, component: str, patterns: Iterable[str]) -> bool:
    """An ignore pattern is an fnmatch pattern tried against the full module
    name and against the name relative to its component (the part after
    "<component>.")."""
    rel = module_name[len(component) + 1:] if module_name.startswith(component + ".") else module_name
    return any(fnmatch.fnmatchcase(module_name, pat) or fnmatch.fnmatchcase(rel, pat) for pat in patterns)


def layer_factor(threshold: Optional[float], target_sparsity: Optional[float],
                 coefficients: Optional[Sequence[float]], seqlen: int, ignored: bool = False) -> Optional[float]:
    """The factor a layer hands to the kernel before the timestep gate, or
    None when the layer runs dense.

    threshold: factor = threshold * seqlen (so lambda = threshold).
    target_sparsity: factor = a * exp(b * s) with the layer's stamped
    coefficients (a, b); a layer without coefficients runs dense.
    A layer matched by an ignore pattern stays dense whatever the control
    (the page: such layers stay dense regardless of the user
    configuration)."""
    check_spec(threshold, target_sparsity)
    if ignored:
        return None
    if threshold is not None:
        return threshold * seqlen
    if coefficients is None:
        return None
    a, b = coefficients
    return a * math.exp(b * target_sparsity)


def gate_open(t: Optional[float], disabled_until_timestep: float) -> bool:
    """Whether skipping is active on a step with normalized timestep t.

    0 is a sentinel: the gate is off and t is never read.  A positive cutoff
    D enables the gate: skipping is active once t <= D; while t > D, or when
    the pipeline publishes no t, the call runs dense."""
    if disabled_until_timestep == 0.0:
        return True
    if t is None:
        return False
    return t <= disabled_until_timestep


def effective_factor(threshold, target_sparsity, coefficients, seqlen, t, disabled_until_timestep,
                     ignored=False):
    """layer_factor, then the gate: 0.0 means no skipping on this call."""
    f = layer_factor(threshold, target_sparsity, coefficients, seqlen, ignored)
    if f is None or not gate_open(t, disabled_until_timestep):
        return 0.0
    return f


def dense_steps(ts: Sequence[float], disabled_until_timestep: float) -> int:
    """Number of denoising steps that run dense: those with t above the
    cutoff (a cutoff of 0 gates nothing)."""
    if disabled_until_timestep == 0.0:
        return 0
    return sum(1 for t in ts if t > disabled_until_timestep)


def flow_shift_schedule(shift: float, num_inference_steps: int) -> List[float]:
    """Published t of a flow-shifted rectified-flow schedule:
    num_inference_steps uniform positions u from 1 to 0, each mapped to
    t = s u / (1 + (s - 1) u); the denoiser runs on all but the last point."""
    n = num_inference_steps
    us = [1.0 - i / (n - 1) for i in range(n)]
    ts = [shift * u / (1.0 + (shift - 1.0) * u) for u in us]
    return ts[:-1]
