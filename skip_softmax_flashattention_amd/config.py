"""Host-side Skip-Softmax configuration: the factor each attention layer
hands to ``ssa_fwd`` on each denoising step.

The rules ("Skip-Softmax" design document of vLLM-Omni, sections "From
configuration to the kernel threshold" and "Timestep gating") are decided by
the library's host functions (``ssa_check_formula``, ``ssa_check_spec``,
``ssa_ignore_match``, ``ssa_layer_factor``, ``ssa_dense_steps``,
``ssa_flow_shift_schedule``); this module only reads the checkpoint's
``sparse_attention_config`` JSON and passes its fields to them.

    cfg = SkipSoftmaxConfig.from_checkpoint(
        {"transformer": json.load(open(".../transformer/config.json")),
         "transformer_2": None},            # unreadable -> that component stays dense
        target_sparsity=0.7, disabled_until_timestep=0.93)
    factor = cfg.factor("transformer.blocks.7.attn1", seqlen=S, t=0.9)
    ssa.fwd(q, k, v, factor=factor)          # factor 0.0 runs dense
"""
from __future__ import annotations

import ctypes
import dataclasses
import warnings
from typing import Dict, List, Optional, Sequence, Tuple

from . import SsaError, load_library

SSA_OK = 0


def _lib():
    lib = load_library()
    if not getattr(lib, "_ssa_config_ready", False):
        I, D, P, C = ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_char_p
        lib.ssa_check_formula.argtypes = [C]
        lib.ssa_check_spec.argtypes = [I, D, I, D, I]
        lib.ssa_ignore_match.argtypes = [C, C, ctypes.POINTER(C), I, ctypes.POINTER(I)]
        lib.ssa_layer_factor.argtypes = [I, D, I, D, I, I, D, D, I, I, D, D, ctypes.POINTER(D)]
        lib.ssa_dense_steps.argtypes = [ctypes.POINTER(D), I, D, ctypes.POINTER(I)]
        lib.ssa_flow_shift_schedule.argtypes = [D, I, ctypes.POINTER(D)]
        for name in ("ssa_check_formula", "ssa_check_spec", "ssa_ignore_match", "ssa_layer_factor",
                     "ssa_dense_steps", "ssa_flow_shift_schedule"):
            getattr(lib, name).restype = I
        lib._ssa_config_ready = True
    return lib


def _check(code: int, what: str) -> None:
    if code != SSA_OK:
        raise SsaError(code, what)


@dataclasses.dataclass
class ComponentCalibration:
    """The skip_softmax group of one transformer component's config."""

    a: float
    b: float
    ignore: List[str]


def read_component(config: Optional[dict]) -> Optional[ComponentCalibration]:
    """The skip_softmax calibration of one component's config.json (as a
    dict), or None if it has none.  A formula other than the accepted curve
    raises (the page rejects such a checkpoint at startup)."""
    if not config:
        return None
    groups = (config.get("sparse_attention_config") or {}).get("config_groups") or {}
    for group in groups.values():
        if group.get("algorithm") != "skip_softmax":
            continue
        tsf = group.get("threshold_scale_factor") or {}
        formula = tsf.get("formula", "")
        _check(_lib().ssa_check_formula(formula.encode()), f"unsupported calibration formula {formula!r}")
        coef = tsf.get("coefficients") or {}
        return ComponentCalibration(float(coef["a"]), float(coef["b"]), [str(p) for p in group.get("ignore", [])])
    return None


class SkipSoftmaxConfig:
    """User control (threshold or target_sparsity, plus the timestep cutoff)
    and the per-component calibrations of a checkpoint."""

    def __init__(self, components: Dict[str, Optional[ComponentCalibration]], *,
                 threshold: Optional[float] = None, target_sparsity: Optional[float] = None,
                 disabled_until_timestep: float = 0.0):
        self.components = dict(components)
        self.threshold = threshold
        self.target_sparsity = target_sparsity
        self.disabled_until_timestep = float(disabled_until_timestep)
        has_cal = any(c is not None for c in self.components.values())
        _check(_lib().ssa_check_spec(threshold is not None, float(threshold or 0.0),
                                     target_sparsity is not None, float(target_sparsity or 0.0), has_cal),
               "invalid skip-softmax control: give exactly one of threshold and target_sparsity; "
               "target_sparsity needs a calibrated checkpoint (else use threshold)")
        self._warned_no_t = False

    @classmethod
    def from_checkpoint(cls, component_configs: Dict[str, Optional[dict]], **control) -> "SkipSoftmaxConfig":
        """component_configs: component name -> its parsed config.json, or
        None when it could not be read (that component then stays dense, with
        a warning, as long as another component is calibrated)."""
        comps = {}
        for name, cfg in component_configs.items():
            if cfg is None:
                warnings.warn(f"skip-softmax: config of component {name!r} could not be read; it stays dense")
            comps[name] = read_component(cfg)
        return cls(comps, **control)

    def _component_of(self, module_name: str) -> Tuple[Optional[str], Optional[ComponentCalibration]]:
        for name, cal in self.components.items():
            if module_name == name or module_name.startswith(name + "."):
                return name, cal
        return None, None

    def ignored(self, module_name: str) -> bool:
        """Whether the layer matches an ignore pattern of its component."""
        comp, cal = self._component_of(module_name)
        if cal is None or not cal.ignore:
            return False
        pats = (ctypes.c_char_p * len(cal.ignore))(*[p.encode() for p in cal.ignore])
        matched = ctypes.c_int()
        _check(_lib().ssa_ignore_match(module_name.encode(), comp.encode(), pats, len(cal.ignore),
                                       ctypes.byref(matched)), "ignore matching failed")
        return bool(matched.value)

    def coefficients(self, module_name: str) -> Optional[Tuple[float, float]]:
        """(a, b) of the layer's component, or None if it has no calibration."""
        _, cal = self._component_of(module_name)
        return None if cal is None else (cal.a, cal.b)

    def factor(self, module_name: str, seqlen: int, t: Optional[float] = None) -> float:
        """The factor for ssa_fwd on this call (0.0 = dense)."""
        coef = self.coefficients(module_name)
        ign = self.ignored(module_name)
        if t is None and self.disabled_until_timestep > 0.0 and not self._warned_no_t:
            warnings.warn("skip-softmax: no timestep published; the cutoff keeps attention dense")
            self._warned_no_t = True
        out = ctypes.c_double()
        a, b = coef if coef is not None else (0.0, 0.0)
        _check(_lib().ssa_layer_factor(self.threshold is not None, float(self.threshold or 0.0),
                                       self.target_sparsity is not None, float(self.target_sparsity or 0.0),
                                       ign, coef is not None, a, b, int(seqlen), t is not None, float(t or 0.0),
                                       self.disabled_until_timestep, ctypes.byref(out)),
               "could not resolve the layer's factor")
        return out.value


def dense_steps(ts: Sequence[float], disabled_until_timestep: float) -> int:
    """Denoising steps that run dense under the cutoff."""
    arr = (ctypes.c_double * max(1, len(ts)))(*ts)
    out = ctypes.c_int()
    _check(_lib().ssa_dense_steps(arr, len(ts), float(disabled_until_timestep), ctypes.byref(out)),
           "dense_steps failed")
    return out.value


def flow_shift_schedule(shift: float, num_inference_steps: int) -> List[float]:
    """Published timesteps of a flow-shifted rectified-flow schedule."""
    n = int(num_inference_steps)
    arr = (ctypes.c_double * max(1, n - 1))()
    _check(_lib().ssa_flow_shift_schedule(float(shift), n, arr), "invalid schedule")
    return list(arr[: n - 1])
