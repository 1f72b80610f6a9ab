"""Pins for the configuration oracle (oracle/config.py): facts the pages
print, each a function taking the oracle module so that the same pins can run
against planted mistakes (tests/test_config_mutants.py).

"Skip-Softmax" design document of vLLM-Omni:
  * "Timestep gating", "Mapping the cutoff to denoising steps": the MiniMax-H3
    schedule's first timesteps and dense-step table
    (tests/golden/flow_shift_minimax_h3.json);
  * "Skip-Softmax calibration config": the Wan 2.2 coefficients
    (tests/golden/wan22_calibration.json) and the ignore example;
  * "From configuration to the kernel threshold": threshold = lambda at any
    length, threshold 0 skips nothing, one formula, exclusive controls;
  * "Timestep gating": 0 is a sentinel, cutoff 1.0 gives no dense steps, an
    unpublished t keeps the call dense.
"""
import itertools
import json
import math
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_flow_shift_table(ocfg):
    g = _golden("flow_shift_minimax_h3.json")
    ts = ocfg.flow_shift_schedule(g["shift"], g["num_inference_steps"])
    assert len(ts) == g["forwards"]
    assert [round(t, 3) for t in ts[:5]] == g["first_t_3dp"]
    assert sum(t > 0.9 for t in ts) == g["steps_above_0.9"]
    for cut, (dense, skip) in g["table"].items():
        n = ocfg.dense_steps(ts, float(cut))
        assert (n, len(ts) - n) == (dense, skip), cut
    assert all(a > b for a, b in zip(ts, ts[1:])), "t only decreases"


def pin_threshold_is_lambda_at_any_length(ocfg):
    for thr, n in itertools.product((0.0, 1e-3, 0.5, 2.0), (1, 4096, 32760)):
        f = ocfg.layer_factor(thr, None, None, n)
        assert f / n == pytest.approx(thr, rel=0, abs=1e-15)
    assert ocfg.effective_factor(0.0, None, None, 100, None, 0.0) == 0.0   # threshold 0: no skipping


def pin_calibrated_wan_coefficients(ocfg):
    cfg = _golden("wan22_calibration.json")["sparse_attention_config"]["config_groups"]["group_0"]
    c = cfg["threshold_scale_factor"]["coefficients"]
    f = ocfg.layer_factor(None, cfg["target_sparsity"], (c["a"], c["b"]), 32760)
    assert f == pytest.approx(c["a"] * math.exp(c["b"] * 0.7), rel=1e-15)
    assert f / 32760 == pytest.approx(1.8594, abs=1e-4)        # lambda above 1 at Wan's length
    assert ocfg.layer_factor(None, 0.7, None, 32760) is None   # no coefficients: dense


def pin_ignore_example(ocfg):
    pats = ["blocks.0.attn1", "blocks.0.attn2", "blocks.1.attn1"]
    assert ocfg.is_ignored("transformer.blocks.0.attn1", "transformer", pats)
    assert ocfg.is_ignored("transformer_2.blocks.0.attn1", "transformer_2", pats)
    assert not ocfg.is_ignored("transformer.blocks.1.attn2", "transformer", pats)
    assert not ocfg.is_ignored("transformer.blocks.10.attn1", "transformer", pats)
    assert ocfg.is_ignored("transformer.blocks.3.attn1", "transformer", ["blocks.*.attn1"])
    assert ocfg.layer_factor(0.01, None, None, 100, ignored=True) is None   # dense whatever the control


def pin_gate(ocfg):
    assert ocfg.gate_open(None, 0.0)          # sentinel: t not read
    assert ocfg.gate_open(0.95, 0.0)
    assert not ocfg.gate_open(None, 0.93)     # no t published: dense
    assert not ocfg.gate_open(0.95, 0.93)
    assert ocfg.gate_open(0.93, 0.93)         # at the cutoff: active
    assert ocfg.dense_steps([1.0, 0.99, 0.5], 1.0) == 0
    assert ocfg.dense_steps([1.0, 0.99, 0.5], 0.0) == 0


def _rejects(fn, *args):
    try:
        fn(*args)
    except ValueError:
        return
    raise AssertionError(f"{fn.__name__}{args} was accepted")


def pin_rejections(ocfg):
    _rejects(ocfg.check_spec, 0.1, 0.5)
    _rejects(ocfg.check_spec, None, None)
    _rejects(ocfg.check_spec, -1.0, None)
    _rejects(ocfg.check_formula, "a * b ** target_sparsity")
    ocfg.check_formula("a * exp(b * target_sparsity)")


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
