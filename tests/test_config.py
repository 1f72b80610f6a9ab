"""Host-side configuration: the oracle (oracle/config.py) against what the
pages print, and the library's host functions against the oracle.  CPU only:
the library's configuration entry points make no HIP call.

Pins ("Skip-Softmax" design document of vLLM-Omni):
  * section "Timestep gating", "Mapping the cutoff to denoising steps": the
    MiniMax-H3 schedule's first timesteps and its dense-step table
    (tests/golden/flow_shift_minimax_h3.json);
  * section "Skip-Softmax calibration config": the Wan 2.2 coefficients
    (tests/golden/wan22_calibration.json) and the ignore example
    (blocks.0.attn1 matches transformer.blocks.0.attn1 and
    transformer_2.blocks.0.attn1);
  * section "From configuration to the kernel threshold": threshold = lambda
    for any length, threshold 0 skips nothing, one accepted formula, two
    exclusive controls, target_sparsity without calibration fails;
  * section "Timestep gating": 0 is a sentinel (t never read), a cutoff of
    1.0 gives no dense steps, an unpublished t keeps the call dense.
"""
import itertools
import json
import math
import os
import random

import pytest

from oracle import config as ocfg
from tests import config_pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- oracle pins
@pytest.mark.parametrize("pin", config_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ocfg)


# ---------------------------------------------------------------- library vs oracle
@pytest.fixture(scope="module")
def cfgmod():
    from skip_softmax_flashattention_amd import config as m
    return m


def test_library_schedule_and_dense_steps(cfgmod):
    g = _golden("flow_shift_minimax_h3.json")
    for shift, n in ((12.0, 50), (5.0, 30), (1.0, 10), (3.5, 2)):
        lib_ts = cfgmod.flow_shift_schedule(shift, n)
        ref = ocfg.flow_shift_schedule(shift, n)
        assert lib_ts == pytest.approx(ref, rel=0, abs=1e-15)
    ts = cfgmod.flow_shift_schedule(g["shift"], g["num_inference_steps"])
    for cut, (dense, _) in g["table"].items():
        assert cfgmod.dense_steps(ts, float(cut)) == dense
    rng = random.Random(5)
    for _ in range(200):
        seq = [rng.random() for _ in range(rng.randint(0, 20))]
        cut = rng.choice([0.0, 1.0, rng.random()])
        assert cfgmod.dense_steps(seq, cut) == ocfg.dense_steps(seq, cut)


def test_library_layer_factor_matches_oracle(cfgmod):
    import ctypes
    lib = cfgmod._lib()
    rng = random.Random(9)
    for _ in range(2000):
        use_thr = rng.random() < 0.5
        thr = rng.choice([0.0, 1e-4, 0.01, 0.7, 3.0]) if use_thr else None
        tgt = None if use_thr else rng.choice([0.0, 0.5, 0.7, 0.9])
        coef = rng.choice([None, (2822.6209952221557, 4.388250623520793), (2.05, 13.28)])
        ign = rng.random() < 0.2
        n = rng.choice([1, 1024, 32760])
        t = rng.choice([None, 1.0, 0.95, 0.93, 0.5])
        cut = rng.choice([0.0, 0.93, 1.0])
        out = ctypes.c_double()
        a, b = coef if coef else (0.0, 0.0)
        rc = lib.ssa_layer_factor(thr is not None, thr or 0.0, tgt is not None, tgt or 0.0, ign, coef is not None,
                                  a, b, n, t is not None, t or 0.0, cut, ctypes.byref(out))
        assert rc == 0
        ref = ocfg.effective_factor(thr, tgt, coef, n, t, cut, ignored=ign)
        assert out.value == pytest.approx(ref, rel=1e-15, abs=0), (thr, tgt, coef, ign, n, t, cut)


def test_library_ignore_matches_oracle(cfgmod):
    import ctypes
    lib = cfgmod._lib()
    pats_sets = [["blocks.0.attn1", "blocks.0.attn2", "blocks.1.attn1"], ["blocks.*.attn2"], ["*attn1"],
                 ["transformer_2.blocks.[0-3].attn?"], []]
    names = ["transformer.blocks.0.attn1", "transformer_2.blocks.0.attn1", "transformer.blocks.1.attn2",
             "transformer.blocks.12.attn2", "transformer_2.blocks.2.attn1", "transformer_2.blocks.7.attn2",
             "blocks.0.attn1"]
    for pats, name in itertools.product(pats_sets, names):
        comp = name.split(".")[0] if name.startswith("transformer") else ""
        arr = (ctypes.c_char_p * max(1, len(pats)))(*[p.encode() for p in pats])
        m = ctypes.c_int()
        assert lib.ssa_ignore_match(name.encode(), comp.encode(), arr, len(pats), ctypes.byref(m)) == 0
        assert bool(m.value) == ocfg.is_ignored(name, comp, pats), (pats, name)


def test_library_checks(cfgmod):
    lib = cfgmod._lib()
    assert lib.ssa_check_formula(b"a * exp(b * target_sparsity)") == 0
    assert lib.ssa_check_formula(b"a*exp(b*target_sparsity)") == -7
    assert lib.ssa_check_spec(1, 0.1, 1, 0.5, 1) == -1
    assert lib.ssa_check_spec(0, 0.0, 0, 0.0, 1) == -1
    assert lib.ssa_check_spec(1, -0.1, 0, 0.0, 0) == -3
    assert lib.ssa_check_spec(0, 0.0, 1, 0.7, 0) == -4   # needs a calibration: use threshold instead
    assert lib.ssa_check_spec(1, 0.01, 0, 0.0, 0) == 0


def test_checkpoint_config_end_to_end(cfgmod):
    wan = _golden("wan22_calibration.json")
    wan["sparse_attention_config"]["config_groups"]["group_0"]["ignore"] = ["blocks.0.attn1", "blocks.0.attn2"]
    with pytest.warns(UserWarning):
        cfg = cfgmod.SkipSoftmaxConfig.from_checkpoint({"transformer": wan, "transformer_2": None},
                                                       target_sparsity=0.7, disabled_until_timestep=0.93)
    c = wan["sparse_attention_config"]["config_groups"]["group_0"]["threshold_scale_factor"]["coefficients"]
    want = c["a"] * math.exp(c["b"] * 0.7)
    assert cfg.factor("transformer.blocks.5.attn1", 32760, t=0.9) == pytest.approx(want, rel=1e-15)
    assert cfg.factor("transformer.blocks.5.attn1", 32760, t=0.95) == 0.0      # above the cutoff
    assert cfg.factor("transformer.blocks.0.attn1", 32760, t=0.5) == 0.0       # ignored layer
    assert cfg.factor("transformer_2.blocks.5.attn1", 32760, t=0.5) == 0.0     # unreadable component
    with pytest.warns(UserWarning):
        assert cfg.factor("transformer.blocks.5.attn1", 32760) == 0.0          # no t published
    bad = json.loads(json.dumps(wan))
    bad["sparse_attention_config"]["config_groups"]["group_0"]["threshold_scale_factor"]["formula"] = "a * b"
    with pytest.raises(Exception):
        cfgmod.SkipSoftmaxConfig.from_checkpoint({"transformer": bad}, target_sparsity=0.7)
    with pytest.raises(Exception):
        cfgmod.SkipSoftmaxConfig.from_checkpoint({"transformer": None}, target_sparsity=0.7)
    thr = cfgmod.SkipSoftmaxConfig.from_checkpoint({"transformer": {}}, threshold=0.01)
    assert thr.factor("transformer.blocks.5.attn1", 4096) == pytest.approx(0.01 * 4096, rel=1e-15)
