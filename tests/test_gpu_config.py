"""The host configuration carried through the kernel ("Skip-Softmax" design
document of vLLM-Omni, sections "From configuration to the kernel threshold",
"Skip-Softmax calibration config" and "Timestep gating"): a checkpoint's
calibration config and the user control resolve one factor per layer and
denoising step, the timestep gate is applied to it before the kernel, and the
kernel runs on that factor.

Each case resolves the factor with the library (SkipSoftmaxConfig, over the
Wan 2.2 calibration config the design document prints, with an ignore list)
and with the configuration oracle (oracle/config.py, effective_factor), then
runs ssa.fwd on a grid-locality workload with the library's factor and
compares the result with the attention oracle at the oracle's factor:
  * a step above the cutoff, an ignored layer and an unpublished timestep run
    dense: no tile skipped, the output that of lambda = 0;
  * a step at or below the cutoff skips with factor a * exp(b * s): tile
    mask, O and LSE against the oracle (tests/parity.py's bar).
The timesteps are those of the MiniMax-H3 flow-shift schedule the same
section tabulates (shift 12, 50 points): its last dense step and its first
step with skipping under the cutoff 0.93.
"""
import json
import math
import os
import warnings

import numpy as np
import pytest
import torch

from oracle import config as ocfg
from skip_softmax_flashattention_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CUTOFF = 0.93
TARGET = 0.7
IGNORE = ["blocks.0.attn1", "blocks.0.attn2"]


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    return m


@pytest.fixture(scope="module")
def setup():
    from skip_softmax_flashattention_amd import config as cfgmod
    with open(os.path.join(GOLDEN, "wan22_calibration.json")) as f:
        wan = json.load(f)
    group = wan["sparse_attention_config"]["config_groups"]["group_0"]
    group["ignore"] = list(IGNORE)
    coef = group["threshold_scale_factor"]["coefficients"]
    cfg = cfgmod.SkipSoftmaxConfig.from_checkpoint({"transformer": wan}, target_sparsity=TARGET,
                                                   disabled_until_timestep=CUTOFF)
    ts = cfgmod.flow_shift_schedule(12.0, 50)
    n_dense = cfgmod.dense_steps(ts, CUTOFF)
    assert n_dense == sum(1 for t in ocfg.flow_shift_schedule(12.0, 50) if t > CUTOFF)
    assert ts[n_dense - 1] > CUTOFF >= ts[n_dense]
    return cfg, (coef["a"], coef["b"]), ts, n_dense


def _cases(ts, n_dense):
    return [
        ("transformer.blocks.5.attn1", ts[n_dense - 1], "last dense step, above the cutoff"),
        ("transformer.blocks.5.attn1", ts[n_dense], "first step under the cutoff"),
        ("transformer.blocks.5.attn1", 0.2, "late step"),
        ("transformer.blocks.0.attn1", ts[n_dense], "ignored layer under the cutoff"),
        ("transformer.blocks.5.attn1", None, "no timestep published"),
    ]


@pytest.mark.parametrize("case", range(5))
def test_config_factor_through_kernel(ssa, setup, case):
    cfg, (a, b), ts, n_dense = setup
    layer, t, what = _cases(ts, n_dense)[case]
    w = inputs.grid_small(31, (4, 12, 20), heads=2)
    S = w.q.shape[2]
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")          # an unpublished t warns once
        factor = cfg.factor(layer, seqlen=S, t=t)
    want = ocfg.effective_factor(None, TARGET, (a, b), S, t, CUTOFF,
                                 ignored=ocfg.is_ignored(layer, "transformer", IGNORE))
    print(f"[case] config -> kernel: {what}: layer {layer} t={t} factor {factor!r} (oracle {want!r})", flush=True)
    assert factor == pytest.approx(want, rel=1e-15, abs=0.0)
    dense_expected = t is None or t > CUTOFF or "ignored" in what
    if dense_expected:
        assert factor == 0.0
    else:
        assert factor == pytest.approx(a * math.exp(b * TARGET), rel=1e-15)
    q, k, v = (x.cuda() for x in (w.q, w.k, w.v))
    o, lse, cnt = ssa.fwd(q, k, v, scale=w.scale, factor=factor)
    torch.cuda.synchronize()
    if dense_expected:
        od, lsed, _ = ssa.fwd(q, k, v, scale=w.scale, factor=0.0)
        torch.cuda.synchronize()
        assert int(cnt.sum()) == 0
        assert torch.equal(o, od) and torch.equal(lse, lsed)
    rep = parity.check_fixed(ssa, w, factor=want)
    print(f"[case] config -> kernel: {what}: {rep}", flush=True)
    parity.assert_bar(rep)
    if not dense_expected:
        assert rep.skipped > 0
        assert int(cnt.sum()) == rep.skipped
