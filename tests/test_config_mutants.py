"""Plant plausible mistakes in copies of the configuration oracle
(oracle/config.py, on the CPU) and check that every one fails at least one
pin from tests/config_pins.py."""
import os
import types

import pytest

from tests import config_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "config.py")

MUTANTS = [
    ("gate opens strictly below the cutoff", "return t <= disabled_until_timestep", "return t < disabled_until_timestep"),
    ("dense steps count t at the cutoff", "return sum(1 for t in ts if t > disabled_until_timestep)",
     "return sum(1 for t in ts if t >= disabled_until_timestep)"),
    ("zero cutoff gates every step", "    if disabled_until_timestep == 0.0:\n        return 0\n", ""),
    ("no t published opens the gate", "    if t is None:\n        return False", "    if t is None:\n        return True"),
    ("flow shift without the -1", "shift * u / (1.0 + (shift - 1.0) * u)", "shift * u / (1.0 + shift * u)"),
    ("schedule keeps the last point", "    return ts[:-1]", "    return ts"),
    ("threshold not scaled by the length", "        return threshold * seqlen", "        return threshold"),
    ("calibrated curve with exp(b) * s", "return a * math.exp(b * target_sparsity)", "return a * math.exp(b) * target_sparsity"),
    ("ignore only the full name", "fnmatch.fnmatchcase(module_name, pat) or fnmatch.fnmatchcase(rel, pat)",
     "fnmatch.fnmatchcase(module_name, pat)"),
    ("ignored layers keep the threshold", "    if ignored:\n        return None\n", ""),
    ("both controls accepted", "    if (threshold is None) == (target_sparsity is None):", "    if threshold is None and target_sparsity is None:"),
    ("any formula accepted", "    if formula != FORMULA:", "    if False:"),
]


def _load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("config_mutant")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    assert old != new, f"mutant '{name}' changes nothing"
    mod = _load_mutant(old, new)
    failed = []
    for pin in config_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant '{name}' passed every pin"
