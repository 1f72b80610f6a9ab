"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
every one of them fails at least one pin from tests/oracle_pins.py.

A mutant is made by a textual replacement in oracle/skip_attention.py; the
test first checks that the replacement really changes the source, so a
refactor of the oracle cannot silently turn a mutant into the original.
"""
import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "skip_attention.py")

MUTANTS = [
    ("score scale dropped",
     "s = float(scale) * (qr @ k[c0:c1].T)", "s = (qr @ k[c0:c1].T)"),
    ("q and k swapped in the dense scores",
     "s = float(scale) * (q[r] @ k.T)", "s = float(scale) * (k[r] @ q.T)"),
    ("margin sign flipped",
     "d = tile_max.astype(np.float32) - m.astype(np.float32)",
     "d = m.astype(np.float32) - tile_max.astype(np.float32)"),
    ("vote on any row instead of every row",
     "margin[:, kt] = d.max(axis=1)", "margin[:, kt] = d.min(axis=1)"),
    ("non-strict comparison",
     "skip = margin[:, kt] < np.float32(ln_lambda)", "skip = margin[:, kt] <= np.float32(ln_lambda)"),
    ("padding rows vote",
     "d = np.where(valid, d, np.float32(-np.inf))", "d = d"),
    ("rescale factor inverted",
     "alpha = np.exp(m[kb] - m_new)", "alpha = np.exp(m_new - m[kb])"),
    ("l not rescaled",
     "l[kb] = alpha * l[kb] + p.sum(axis=2)", "l[kb] = l[kb] + p.sum(axis=2)"),
    ("tile drops its last key",
     "c0, c1 = kt * block_k, min(S, (kt + 1) * block_k)",
     "c0, c1 = kt * block_k, min(S, (kt + 1) * block_k - 1)"),
    ("running max taken after absorbing the tile",
     "d = tile_max.astype(np.float32) - m.astype(np.float32)",
     "d = tile_max.astype(np.float32) - np.maximum(m, tile_max).astype(np.float32)"),
    ("skipped tiles still raise m",
     "        if not keep.any():\n            continue\n",
     "        m = np.maximum(m, np.where(skip[:, None], tile_max, -np.inf))\n"
     "        if not keep.any():\n            continue\n"),
    ("lse without the running max",
     "lse = m + np.log(l)", "lse = np.log(l)"),
    ("dense lse without the row max",
     "lse[c0:c0 + chunk] = mx[:, 0] + np.log(den)", "lse[c0:c0 + chunk] = np.log(den)"),
    ("threshold not divided by length",
     "lam = float(factor) / float(seqlen)", "lam = float(factor)"),
    ("calibrated curve with exp(b) * s",
     "lam = float(a) * math.exp(float(b) * float(target_sparsity)) / float(seqlen)",
     "lam = float(a) * math.exp(float(b)) * float(target_sparsity) / float(seqlen)"),
    ("zero threshold not special",
     "    if lam == 0.0:\n        return None\n", "    if lam == 0.0:\n        return np.float32(-1e30)\n"),
    ("masked closed form keeps skipped keys",
     "allowed = ~skipped[qb][key_tile]", "allowed = np.ones_like(skipped[qb][key_tile])"),
    ("prefix max includes the current tile",
     "np.maximum.accumulate(tmax, axis=1)[:, :-1]",
     "np.maximum.accumulate(tmax, axis=1)[:, 1:]"),
    ("varlen uses the packed length",
     "r = skip_attention(qs, ks, vs, scale, ln_lambda_f32(lambdas[bi]),",
     "r = skip_attention(qs, ks, vs, scale, ln_lambda_f32(lambdas[0]),"),
    ("virtual score without the log count",
     "s_virt = float(scale) * (q[r0:r1] @ kmean[sk].T) + np.log(counts[sk])[None, :]",
     "s_virt = float(scale) * (q[r0:r1] @ kmean[sk].T)"),
    ("virtual value is the tile sum",
     "vmean = np.stack([v[t * block_k:min(S, (t + 1) * block_k)].mean(axis=0)",
     "vmean = np.stack([v[t * block_k:min(S, (t + 1) * block_k)].sum(axis=0)"),
    ("virtual key is the tile maximum",
     "kmean = np.stack([k[t * block_k:min(S, (t + 1) * block_k)].mean(axis=0)",
     "kmean = np.stack([k[t * block_k:min(S, (t + 1) * block_k)].max(axis=0)"),
    ("ragged tile counted as full",
     "counts = np.array([min(S, (t + 1) * block_k) - t * block_k for t in range(nkt)], dtype=np.float64)",
     "counts = np.array([block_k for t in range(nkt)], dtype=np.float64)"),
    ("virtual keys double-count kept keys",
     "kept = ~sk[key_tile]", "kept = np.ones(S, dtype=bool)"),
    ("row maxima: last partial tile dropped",
     "        if nfull < nkt:\n            out[r0:r0 + chunk, nfull] = s[:, nfull * block_k:].max(axis=1)\n",
     "        if nfull < nkt:\n            out[r0:r0 + chunk, nfull] = s[:, (nfull - 1) * block_k:].max(axis=1)\n"),
    ("row maxima without the scale",
     "s = float(scale) * (q[r0:r0 + chunk] @ kT)", "s = (q[r0:r0 + chunk] @ kT)"),
    ("row-maxima recurrence: skipped tiles raise m",
     "m = np.where(skip[..., None], m, np.maximum(m, t))", "m = np.maximum(m, t)"),
    ("row-maxima recurrence: padding rows vote",
     "d = np.where(valid, t - m, np.float32(-np.inf))", "d = t - m"),
    ("row-maxima recurrence: vote on any row",
     "margin[..., kt] = d.max(axis=-1)", "margin[..., kt] = d.min(axis=-1)"),
    ("row-maxima recurrence: non-strict comparison",
     "skip = margin[..., kt] < np.float32(ln_lambda)", "skip = margin[..., kt] <= np.float32(ln_lambda)"),
    ("lambda for a fraction one step too low",
     "ln_lam = float(np.nextafter(np.float32(edge), np.float32(np.inf)))", "ln_lam = float(np.float32(edge))"),
    ("lambda for a fraction with the count rounded down",
     "need = int(math.ceil(fraction * n))", "need = max(1, int(math.floor(fraction * n)))"),
    ("lambda for a fraction off by one tile",
     "edge = flat[need - 1]", "edge = flat[min(need, n - 1)]"),
]


def _load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash the mutant causes
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant '{name}' passed every pin"
