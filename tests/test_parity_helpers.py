"""The whole-mask comparison the full-size GPU tests use (tests/parity.py,
whole_mask_forced), exercised on the CPU with masks the oracle makes: its own
mask passes, a decision flipped outside the 1e-3 band fails, and one flipped
inside the band passes and is counted."""
import numpy as np
import pytest

import oracle
from tests import parity
from tests.oracle_pins import _peaky_head


def _heads():
    q, k, _ = _peaky_head(21, 700, 16)
    return np.stack([oracle.tile_row_maxima_head(a, b, 2.0, block_k=32) for a, b in ((q, k), (k, q))])


def _forced_margins(tms, mask, ln):
    return np.stack([oracle.skip_mask_from_row_maxima(tms[h], ln, forced_skip=mask[h], block_q=32)[1]
                     for h in range(len(tms))])


@pytest.mark.parametrize("lam", [0.1, 4.0])
def test_own_mask_passes_and_flips_are_caught(lam):
    tms = _heads()
    ln = oracle.ln_lambda_f32(lam)
    mask, margins = oracle.skip_mask_from_row_maxima(tms, ln, block_q=32)
    assert 0 < mask.sum() < mask.size
    exact, differ = parity.whole_mask_forced(mask, _forced_margins(tms, mask, ln), ln)
    assert differ == 0 and exact > 0.9 * mask.size
    # flip the decision with the largest distance from ln(lambda)
    far = np.unravel_index(np.argmax(np.where(np.isfinite(margins), np.abs(margins - ln), -1.0)), mask.shape)
    bad = mask.copy()
    bad[far] = ~bad[far]
    with pytest.raises(AssertionError, match="outside the band"):
        parity.whole_mask_forced(bad, _forced_margins(tms, bad, ln), ln)


def test_flip_inside_the_band_is_tolerated():
    tms = _heads()
    _, margins = oracle.skip_mask_from_row_maxima(tms, oracle.ln_lambda_f32(0.1), block_q=32)
    # ln(lambda) placed exactly on a negative margin: the strict test keeps that tile
    ln = np.float32(np.sort(margins[np.isfinite(margins) & (margins < -0.5)])[len(margins) // 3])
    mask, margins = oracle.skip_mask_from_row_maxima(tms, ln, block_q=32)
    tie = np.argwhere(margins == ln)
    assert len(tie) and not mask[tuple(tie[0])]
    flipped = mask.copy()
    flipped[tuple(tie[0])] = True
    exact, differ = parity.whole_mask_forced(flipped, _forced_margins(tms, flipped, ln), ln)
    assert differ == 1
