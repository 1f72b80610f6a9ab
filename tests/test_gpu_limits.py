"""The entry points at their largest accepted key-tile counts, on the GPU.

Grid-locality inputs (the Wan-like generator) at lengths where the tile
counts reach the limits the entries document:

  * the plain pass at 2,048 key tiles (S = 262,144);
  * virtual tiles at their limit of 2,048 key tiles (S = 262,144);
  * FP8 scores at their limit of 4,096 key tiles (S = 524,288).

Each checks sampled query blocks (the first, the last and random ones) of
one head against the oracle.  Rows are independent given K and V, so a
sampled block is checked exactly.  One tile past each limit is refused with
SSA_ERR_UNSUPPORTED on the host; tests/test_abi.py checks that without a GPU.
"""
import numpy as np
import pytest

from oracle import c_oracle
from skip_softmax_flashattention_amd import inputs
from tests import parity
from tests.test_gpu_fp8 import _check_attention as _check_fp8_attention
from tests.test_gpu_fp8 import _check_quant as _check_fp8_quant
from tests.test_gpu_virtual import _check as _check_virtual

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    return m


def _blocks(S, n, seed):
    nqb = -(-S // 64)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, nqb - 1], rng.choice(nqb, n, replace=False)]))


@pytest.fixture(scope="module")
def w2048():
    return inputs.grid_small(31, (64, 64, 64), heads=1)


def test_plain_at_2048_tiles(ssa, w2048):
    """S = 262,144 at threshold 1e-3, against the single-precision C oracle."""
    S = w2048.q.shape[2]
    assert -(-S // 128) == 2048
    qbs = _blocks(S, 5, 41)
    print(f"[case] plain S={S} blocks={qbs.tolist()}", flush=True)
    rep = parity.check_fixed(ssa, w2048, threshold=1e-3, qblocks=qbs, ref=c_oracle.oracle().skip_head)
    print(f"[case] plain S={S}: {rep}", flush=True)
    parity.assert_bar(rep)
    assert rep.skipped > 0


def test_virtual_at_2048_tiles(ssa, w2048):
    """Virtual tiles at their limit, S = 262,144, threshold 1e-3."""
    S = w2048.q.shape[2]
    mask, _, _ = _check_virtual(ssa, w2048, f"virtual S={S}", qblocks=_blocks(S, 3, 42), threshold=1e-3)
    assert mask.any()


def test_fp8_at_4096_tiles(ssa):
    """FP8 scores at their limit, S = 524,288: the quantiser on sampled tokens
    and tiles, the attention on sampled blocks at threshold 1e-3."""
    w = inputs.grid_small(32, (64, 64, 128), heads=1)
    S = w.q.shape[2]
    assert -(-S // 128) == 4096
    rng = np.random.default_rng(43)
    _check_fp8_quant(ssa, w, rows=np.sort(rng.choice(S, 4000, replace=False)),
                     tiles=np.concatenate([[0, 4095], np.sort(rng.choice(4096, 16, replace=False))]))
    mask = _check_fp8_attention(ssa, w, f"fp8 S={S}", qblocks=_blocks(S, 2, 44), threshold=1e-3)
    assert mask.any()
