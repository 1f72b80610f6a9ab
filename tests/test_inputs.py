"""Seeded input generators: shapes, dtypes, determinism and layout."""
import hashlib

import numpy as np
import torch

from skip_softmax_flashattention_amd import inputs


def _digest(w):
    h = hashlib.sha256()
    for t in (w.q, w.k, w.v):
        h.update(t.view(torch.int16).numpy().tobytes())
    return h.hexdigest()


def test_tiny_shape_and_determinism():
    a, b = inputs.tiny(), inputs.tiny()
    assert a.q.shape == (1, 2, 1024, 128) and a.q.dtype == torch.bfloat16
    assert _digest(a) == _digest(b)
    assert _digest(a) != _digest(inputs.tiny(seed=1))
    assert abs(a.scale - 1 / np.sqrt(128)) < 1e-7


def test_mid_k_is_q():
    w = inputs.mid()
    assert w.q.shape == (2, 8, 4096, 128)
    assert torch.equal(w.q, w.k)


def test_grid_embedding_norm_and_layout():
    pe = inputs.grid_embedding(21, 30, 52)
    assert pe.shape == (32760, 128)
    assert np.allclose((pe ** 2).sum(1), 64.0)
    # raster order: token n = (t * 30 + h) * 52 + w shares its frame channels with n + 1
    assert np.array_equal(pe[0, :44], pe[51, :44])
    assert not np.array_equal(pe[0, :44], pe[30 * 52, :44])


def test_wan_like_small_heads():
    w = inputs.wan(heads=1)
    assert w.q.shape == (1, 1, 32760, 128) and w.k.shape == w.q.shape


def test_long_has_sinks():
    w = inputs.long_seq(heads=1)
    assert w.q.shape == (1, 1, 36864, 128)
    norms = w.k.float().norm(dim=-1)[0, 0]
    assert int((norms > 2.5 * norms.median()).sum()) == 737


def test_varlen_packing():
    w = inputs.varlen(heads=2, grids=((2, 4, 8), (3, 5, 7)))
    assert w.cu_seqlens.tolist() == [0, 64, 169]
    assert w.q.shape == (169, 2, 128)
    parts = inputs.unpack_varlen(w.q, w.cu_seqlens)
    assert [p.shape for p in parts] == [(1, 2, 64, 128), (1, 2, 105, 128)]
    assert torch.equal(parts[1][0, 1, 3], w.q[64 + 3, 1])
