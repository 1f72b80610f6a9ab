"""Virtual tiles for skipped tiles (the fwd_virtual entry point) against the
CPU oracle's closed form ("Triage: Skip, Skim, or Refine Attention Tiles in
Video Diffusion Transformers", section 6.1 "Skipping with Virtual Tiles").

Bar: the same as the plain path (tests/parity.py).  The skip mask is the plain
method's, so the mask and counts must equal those of fwd_debug bit for bit;
O and LSE are compared with oracle.virtual_tile_head under the GPU's own mask.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from skip_softmax_flashattention_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    return m


def _check(ssa, w, name, qblocks=None, heads=None, **kw):
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    B, H, S, D = q.shape
    print(f"[case] {name} shape={tuple(q.shape)} {kw}", flush=True)
    o, lse, cnt = ssa.fwd_virtual(q, k, v, scale=w.scale, **kw)
    o2, lse2, cnt2 = ssa.fwd_virtual(q, k, v, scale=w.scale, **kw)
    _, _, cntd, mask, _ = ssa.fwd_debug(q, k, v, scale=w.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "fwd_virtual not deterministic"
    assert torch.equal(cnt, cntd), "virtual tiles changed the skip decisions"
    mask = mask.cpu().numpy().astype(bool)
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    nqb = mask.shape[2]
    qbs = np.arange(nqb) if qblocks is None else np.asarray(qblocks)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    errs, lerrs = [], []
    for (b, h) in heads:
        qd, kd, vd = (oracle.from_bf16(t[b, h]) for t in (w.q, w.k, w.v))
        ref_o, ref_lse = oracle.virtual_tile_head(qd, kd, vd, w.scale, mask[b, h][qbs], qblocks=qbs)
        rows = (qbs[:, None] * oracle.BLOCK_Q + np.arange(oracle.BLOCK_Q)[None, :]).reshape(-1)
        valid = rows < S
        errs.append(np.abs(o_np[b, h][rows[valid]] - ref_o.reshape(-1, D)[valid]))
        lerrs.append(np.abs(lse_np[b, h][rows[valid]] - ref_lse.reshape(-1)[valid]))
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    print(f"[case] {name}: skipped {int(mask.sum())}/{mask.size}, max|dO| {err.max():.2e} "
          f"mean|dO| {err.mean():.2e} max|dLSE| {lerr.max():.2e}", flush=True)
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    assert err.max() <= parity.O_MAX and err.mean() <= parity.O_MEAN
    assert lerr.max() <= parity.LSE_MAX
    return mask, o, lse


@pytest.mark.parametrize("factor", [0.5, 4.0, 40.0])
def test_virtual_tiny(ssa, factor):
    _check(ssa, inputs.tiny(), "virtual tiny", factor=factor)


@pytest.mark.parametrize("grid,factor", [((3, 10, 13), 0.05), ((3, 10, 13), 2.0), ((4, 16, 16), 0.5),
                                         ((5, 9, 23), 20.0)])
def test_virtual_grid(ssa, grid, factor):
    """Grid-local inputs with ragged query blocks and key tiles."""
    w = inputs.grid_small(11, grid, heads=2)
    S = w.q.shape[2]
    mask, _, _ = _check(ssa, w, f"virtual grid {grid}", factor=factor * S)
    assert mask.any()


def test_virtual_lambda_above_one(ssa):
    w = inputs.grid_small(12, (4, 12, 20), heads=2)
    _check(ssa, w, "virtual lambda > 1", threshold=3.0)


def test_virtual_without_skips_is_plain(ssa):
    """lambda = 0: no tile is virtual and the result is fwd's, bit for bit."""
    w = inputs.grid_small(13, (3, 10, 13), heads=2)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    o, lse, cnt = ssa.fwd_virtual(q, k, v, scale=w.scale, factor=0.0)
    o2, lse2, cnt2 = ssa.fwd(q, k, v, scale=w.scale, factor=0.0)
    torch.cuda.synchronize()
    assert int(cnt.sum()) == 0
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_virtual_constant_tiles_recover_dense(ssa):
    """Keys equal within each 128-key tile: a virtual key stands for its tile
    exactly, so the result is dense attention whatever is skipped.  Tile 0's
    key is aligned with every query (score about 4.3) and the other tiles
    keys are random (scores about N(0, 0.6)), so every later tile is skipped
    while still holding a large share of the softmax mass; values are
    constant per tile plus noise, so leaving that mass out moves O visibly."""
    rng = np.random.default_rng(14)
    B, H, S, D = 1, 2, 1000, 128
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    nkt = -(-S // 128)
    tile_keys = rng.standard_normal((B, H, nkt, D))
    tile_keys[:, :, 0] = 7.0 * u
    k = np.repeat(tile_keys, 128, axis=2)[:, :, :S]
    q = 7.0 * u + 0.3 * rng.standard_normal((B, H, S, D))
    v = np.repeat(rng.standard_normal((B, H, nkt, D)), 128, axis=2)[:, :, :S] + 0.1 * rng.standard_normal((B, H, S, D))
    t = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
    q_, k_, v_ = t(q), t(k), t(v)
    o, lse, cnt = ssa.fwd_virtual(q_, k_, v_, threshold=0.2)
    od, lsed, _ = ssa.fwd(q_, k_, v_, factor=0.0)
    os_, _, _ = ssa.fwd(q_, k_, v_, threshold=0.2)
    torch.cuda.synchronize()
    nqb = -(-S // 64)
    err = (o.float() - od.float()).abs()
    err_skip = (os_.float() - od.float()).abs()
    print(f"[case] constant tiles: skipped {int(cnt.sum())}/{B * H * nqb * nkt}, "
          f"max|O_virtual - O_dense| {float(err.max()):.2e}, max|O_skip - O_dense| {float(err_skip.max()):.2e}",
          flush=True)
    assert int(cnt.sum()) == B * H * nqb * (nkt - 1)
    assert float(err.max()) <= parity.O_MAX and float(err.mean()) <= parity.O_MEAN
    assert float((lse - lsed).abs().max()) <= parity.LSE_MAX
    assert float(err_skip.max()) > 10 * float(err.max())


def test_virtual_wan_like_sampled(ssa):
    """Full Wan-like problem at the lambda for 75% skipped tiles; seeded
    samples of query blocks against the oracle, plus the error to dense
    attention with and without the virtual tiles (reported)."""
    w = inputs.wan()
    lam = json.load(open(os.path.join(GOLDEN, "wan_lambdas.json")))["lambda"]["0.75"]
    S = w.q.shape[2]
    rng = np.random.default_rng(15)
    qbs = np.sort(rng.choice(-(-S // 64), 6, replace=False))
    qbs[-1] = -(-S // 64) - 1                      # the ragged last block
    _check(ssa, w, "virtual wan-like", qblocks=qbs, heads=[(0, 0), (0, 17), (0, 39)], factor=lam * S)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    ov, _, _ = ssa.fwd_virtual(q, k, v, scale=w.scale, factor=lam * S)
    os_, _, _ = ssa.fwd(q, k, v, scale=w.scale, factor=lam * S)
    od, _, _ = ssa.fwd(q, k, v, scale=w.scale, factor=0.0)
    torch.cuda.synchronize()
    den = od.float().abs().sum()
    rel_skip = float((os_.float() - od.float()).abs().sum() / den)
    rel_virt = float((ov.float() - od.float()).abs().sum() / den)
    print(f"[case] wan-like rel-L1 to dense: skip {rel_skip:.4e}, virtual tiles {rel_virt:.4e}", flush=True)


def test_virtual_long_sampled(ssa):
    """Long-sequence workload (S = 36864, H = 24, 2% sink keys) at threshold
    1e-3: sampled query blocks of two heads against the oracle."""
    w = inputs.long_seq()
    S = w.q.shape[2]
    rng = np.random.default_rng(16)
    qbs = np.sort(rng.choice(-(-S // 64), 5, replace=False))
    qbs[-1] = -(-S // 64) - 1
    _check(ssa, w, "virtual long", qblocks=qbs, heads=[(0, 0), (0, 23)], threshold=1e-3)


@pytest.mark.parametrize("control", ["threshold", "calib", "seqlen"])
def test_virtual_batched_controls(ssa, control):
    """B = 2 with each threshold control, including a seqlen other than S."""
    a, b = inputs.grid_small(33, (4, 12, 20), heads=2), inputs.grid_small(34, (4, 12, 20), heads=2)
    w = inputs.Workload("grid batch 2", torch.cat([a.q, b.q]), torch.cat([a.k, b.k]), torch.cat([a.v, b.v]))
    S = w.q.shape[2]
    kw = {"threshold": dict(threshold=0.01), "calib": dict(calib=(2.05276, 13.2810, 0.5)),
          "seqlen": dict(factor=0.02 * S, seqlen=2 * S)}[control]
    mask, _, _ = _check(ssa, w, f"virtual batched {control}", **kw)
    assert mask.any()


@pytest.mark.parametrize("S", [1, 63, 129, 300])
def test_virtual_edge_lengths(ssa, S):
    """Shorter than a query block, one key past a tile, ragged in both."""
    w = inputs.random_qkv(200 + S, 2, 3, S, qk_gain=2.0)
    _check(ssa, w, f"virtual edge S={S}", factor=0.3 * S)


@pytest.mark.parametrize("i", range(0, 16, 2))
def test_random_grid_sweep(ssa, i):
    """Every other case of the plain path's seeded shape sweep (ragged
    grid-local problems at thresholds 0.05 to 10) on the virtual-tile entry."""
    from tests.test_gpu_parity import _sweep_case
    w, lam = _sweep_case(i)
    _check(ssa, w, f"virtual-tile sweep {i} S={w.q.shape[2]} lambda={lam:.4g}", threshold=lam)
