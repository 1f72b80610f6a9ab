"""FP8 scores (quantize_qk_fp8 + fwd_fp8) against the CPU oracle.

The quantiser is integer work: codes and scales must equal the oracle's
(oracle/fp8.py) bit for bit.  The attention is compared with the oracle's
recurrence run on the dequantised operands.  The E4M3 MFMA does not sum its
products exactly: it stays within about 2^-12 of the sum of the products'
magnitudes (random codes over the full range), which
test_fp8_mfma_dot_error_within_eps measures on every run.  The bound used
here is EPS = 2^-10 of that sum, per score (oracle.fp8.score_error_bound):
  * mask: identical to the oracle outside a band of 1e-3 plus twice the largest
    bound of the block's rows (the margin is a difference of two scores);
  * O: against the oracle forced to the GPU's mask, the bars of tests/parity.py;
  * LSE: within 1e-3 plus twice the row's bound.
At full size (Wan-like, long sequence) the quantiser and the tile mask are
checked over the whole problem, O and LSE on sampled query blocks.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle
from oracle import fp8 as ofp8
from skip_softmax_flashattention_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS = 2.0 ** -10


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    return m


def _check_quant(ssa, w, heads=None, rows=None, tiles=None):
    q, k = w.q.cuda(), w.k.cuda()
    q8, k8, qs, ks = (t.cpu().numpy() for t in ssa.quantize_qk_fp8(q, k))
    B, H, S, D = w.q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    out = {}
    for (b, h) in heads:
        ref = ofp8.quantize_head(oracle.from_bf16(w.q[b, h]), oracle.from_bf16(w.k[b, h]))
        r = np.arange(S) if rows is None else rows
        t = np.arange(ks.shape[2]) if tiles is None else tiles
        assert (q8[b, h][r] == ref.q_codes[r]).all(), f"q codes differ in head {(b, h)}"
        assert (qs[b, h][r] == ref.q_scale[r]).all(), f"q scales differ in head {(b, h)}"
        assert (ks[b, h][t] == ref.k_scale[t]).all(), f"k scales differ in head {(b, h)}"
        for ti in t:
            sl = slice(128 * ti, min(S, 128 * (ti + 1)))
            assert (k8[b, h][sl] == ref.k_codes[sl]).all(), f"k codes differ in head {(b, h)} tile {ti}"
        out[(b, h)] = ref
    return out


def _check_attention(ssa, w, name, qblocks=None, heads=None, **kw):
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    B, H, S, D = q.shape
    print(f"[case] {name} shape={tuple(q.shape)} {kw}", flush=True)
    q8, k8, qs, ks = ssa.quantize_qk_fp8(q, k)
    o, lse, cnt = ssa.fwd_fp8(q8, k8, qs, ks, v, scale=w.scale, **kw)
    o2, lse2, cnt2, mask, _ = ssa.fwd_fp8(q8, k8, qs, ks, v, scale=w.scale, debug=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(cnt, cnt2), "product and debug entries differ"
    mask = mask.cpu().numpy().astype(bool)
    assert (cnt.cpu().numpy() == mask.sum(-1)).all()
    n = S if kw.get("seqlen") is None else kw["seqlen"]
    if kw.get("threshold") is not None:
        lam = oracle.resolve_lambda(threshold=kw["threshold"])
    elif kw.get("calib") is not None:
        a, bb, ts = kw["calib"]
        lam = oracle.resolve_lambda(a=a, b=bb, target_sparsity=ts, seqlen=n)
    else:
        lam = oracle.resolve_lambda(factor=kw["factor"], seqlen=n)
    ln = oracle.ln_lambda_f32(lam)
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    nqb = mask.shape[2]
    qbs = np.arange(nqb) if qblocks is None else np.asarray(qblocks)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    errs, lerr_over, exempt, worst_bound = [], [], 0, 0.0
    for (b, h) in heads:
        ops = ofp8.quantize_head(oracle.from_bf16(w.q[b, h]), oracle.from_bf16(w.k[b, h]))
        vd = oracle.from_bf16(w.v[b, h])
        rows = (qbs[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
        valid = rows < S
        bound_rows = np.zeros(rows.shape)
        bound_rows[valid] = ofp8.score_error_bound(ops, w.scale, rows[valid], EPS).max(axis=1)
        worst_bound = max(worst_bound, float(bound_rows.max()))
        own = oracle.skip_head(ops.q, ops.k, vd, w.scale, ln, qblocks=qbs)
        gm = mask[b, h][qbs]
        if ln is not None:
            band = 1e-3 + 2 * bound_rows.reshape(len(qbs), 64).max(axis=1)[:, None]
            near = np.abs(own.margin.astype(np.float64) - float(ln)) <= band
            bad = (gm != own.skipped) & ~near
            assert not bad.any(), f"{int(bad.sum())} tile decisions differ outside the band"
            exempt += int((near & (gm != own.skipped)).sum())
        forced = oracle.skip_head(ops.q, ops.k, vd, w.scale, None, qblocks=qbs, forced_skip=gm)
        o_ref = forced.o.reshape(-1, D)[valid]
        lse_ref = forced.lse.reshape(-1)[valid]
        errs.append(np.abs(o_np[b, h][rows[valid]] - o_ref))
        lerr_over.append(np.abs(lse_np[b, h][rows[valid]] - lse_ref) - (1e-3 + 2 * bound_rows[valid]))
    err = np.concatenate(errs)
    lover = np.concatenate(lerr_over)
    print(f"[case] {name}: skipped {int(mask.sum())}/{mask.size} exempt {exempt}, max|dO| {err.max():.2e} "
          f"mean|dO| {err.mean():.2e}, max(|dLSE| - tol) {lover.max():.2e}, largest score bound {worst_bound:.2e}",
          flush=True)
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    assert err.max() <= parity.O_MAX and err.mean() <= parity.O_MEAN
    assert lover.max() <= 0.0
    return mask


def test_fp8_mfma_dot_error_within_eps(ssa):
    """The E4M3 MFMA's summation error, measured on every run against the
    bound the FP8 tests use: |computed - exact| <= EPS * sum |q_d k_d| (times
    the scales).  Each of 4096 heads holds one query and one key (S = 1), so
    the kernel's LSE is exactly its one score, up to float rounding of the
    score factor and the exponent reference (about 1e-6 of the score, which
    the sum of magnitudes bounds).  Half the heads use E4M3 codes drawn
    uniformly over every finite code (one element of each row set to 448, so
    the scale is 1 and the codes pass through the quantiser unchanged), half
    use normal values times 2^U(-8, 0) (a wide spread of exponents in every
    dot product).  The exact dot product of decoded codes is exact in
    float64."""
    rng = np.random.default_rng(90)
    H, D = 4096, 128
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.empty((2, H, D))
    for i in range(2):
        codes = rng.choice(finite, size=(H // 2, D))
        x = ofp8.e4m3_decode(codes)
        x[:, 0] = 448.0
        vals[i, : H // 2] = x
        vals[i, H // 2:] = rng.standard_normal((H // 2, D)) * np.exp2(rng.uniform(-8, 0, (H // 2, D)))
    t = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).reshape(1, H, 1, D).cuda()
    q, k = t(vals[0]), t(vals[1])
    v = torch.ones_like(q)
    scale = float(np.float32(1 / np.sqrt(D)))
    q8, k8, qs, ks = ssa.quantize_qk_fp8(q, k)
    _, lse, _ = ssa.fwd_fp8(q8, k8, qs, ks, v, scale=scale, factor=0.0)
    torch.cuda.synchronize()
    dq = ofp8.e4m3_decode(q8.cpu().numpy().reshape(H, D))
    dk = ofp8.e4m3_decode(k8.cpu().numpy().reshape(H, D))
    fac = scale * qs.cpu().numpy().reshape(H).astype(np.float64) * ks.cpu().numpy().reshape(H).astype(np.float64)
    exact = fac * (dq * dk).sum(axis=1)
    unit = fac * np.abs(dq * dk).sum(axis=1)
    assert (q8.cpu().numpy().reshape(H, D)[: H // 2] == ofp8.e4m3_encode(vals[0, : H // 2].astype(np.float32))).all()
    ratio = np.abs(lse.cpu().numpy().reshape(H).astype(np.float64) - exact) / unit
    print(f"[case] fp8 MFMA dot error: max {ratio.max():.3e} = 2^{np.log2(ratio.max()):.2f} of sum|ab| "
          f"(uniform codes {ratio[: H // 2].max():.3e}, spread normals {ratio[H // 2:].max():.3e}); bound EPS = 2^-10",
          flush=True)
    assert np.isfinite(ratio).all()
    assert ratio.max() <= EPS


def test_quantize_tiny(ssa):
    _check_quant(ssa, inputs.tiny())


@pytest.mark.parametrize("grid", [(3, 10, 13), (5, 9, 23)])
def test_quantize_ragged(ssa, grid):
    w = inputs.grid_small(21, grid, heads=3)
    _check_quant(ssa, w)


def test_quantize_zero_and_extreme_rows(ssa):
    """An all-zero token (scale 1, codes 0), a token of one huge value and a
    key tile of tiny values."""
    rng = np.random.default_rng(22)
    q = rng.standard_normal((1, 1, 300, 128))
    k = rng.standard_normal((1, 1, 300, 128))
    q[0, 0, 5] = 0.0
    q[0, 0, 6] = 1e-3 * rng.standard_normal(128)
    q[0, 0, 6, 3] = 300.0
    k[0, 0, 128:256] *= 1e-4
    t = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    w = inputs.Workload("extreme", t(q), t(k), t(k))
    _check_quant(ssa, w)


@pytest.mark.parametrize("factor", [0.0, 4.0])
def test_fp8_tiny(ssa, factor):
    m = _check_attention(ssa, inputs.tiny(), "fp8 tiny", factor=factor)
    if factor == 0.0:
        assert not m.any()


@pytest.mark.parametrize("grid,factor", [((3, 10, 13), 0.05), ((4, 16, 16), 0.5), ((5, 9, 23), 20.0)])
def test_fp8_grid(ssa, grid, factor):
    w = inputs.grid_small(23, grid, heads=2)
    S = w.q.shape[2]
    m = _check_attention(ssa, w, f"fp8 grid {grid}", factor=factor * S)
    assert m.any()


def test_fp8_lambda_above_one(ssa):
    w = inputs.grid_small(24, (4, 12, 20), heads=2)
    _check_attention(ssa, w, "fp8 lambda > 1", threshold=3.0)


def _whole_fp8(ssa, w, name, mask, ln):
    """The whole problem (B = 1): the quantiser's codes and scales of every
    head bit for bit, and every tile decision against the oracle's decision
    recurrence on the dequantised operands (oracle.tile_row_maxima_head,
    oracle.skip_mask_from_row_maxima driven by the kernel's mask).  The band
    of a block is 1e-3 plus twice the largest bound of its rows, each row's
    bound taken with Cauchy-Schwarz, |decode(q_i)| |decode(k_c)| >=
    sum_d |decode(q_id)| |decode(k_cd)|, so it is never below the one the
    sampled checks use (oracle.fp8.score_error_bound)."""
    q8, k8, qs, ks = (t.cpu().numpy() for t in ssa.quantize_qk_fp8(w.q.cuda(), w.k.cuda()))
    H, S = w.q.shape[1], w.q.shape[2]
    nqb = -(-S // 64)

    def head(h):
        ops = ofp8.quantize_head(oracle.from_bf16(w.q[0, h]), oracle.from_bf16(w.k[0, h]))
        same = bool((q8[0, h] == ops.q_codes).all() and (k8[0, h] == ops.k_codes).all()
                    and (qs[0, h] == ops.q_scale).all() and (ks[0, h] == ops.k_scale).all())
        tm = oracle.tile_row_maxima_head(ops.q, ops.k, w.scale)
        _, margins = oracle.skip_mask_from_row_maxima(tm, ln, forced_skip=mask[0, h])
        nq = np.linalg.norm(ofp8.e4m3_decode(ops.q_codes), axis=1) * ops.q_scale.astype(np.float64)
        nk = np.linalg.norm(ofp8.e4m3_decode(ops.k_codes), axis=1) * ops.k_scale[np.arange(S) // 128]
        bound = np.zeros(nqb * 64)
        bound[:S] = EPS * w.scale * nq * nk.max()
        band = 1e-3 + 2 * bound.reshape(nqb, 64).max(axis=1)[:, None]
        near = np.abs(margins.astype(np.float64) - float(ln)) <= band
        diff = mask[0, h] != (margins < np.float32(ln))
        return same, int((diff & ~near).sum()), int((diff & near).sum()), int((~near).sum()), float(band.max())

    with threadpool_limits(1), ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        res = list(ex.map(head, range(H)))
    print(f"[whole fp8] {name}: {H} heads: quantiser {'equal' if all(r[0] for r in res) else 'DIFFERS'}; "
          f"{sum(r[3] for r in res)} tiles outside the band, {sum(r[1] for r in res)} of them different; "
          f"{sum(r[2] for r in res)} inside the band different; widest band {max(r[4] for r in res):.2e}", flush=True)
    assert all(r[0] for r in res), [h for h, r in enumerate(res) if not r[0]]
    assert sum(r[1] for r in res) == 0


def test_fp8_wan_like(ssa):
    """The full Wan-like problem: the quantiser and the tile mask over the
    whole problem, sampled query blocks of the attention's O and LSE, and the
    FP8 output's distance to the bf16 path's (reported)."""
    w = inputs.wan()
    S = w.q.shape[2]
    rng = np.random.default_rng(25)
    lam = json.load(open(os.path.join(GOLDEN, "wan_lambdas.json")))["lambda"]["0.75"]
    qbs = np.sort(rng.choice(-(-S // 64), 5, replace=False))
    qbs[-1] = -(-S // 64) - 1
    mask = _check_attention(ssa, w, "fp8 wan-like", qblocks=qbs, heads=[(0, 0), (0, 39)], factor=lam * S)
    _whole_fp8(ssa, w, "wan-like", mask, oracle.ln_lambda_f32(oracle.resolve_lambda(factor=lam * S, seqlen=S)))
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    q8, k8, qs, ks = ssa.quantize_qk_fp8(q, k)
    o8, _, c8 = ssa.fwd_fp8(q8, k8, qs, ks, v, scale=w.scale, factor=lam * S)
    ob, _, cb = ssa.fwd(q, k, v, scale=w.scale, factor=lam * S)
    od, _, _ = ssa.fwd(q, k, v, scale=w.scale, factor=0.0)
    torch.cuda.synchronize()
    den = od.float().abs().sum()
    print(f"[case] wan-like: skipped fp8 {int(c8.sum())} bf16 {int(cb.sum())}; rel-L1 to bf16 dense: fp8 "
          f"{float((o8.float() - od.float()).abs().sum() / den):.4e}, bf16 {float((ob.float() - od.float()).abs().sum() / den):.4e}",
          flush=True)


def test_fp8_long(ssa):
    """Long-sequence workload (S = 36864, H = 24, 2% sink keys scaled x4) at
    threshold 1e-3: the quantiser and the tile mask over the whole problem,
    O and LSE on sampled blocks."""
    w = inputs.long_seq()
    S = w.q.shape[2]
    rng = np.random.default_rng(26)
    qbs = np.sort(rng.choice(-(-S // 64), 5, replace=False))
    qbs[-1] = -(-S // 64) - 1
    mask = _check_attention(ssa, w, "fp8 long", qblocks=qbs, heads=[(0, 0), (0, 23)], threshold=1e-3)
    _whole_fp8(ssa, w, "long", mask, oracle.ln_lambda_f32(1e-3))


def _batched(seed):
    a, b = inputs.grid_small(seed, (4, 12, 20), heads=2), inputs.grid_small(seed + 1, (4, 12, 20), heads=2)
    return inputs.Workload("grid batch 2", torch.cat([a.q, b.q]), torch.cat([a.k, b.k]), torch.cat([a.v, b.v]))


@pytest.mark.parametrize("control", ["threshold", "calib", "seqlen"])
def test_fp8_batched_controls(ssa, control):
    """B = 2 with each threshold control, including a seqlen other than S."""
    w = _batched(27)
    S = w.q.shape[2]
    kw = {"threshold": dict(threshold=0.01), "calib": dict(calib=(2.05276, 13.2810, 0.5)),
          "seqlen": dict(factor=0.02 * S, seqlen=2 * S)}[control]
    m = _check_attention(ssa, w, f"fp8 batched {control}", **kw)
    assert m.any()


@pytest.mark.parametrize("S", [1, 63, 129, 300])
def test_fp8_edge_lengths(ssa, S):
    """Shorter than a query block, one key past a tile, ragged in both."""
    w = inputs.random_qkv(200 + S, 2, 3, S, qk_gain=2.0)
    _check_attention(ssa, w, f"fp8 edge S={S}", factor=0.3 * S)


@pytest.mark.parametrize("i", range(0, 16, 2))
def test_random_grid_sweep(ssa, i):
    """Every other case of the plain path's seeded shape sweep (ragged
    grid-local problems at thresholds 0.05 to 10) on the FP8 entry."""
    from tests.test_gpu_parity import _sweep_case
    w, lam = _sweep_case(i)
    _check_attention(ssa, w, f"fp8 sweep {i} S={w.q.shape[2]} lambda={lam:.4g}", threshold=lam)
