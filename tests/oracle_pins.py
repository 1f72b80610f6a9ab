"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
module disagrees with something that does not come from the oracle itself:
a library routine (torch's scaled_dot_product_attention and logsumexp in
float64), brute force in plain Python on tiny inputs, closed forms that follow
from the recurrence, and statements the pages make:

  [design] "Skip-Softmax" design document of vLLM-Omni: section "Algorithm"
           (the test, its upper-bound reading, skipped tiles are left out, the
           log-space form), section "From configuration to the kernel
           threshold" (lambda = factor / max_kv_len, the table of the two
           controls, a zero threshold skips no tiles, the calibration JSON).
  [docs]   "Skip-Softmax" page of the vLLM-Omni documentation: "The
           online-softmax pass" (128-key tiles, scale), "The skip test",
           "The threshold".

The same pins run against mutated copies of the oracle in
test_oracle_mutants.py: every plausible mistake planted there must fail at
least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, *shape, gain=1.0):
    return gain * np.random.default_rng(seed).standard_normal(shape)


def _peaky_head(seed, s, d, gain=3.0):
    """q = k-ish unit directions with a strong diagonal: gives a mix of kept
    and skipped tiles at small block sizes."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((s, d))
    base /= np.linalg.norm(base, axis=1, keepdims=True)
    q = gain * base + 0.3 * rng.standard_normal((s, d))
    k = gain * base + 0.3 * rng.standard_normal((s, d))
    v = rng.standard_normal((s, d))
    return q, k, v


# ---------------------------------------------------------------- dense part
def pin_dense_matches_torch_sdpa(orc):
    """Dense attention equals torch's float64 SDPA; LSE equals torch.logsumexp."""
    q, k, v = _rand(1, 2, 3, 150, 16), _rand(2, 2, 3, 150, 16), _rand(3, 2, 3, 150, 16)
    scale = 0.3
    o, lse = orc.dense_attention(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    ref_lse = torch.logsumexp(scale * tq @ tk.transpose(-1, -2), dim=-1).numpy()
    assert np.abs(o - ref).max() < 1e-12, np.abs(o - ref).max()
    assert np.abs(lse - ref_lse).max() < 1e-12


def pin_dense_bruteforce(orc):
    """Plain-Python softmax attention on a 5-token, 3-channel head."""
    q, k, v = _rand(4, 5, 3), _rand(5, 5, 3), _rand(6, 5, 3)
    scale = 0.7
    o, lse = orc.dense_head(q, k, v, scale)
    for i in range(5):
        s = [scale * sum(q[i][t] * k[j][t] for t in range(3)) for j in range(5)]
        den = sum(math.exp(x) for x in s)
        for t in range(3):
            want = sum(math.exp(s[j]) * v[j][t] for j in range(5)) / den
            assert abs(o[i][t] - want) < 1e-12
        assert abs(lse[i] - math.log(den)) < 1e-12


# ------------------------------------------------------------ threshold zero
def pin_zero_threshold_is_dense(orc):
    """[design] 'From configuration to the kernel threshold': a zero threshold
    skips no tiles, so the pass equals dense attention (ragged S: 300 rows
    give a 44-row last query block and a 44-key last tile)."""
    q, k, v = _rand(7, 1, 2, 300, 32), _rand(8, 1, 2, 300, 32), _rand(9, 1, 2, 300, 32)
    scale = 1 / math.sqrt(32)
    r = orc.skip_attention(q, k, v, scale, orc.ln_lambda_f32(0.0))
    o, lse = orc.dense_attention(q, k, v, scale)
    assert not r.skipped.any()
    assert np.abs(r.o - o).max() < 1e-12
    assert np.abs(r.lse - lse).max() < 1e-12
    assert r.skipped.shape == (1, 2, 5, 3)


def pin_zero_threshold_is_dense_default_tiles_sdpa(orc):
    """Same with the real 64 x 128 tiles, checked directly against torch SDPA."""
    q, k, v = _rand(10, 1, 1, 1000, 128), _rand(11, 1, 1, 1000, 128), _rand(12, 1, 1, 1000, 128)
    scale = 1 / math.sqrt(128)
    r = orc.skip_attention(q, k, v, scale, None)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    assert np.abs(r.o - ref).max() < 1e-12
    assert r.skipped.shape == (1, 1, 16, 8)


# ----------------------------------------------------------- mask closed form
def _bruteforce_mask(q, k, scale, ln_lam, bq, bk):
    """Plain-Python mask for lambda <= 1: skip[qb, kt] iff for every valid row,
    f32(max score in tile kt) - f32(max score over keys before tile kt) < ln_lam."""
    S = len(q)
    D = len(q[0])
    s = [[scale * sum(q[i][t] * k[j][t] for t in range(D)) for j in range(S)] for i in range(S)]
    nqb, nkt = -(-S // bq), -(-S // bk)
    mask = [[False] * nkt for _ in range(nqb)]
    margin = [[0.0] * nkt for _ in range(nqb)]
    for qb in range(nqb):
        for kt in range(nkt):
            worst = -math.inf
            for i in range(qb * bq, min(S, (qb + 1) * bq)):
                tmax = max(s[i][kt * bk:min(S, (kt + 1) * bk)])
                prev = max(s[i][:kt * bk]) if kt > 0 else -math.inf
                d = float(np.float32(tmax) - np.float32(prev)) if kt > 0 else math.inf
                worst = max(worst, d)
            margin[qb][kt] = worst
            mask[qb][kt] = worst < ln_lam
    return np.array(mask), np.array(margin, dtype=np.float32)


def pin_mask_matches_bruteforce(orc):
    """The recurrence's skip decisions equal the closed form computed by brute
    force (40 tokens, 4-row x 8-key tiles, several lambda <= 1)."""
    q, k, v = _peaky_head(13, 40, 4)
    scale = 0.5
    ql, kl = q.tolist(), k.tolist()
    seen_skip = seen_keep = 0
    for lam in (1e-4, 1e-2, 0.2, 0.9, 1.0):
        ln = orc.ln_lambda_f32(lam)
        want, want_margin = _bruteforce_mask(ql, kl, scale, float(ln), 4, 8)
        r = orc.skip_head(q, k, v, scale, ln, block_q=4, block_k=8)
        assert (r.skipped == want).all(), (lam, r.skipped.astype(int), want.astype(int))
        assert np.array_equal(r.margin, want_margin)
        cf = orc.prefix_max_margins_head(q, k, scale, block_q=4, block_k=8)
        assert np.array_equal(cf, want_margin)
        seen_skip += want.sum()
        seen_keep += (~want).sum()
    assert seen_skip > 10 and seen_keep > 10


def pin_mask_matches_bruteforce_ragged(orc):
    """Same with a ragged last query block and last key tile (S = 37)."""
    q, k, v = _peaky_head(14, 37, 3)
    scale = 0.6
    for lam in (1e-3, 0.05, 0.5):
        ln = orc.ln_lambda_f32(lam)
        want, _ = _bruteforce_mask(q.tolist(), k.tolist(), scale, float(ln), 5, 7)
        r = orc.skip_head(q, k, v, scale, ln, block_q=5, block_k=7)
        assert (r.skipped == want).all()


def _bruteforce_recurrence_mask(q, k, scale, ln_lam, bq, bk, forced=None):
    """Plain-Python decisions for any lambda: per row a running maximum that
    only kept tiles raise, the float32 margin against it, a tile skipped when
    every valid row's margin is below ln_lam (or as ``forced`` says)."""
    S, D = len(q), len(q[0])
    nqb, nkt = -(-S // bq), -(-S // bk)
    mask = [[False] * nkt for _ in range(nqb)]
    margin = [[0.0] * nkt for _ in range(nqb)]
    for qb in range(nqb):
        rows = range(qb * bq, min(S, (qb + 1) * bq))
        m = {i: -math.inf for i in rows}
        for kt in range(nkt):
            keys = range(kt * bk, min(S, (kt + 1) * bk))
            tmax = {i: max(scale * sum(q[i][t] * k[j][t] for t in range(D)) for j in keys) for i in rows}
            worst = -math.inf
            for i in rows:
                d = math.inf if m[i] == -math.inf else float(np.float32(tmax[i]) - np.float32(m[i]))
                worst = max(worst, d)
            margin[qb][kt] = worst
            skip = bool(forced[qb][kt]) if forced is not None else worst < ln_lam
            mask[qb][kt] = skip
            if not skip:
                for i in rows:
                    m[i] = max(m[i], tmax[i])
    return np.array(mask), np.array(margin, dtype=np.float32)


def pin_row_maxima_mask_bruteforce(orc):
    """tile_row_maxima_head + skip_mask_from_row_maxima (the decisions of a
    whole head from per-row tile maxima) equal plain-Python brute force for
    lambda below and above 1 (above 1 a skipped tile may hold a row's new
    maximum, which the running maximum then never sees), with a ragged last
    query block and key tile, and with a forced mask; and they equal
    skip_head's decisions and margins on a larger head."""
    q, k, v = _peaky_head(16, 43, 4)
    scale = 0.55
    ql, kl = q.tolist(), k.tolist()
    tm = orc.tile_row_maxima_head(q, k, scale, block_k=6, chunk=7)
    assert tm.dtype == np.float32 and tm.shape == (43, 8)
    for i in (0, 20, 42):
        for kt in (0, 3, 7):
            s = [scale * sum(ql[i][t] * kl[j][t] for t in range(4)) for j in range(6 * kt, min(43, 6 * kt + 6))]
            assert tm[i, kt] == np.float32(max(s))
    above = 0
    for lam in (1e-3, 0.2, 1.0, 2.5, 20.0):
        ln = orc.ln_lambda_f32(lam)
        want, want_margin = _bruteforce_recurrence_mask(ql, kl, scale, float(ln), 5, 6)
        got, got_margin = orc.skip_mask_from_row_maxima(tm, ln, block_q=5)
        assert np.array_equal(got, want), (lam, got.astype(int), want.astype(int))
        assert np.array_equal(got_margin, want_margin), lam
        if lam > 1:
            above += int((want & (want_margin > 0)).sum())   # skipped although a row's maximum rose
    assert above > 0
    # ln(lambda) equal to a block's margin: the strict test keeps that tile
    _, m0 = _bruteforce_recurrence_mask(ql, kl, scale, float(orc.ln_lambda_f32(0.2)), 5, 6)
    tie = np.float32(np.sort(m0[np.isfinite(m0) & (m0 < 0)])[-1])
    want, _ = _bruteforce_recurrence_mask(ql, kl, scale, float(tie), 5, 6)
    got, got_margin = orc.skip_mask_from_row_maxima(tm, tie, block_q=5)
    assert np.array_equal(got, want) and (~got[got_margin == tie]).all() and (got_margin == tie).any()
    forced = np.random.default_rng(5).random((9, 8)) < 0.5
    want, want_margin = _bruteforce_recurrence_mask(ql, kl, scale, 0.0, 5, 6, forced=forced.tolist())
    got, got_margin = orc.skip_mask_from_row_maxima(tm, None, forced_skip=forced, block_q=5)
    assert np.array_equal(got, forced) and np.array_equal(got_margin, want_margin)
    got, _ = orc.skip_mask_from_row_maxima(tm, None, block_q=5)
    assert not got.any()
    # a larger head against skip_head, two heads stacked on a leading axis
    q2, k2, v2 = _peaky_head(17, 300, 16)
    tms = np.stack([orc.tile_row_maxima_head(q, k, 2.0, block_k=16)
                    for q, k in ((q2, k2), (k2, q2))])
    for lam in (0.05, 3.0):
        ln = orc.ln_lambda_f32(lam)
        got, got_margin = orc.skip_mask_from_row_maxima(tms, ln, block_q=32)
        for h, (qh, kh, vh) in enumerate(((q2, k2, v2), (k2, q2, v2))):
            r = orc.skip_head(qh, kh, vh, 2.0, ln, block_q=32, block_k=16)
            assert np.array_equal(got[h], r.skipped) and np.array_equal(got_margin[h], r.margin)
            assert 0 < r.skipped.sum() < r.skipped.size


def pin_monotone_in_lambda(orc):
    """For lambda <= 1 a larger lambda skips a superset of tiles."""
    q, k, v = _peaky_head(15, 96, 8)
    prev = None
    for lam in (1e-5, 1e-3, 1e-2, 0.1, 0.5, 1.0):
        r = orc.skip_head(q, k, v, 0.4, orc.ln_lambda_f32(lam), block_q=8, block_k=16)
        if prev is not None:
            assert (r.skipped | ~prev).all() and (r.skipped >= prev).all()
        prev = r.skipped


# ---------------------------------------------------- output given the mask
def pin_output_is_masked_softmax(orc):
    """[design] 'Algorithm': a skipped tile's contribution to l and O is left
    out, so the result is softmax attention over the kept tiles' keys only
    (m is just a stabiliser), for any mask, including ones decided under
    lambda > 1 and forced random masks."""
    q, k, v = _peaky_head(16, 70, 6)
    scale = 0.45
    for lam in (1e-3, 0.3, 1.0, 5.0):
        r = orc.skip_head(q, k, v, scale, orc.ln_lambda_f32(lam), block_q=8, block_k=16)
        o, lse = orc.masked_dense_head(q, k, v, scale, r.skipped, block_q=8, block_k=16)
        assert np.abs(r.o.reshape(-1, 6)[:70] - o).max() < 1e-12
        assert np.abs(r.lse.reshape(-1)[:70] - lse).max() < 1e-12
    rng = np.random.default_rng(17)
    forced = rng.random((9, 5)) < 0.5
    forced[:, 2] = False  # keep at least one tile per block
    r = orc.skip_head(q, k, v, scale, None, forced_skip=forced, block_q=8, block_k=16)
    assert (r.skipped == forced).all()
    o, lse = orc.masked_dense_head(q, k, v, scale, forced, block_q=8, block_k=16)
    assert np.abs(r.o.reshape(-1, 6)[:70] - o).max() < 1e-12


def pin_masked_softmax_against_torch(orc):
    """The masked closed form itself against torch SDPA with a boolean mask."""
    q, k, v = _peaky_head(18, 50, 5)
    rng = np.random.default_rng(19)
    skipped = rng.random((7, 4)) < 0.4
    skipped[:, 0] = False
    o, lse = orc.masked_dense_head(q, k, v, 0.5, skipped, block_q=8, block_k=16)
    allowed = ~skipped[np.arange(50)[:, None] // 8, np.arange(50)[None, :] // 16]
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(allowed), scale=0.5).numpy()
    assert np.abs(o - ref).max() < 1e-12


# ---------------------------------------------------------------- invariants
def pin_skipped_weight_bound(orc):
    """[design] 'Algorithm': exp(tile_max - running_max) bounds the softmax
    weight of every key of the tile, so every key of a skipped tile has dense
    weight below lambda."""
    q, k, v = _peaky_head(20, 128, 8, gain=6.0)
    scale = 0.5
    nskip = 0
    for lam in (1e-4, 1e-2, 0.3):
        r = orc.skip_head(q, k, v, scale, orc.ln_lambda_f32(lam), block_q=8, block_k=16)
        nskip += r.skipped.sum()
        s = scale * q @ k.T
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        for qb, kt in zip(*np.nonzero(r.skipped)):
            blk = p[qb * 8:(qb + 1) * 8, kt * 16:(kt + 1) * 16]
            assert blk.max() <= math.exp(float(r.margin[qb, kt])) * (1 + 1e-12)
            assert blk.max() < lam
    assert nskip > 20


def pin_omitted_mass(orc):
    """LSE_skip = LSE_dense + ln(1 - omega) with omega the dense weight on the
    skipped keys, and |O_skip - O_dense| <= 2 omega max|v| per row."""
    q, k, v = _peaky_head(21, 128, 8, gain=4.0)
    scale = 0.5
    r = orc.skip_head(q, k, v, scale, orc.ln_lambda_f32(0.2), block_q=8, block_k=16)
    assert r.skipped.any()
    o_d, lse_d = orc.dense_head(q, k, v, scale)
    om = orc.skipped_mass_head(q, k, scale, r.skipped, block_q=8, block_k=16)
    s = scale * q @ k.T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    key_tile = np.arange(128) // 16
    om_direct = np.array([p[i, r.skipped[i // 8][key_tile]].sum() for i in range(128)])
    assert np.abs(om - om_direct).max() < 1e-12
    lse = r.lse.reshape(-1)
    assert np.abs(np.exp(lse - lse_d) - (1 - om)).max() < 1e-12
    diff = np.abs(r.o.reshape(-1, 8) - o_d).max(1)
    assert (diff <= 2 * om * np.abs(v).max() + 1e-12).all()


def pin_max_weight_is_inverse_l(orc):
    """The largest softmax weight of a row over the keys that were accumulated
    is exp(m - LSE) = 1/l, so it lies in [1/n_kept, 1] with m the largest kept
    score, found here by brute force from the mask."""
    q, k, v = _peaky_head(23, 96, 8, gain=4.0)
    scale = 0.5
    for lam in (0.0, 0.05, 0.3):
        r = orc.skip_head(q, k, v, scale, orc.ln_lambda_f32(lam), block_q=8, block_k=16)
        lse = r.lse.reshape(-1)
        for i in range(96):
            kept = [c for c in range(96) if not r.skipped[i // 8, c // 16]]
            s = [scale * float(np.dot(q[i], k[c])) for c in kept]
            w = math.exp(max(s) - lse[i])
            assert 1.0 / len(kept) - 1e-12 <= w <= 1.0 + 1e-12, (lam, i, w)
            assert abs(w - 1.0 / sum(math.exp(x - max(s)) for x in s)) < 1e-12
        mp = orc.max_prob_head(q, k, scale, r.skipped, r.lse, block_q=8, block_k=16).reshape(-1)
        for i in range(96):
            kept = [c for c in range(96) if not r.skipped[i // 8, c // 16]]
            s = [scale * float(np.dot(q[i], k[c])) for c in kept]
            assert abs(mp[i] - 1.0 / sum(math.exp(x - max(s)) for x in s)) < 1e-12


def pin_planted_dominant_key(orc):
    """A key in tile 0 that beats every other key of every row of a query
    block by more than -ln(lambda) makes every later tile skippable; the
    result is then softmax attention over tile 0 alone (torch SDPA on that
    slice).  Real geometry: 64-row blocks, 128-key tiles, S = 640."""
    rng = np.random.default_rng(22)
    S, D = 640, 128
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = 0.2 * rng.standard_normal((S, D)) + 3.0 * u
    k = 0.2 * rng.standard_normal((S, D))
    k[5] = 40.0 * u
    v = rng.standard_normal((S, D))
    scale = 1 / math.sqrt(D)
    lam = 1e-3
    r = orc.skip_head(q, k, v, scale, orc.ln_lambda_f32(lam))
    assert r.skipped.shape == (10, 5)
    assert not r.skipped[:, 0].any() and r.skipped[:, 1:].all()
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k[:128], v[:128]))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    assert np.abs(r.o.reshape(-1, D) - ref).max() < 1e-12


def pin_strict_tie_keeps_tile(orc):
    """[design] 'Algorithm' uses a strict '<': a tile whose margin equals
    ln(lambda) exactly is kept; one float32 step higher is skipped."""
    S = 256
    q = np.ones((S, 1))
    k = np.full((S, 1), -10.0)
    k[0] = 0.0          # tile 0 max 0 for every row
    k[128:] = -3.0
    k[200] = -2.0       # tile 1 max -2: margin exactly -2
    v = _rand(23, S, 1)
    lam = math.exp(-2.0)
    ln = orc.ln_lambda_f32(lam)
    assert ln == np.float32(-2.0)
    r = orc.skip_head(q, k, v, 1.0, ln)
    assert (r.margin[:, 1] == np.float32(-2.0)).all()
    assert not r.skipped.any()
    r2 = orc.skip_head(q, k, v, 1.0, np.nextafter(np.float32(-2.0), np.float32(0.0)))
    assert r2.skipped[:, 1].all() and not r2.skipped[:, 0].any()


def pin_running_max_before_update(orc):
    """Reading of 'running_max' as the maximum held before the tile: the first
    tile is always absorbed (margin +inf) even for lambda > 1, and with
    lambda = e^2 a later tile that raises every row's maximum by only 0.5 is
    skipped, leaving softmax over tile 0.  (Under the other reading the first
    tile would be dropped and l would stay 0.)"""
    S = 256
    rng = np.random.default_rng(24)
    q = np.ones((S, 1))
    k = -5.0 + rng.random((S, 1))   # tile 0 scores in [-5, -4)
    k[7] = 0.0                      # tile 0 max 0
    k[128:] = -6.0
    k[130] = 0.5                    # tile 1 max 0.5 > running max 0
    v = rng.standard_normal((S, 3))
    lam = math.exp(2.0)
    r = orc.skip_head(q, k, v, 1.0, orc.ln_lambda_f32(lam))
    assert not r.skipped[:, 0].any() and r.skipped[:, 1].all()
    assert np.isinf(r.margin[:, 0]).all()
    s = k[:128, 0]
    p = np.exp(s - s.max())
    want = (p @ v[:128]) / p.sum()
    assert np.abs(r.o.reshape(-1, 3) - want).max() < 1e-12
    assert np.abs(r.lse.reshape(-1) - (s.max() + np.log(p.sum()))).max() < 1e-12


# ------------------------------------------------------ threshold resolution
def pin_threshold_resolution(orc):
    """[design] 'From configuration to the kernel threshold': lambda =
    factor / max_kv_len; the direct control hands the kernel factor =
    threshold * max_kv_len, so lambda equals the threshold at every length;
    the calibrated control gives factor = a * exp(b * s), i.e. ln(factor) is
    affine in s with intercept ln(a) and slope b (checked on the coefficients
    the page prints for the Wan2.2 T2V A14B checkpoint)."""
    for n in (1024, 4096, 32760):
        for t in (0.0, 1e-4, 0.37, 2.5):
            assert orc.resolve_lambda(threshold=t, seqlen=n) == t
            assert abs(orc.resolve_lambda(factor=t * n, seqlen=n) - t) <= 1e-15 * max(t, 1)
    assert orc.resolve_lambda(factor=3.0, seqlen=1024) == 3.0 / 1024
    with open(os.path.join(GOLDEN, "wan22_calibration.json")) as f:
        cal = json.load(f)
    grp = cal["sparse_attention_config"]["config_groups"]["group_0"]
    a = grp["threshold_scale_factor"]["coefficients"]["a"]
    b = grp["threshold_scale_factor"]["coefficients"]["b"]
    n = 32760
    f0 = orc.resolve_lambda(a=a, b=b, target_sparsity=0.0, seqlen=n) * n
    assert abs(f0 - a) < 1e-9 * a
    xs = np.linspace(0.0, 1.0, 11)
    lf = np.array([math.log(orc.resolve_lambda(a=a, b=b, target_sparsity=x, seqlen=n) * n) for x in xs])
    slope = np.diff(lf) / np.diff(xs)
    assert np.abs(slope - b).max() < 1e-9
    for bad in (dict(threshold=-1.0), dict(factor=float("nan"), seqlen=10), dict(threshold=float("inf"))):
        try:
            orc.resolve_lambda(**bad)
        except ValueError:
            pass
        else:
            raise AssertionError(f"accepted {bad}")
    assert orc.ln_lambda_f32(0.0) is None
    assert orc.ln_lambda_f32(1.0) == np.float32(0.0)


# ------------------------------------------------------------------- varlen
def pin_varlen_blocks_are_independent(orc):
    """Packed sequences never see each other's keys: at lambda = 0 the packed
    result equals torch SDPA with a block-diagonal mask; tiles restart at each
    sequence (ragged lengths 70 and 150)."""
    lens = [70, 150]
    T, H, D = sum(lens), 2, 16
    q, k, v = _rand(25, T, H, D), _rand(26, T, H, D), _rand(27, T, H, D)
    cu = [0, 70, 220]
    o, lse, masks, counts = orc.skip_attention_varlen(q, k, v, cu, 0.25, [0.0, 0.0])
    seg = np.repeat(np.arange(2), lens)
    allowed = torch.from_numpy(seg[:, None] == seg[None, :])
    tq, tk, tv = (torch.from_numpy(x.transpose(1, 0, 2)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=0.25)
    assert np.abs(o - ref.numpy().transpose(1, 0, 2)).max() < 1e-12
    assert [m.shape for m in masks] == [(2, 2, 1), (2, 3, 2)]
    assert counts.shape == (2, 5) and counts.sum() == 0


def pin_varlen_uses_own_length(orc):
    """Each packed sequence normalises lambda by its own length: the packed
    run equals separate runs with lambda_b = factor / S_b."""
    lens = [64 * 3, 64 * 5 + 9]
    H, D = 1, 8
    rng = np.random.default_rng(28)
    parts = [_peaky_head(29 + i, n, D, gain=6.0) for i, n in enumerate(lens)]
    q = np.concatenate([p[0] for p in parts])[:, None, :]
    k = np.concatenate([p[1] for p in parts])[:, None, :]
    v = np.concatenate([p[2] for p in parts])[:, None, :]
    cu = [0, lens[0], sum(lens)]
    factor = 0.3 * lens[0]
    lams = [factor / n for n in lens]
    o, lse, masks, counts = orc.skip_attention_varlen(q, k, v, cu, 0.5, lams, block_q=8, block_k=16)
    for i, n in enumerate(lens):
        r = orc.skip_head(parts[i][0], parts[i][1], parts[i][2], 0.5,
                          orc.ln_lambda_f32(factor / n), block_q=8, block_k=16)
        assert (masks[i][0] == r.skipped).all()
        assert np.abs(o[cu[i]:cu[i + 1], 0] - r.o.reshape(-1, D)[:n]).max() < 1e-12
    assert sum(m.sum() for m in masks) > 0
    assert not (masks[0][0] == orc.skip_head(parts[0][0], parts[0][1], parts[0][2], 0.5,
                orc.ln_lambda_f32(factor / sum(lens)), block_q=8, block_k=16).skipped).all()
    del rng


# ------------------------------------------------------- virtual tiles (Triage)
# "Triage: Skip, Skim, or Refine Attention Tiles in Video Diffusion
# Transformers", section 6.1 "Skipping with Virtual Tiles": a skipped tile is
# represented by its mean key, with a log-count correction of its score, and
# its mean value, inside the same softmax as the real keys.
def _random_mask(seed, nqb, nkt, p=0.5):
    m = np.random.default_rng(seed).random((nqb, nkt)) < p
    m[:, 0] = False                      # the first tile is never skipped
    return m


def pin_virtual_tiles_no_skip_is_dense(orc):
    """With no skipped tile there is no virtual key: dense attention."""
    q, k, v = _rand(40, 150, 16), _rand(41, 150, 16), _rand(42, 150, 16)
    o, lse = orc.virtual_tile_head(q, k, v, 0.4, np.zeros((-(-150 // 8), -(-150 // 16)), bool),
                                   block_q=8, block_k=16)
    od, lsed = orc.dense_head(q, k, v, 0.4)
    assert np.abs(o.reshape(-1, 16)[:150] - od).max() < 1e-12
    assert np.abs(lse.reshape(-1)[:150] - lsed).max() < 1e-12


def pin_virtual_tiles_exact_for_constant_tiles(orc):
    """When all keys of every tile are equal, the mean key with the log-count
    correction stands for its tile exactly: n e^(q.k) = sum over the tile of
    e^(q.k), and the mean value times that weight is the tile's value sum.  So
    any mask gives dense attention.  The last tile is ragged (n < block_k)."""
    S, D, bk = 150, 16, 16
    rng = np.random.default_rng(43)
    kt_keys = rng.standard_normal((-(-S // bk), D))
    k = kt_keys[np.arange(S) // bk]
    q, v = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    mask = _random_mask(44, -(-S // 8), -(-S // bk), p=0.6)
    assert mask[:, -1].any()
    o, lse = orc.virtual_tile_head(q, k, v, 0.7, mask, block_q=8, block_k=bk)
    od, lsed = orc.dense_head(q, k, v, 0.7)
    assert np.abs(o.reshape(-1, D)[:S] - od).max() < 1e-12, np.abs(o.reshape(-1, D)[:S] - od).max()
    assert np.abs(lse.reshape(-1)[:S] - lsed).max() < 1e-12


def pin_virtual_tiles_bruteforce(orc):
    """Pure-Python softmax over (real score, value) pairs of kept tiles and
    (mean-key score + ln n_t, mean value) pairs of skipped tiles."""
    S, D, bq, bk, scale = 40, 4, 8, 16, 0.9
    rng = np.random.default_rng(45)
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    mask = _random_mask(46, -(-S // bq), -(-S // bk), p=0.5)
    mask[1, 2] = True
    o, lse = orc.virtual_tile_head(q, k, v, scale, mask, block_q=bq, block_k=bk)
    for i in range(S):
        qb = i // bq
        items = []
        for t in range(-(-S // bk)):
            keys = list(range(t * bk, min(S, (t + 1) * bk)))
            if not mask[qb, t]:
                for c in keys:
                    items.append((scale * sum(q[i, d] * k[c, d] for d in range(D)), [v[c, d] for d in range(D)]))
            else:
                n = len(keys)
                km = [sum(k[c, d] for c in keys) / n for d in range(D)]
                vm = [sum(v[c, d] for c in keys) / n for d in range(D)]
                items.append((scale * sum(q[i, d] * km[d] for d in range(D)) + math.log(n), vm))
        mx = max(s_ for s_, _ in items)
        ws = [math.exp(s_ - mx) for s_, _ in items]
        den = sum(ws)
        for d in range(D):
            ref = sum(w * val[d] for w, (_, val) in zip(ws, items)) / den
            assert abs(o[qb, i % bq, d] - ref) < 1e-12
        assert abs(lse[qb, i % bq] - (mx + math.log(den))) < 1e-12


def pin_virtual_tiles_between_skip_and_dense(orc):
    """n e^(mean of the scores) <= sum of e^(score) (Jensen), so adding the
    virtual keys raises the log-normaliser of the skip-only pass but never
    above that of dense attention: LSE_skip <= LSE_virtual <= LSE_dense."""
    q, k, v = _peaky_head(47, 300, 16, gain=4.0)
    mask = _random_mask(48, -(-300 // 8), -(-300 // 16), p=0.6)
    o, lse = orc.virtual_tile_head(q, k, v, 0.5, mask, block_q=8, block_k=16)
    _, lse_skip = orc.masked_dense_head(q, k, v, 0.5, mask, block_q=8, block_k=16)
    _, lse_dense = orc.dense_head(q, k, v, 0.5)
    lv = lse.reshape(-1)[:300]
    assert (lv >= lse_skip - 1e-12).all() and (lv <= lse_dense + 1e-12).all()
    assert (lv > lse_skip + 1e-9).mean() > 0.5      # the virtual keys do add weight


def pin_lambda_for_skip_fraction_bruteforce(orc):
    """lambda_for_skip_fraction(margins, f) returns the smallest lambda <= 1
    whose mask margin < ln(lambda) (ln taken as the library takes it: the
    float64 log rounded to float32) skips at least a fraction f of the tiles.
    Brute force: every float32 just above a distinct negative margin is a
    candidate ln(lambda) (the mask only changes there); the answer is the
    smallest candidate that reaches f.  Margins include ties, first tiles
    (+inf) and values at and above 0; a fraction that needs lambda > 1 is
    refused."""
    rng = np.random.default_rng(31)
    m = (rng.standard_normal((20, 13)) * 2.0 - 3.0).astype(np.float32)
    m[:, 0] = np.inf                       # first tiles are never skipped
    m[3, 4:9] = m[2, 5]                    # ties
    m[5, 2] = 0.0
    m[6, 3] = np.float32(0.75)
    cands = sorted({float(np.nextafter(x, np.float32(np.inf))) for x in m.reshape(-1)
                    if np.isfinite(x) and x < 0})
    for frac in (0.0, 1e-3, 0.05, 0.1, 0.37, 0.5, 0.75, 0.85):
        lam = orc.lambda_for_skip_fraction(m, frac)
        if frac == 0.0:
            assert lam == 0.0
            continue
        assert 0.0 < lam < 1.0
        ln = orc.ln_lambda_f32(lam)
        got = float((m < ln).mean())
        assert got >= frac, (frac, got)
        best = next(t for t in cands if float((m < np.float32(t)).mean()) >= frac)
        assert float(ln) == best, (frac, float(ln), best)
    reach = float((m < 0).mean())          # the most lambda <= 1 can skip
    for frac in (reach + 0.01, 0.99):
        try:
            orc.lambda_for_skip_fraction(m, frac)
        except ValueError:
            pass
        else:
            raise AssertionError(f"fraction {frac} needs lambda > 1 and was not refused")


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
