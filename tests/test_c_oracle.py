"""Pins of the plain-C oracle (oracle/skip_attention_c.c), and planted mistakes
that each must fail one of them.

The C oracle computes softmax attention in double precision and the tiled
skip-softmax recurrence in single precision.  Its pins are the textbook
routine (torch's float64 SDPA, with and without a boolean mask), brute force
on tiny inputs, the closed forms the recurrence reduces to, and the
invariants the method states ("Skip-Softmax" design document of vLLM-Omni,
section "Algorithm"; "Skip-Softmax" page of the vLLM-Omni documentation,
sections "The online-softmax pass" and "The skip test").  Inputs are rounded
to bf16 first, so that both sides see exactly the same values.

Tolerances: the double-precision part is held to 1e-12.  The single-precision
recurrence is held to 1e-4 on O and LSE: a 128-channel float dot product
carries a relative error near 1e-5 of |q||k|, which the exponential passes on.
Its tile decisions are compared exactly wherever the reference margin lies
more than 1e-4 from ln(lambda).
"""
import math

import numpy as np
import pytest
import torch

from oracle import c_oracle
from oracle.skip_attention import ln_lambda_f32

TOL32 = 1e-4
BAND = 1e-4


def _bf(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def _rand(seed, *shape, gain=1.0):
    return _bf(gain * np.random.default_rng(seed).standard_normal(shape))


def _peaky_head(seed, s, d, gain=3.0):
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((s, d))
    base /= np.linalg.norm(base, axis=1, keepdims=True)
    q = gain * base + 0.3 * rng.standard_normal((s, d))
    k = gain * base + 0.3 * rng.standard_normal((s, d))
    v = rng.standard_normal((s, d))
    return _bf(q), _bf(k), _bf(v)


def _sdpa(q, k, v, scale, allowed=None):
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = None if allowed is None else torch.from_numpy(allowed)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale).numpy()
    s = scale * tq @ tk.transpose(-1, -2)
    if allowed is not None:
        s = s.masked_fill(~mask, -math.inf)
    return o, torch.logsumexp(s, dim=-1).numpy()


def _bruteforce_margins(q, k, scale, bq, bk):
    """Plain-Python margins for lambda <= 1 (closed form of the recurrence):
    per block and tile, the largest over valid rows of
    f32(max score in the tile) - f32(max score over earlier keys)."""
    S, D = len(q), len(q[0])
    s = [[scale * sum(q[i][t] * k[j][t] for t in range(D)) for j in range(S)] for i in range(S)]
    nqb, nkt = -(-S // bq), -(-S // bk)
    out = np.zeros((nqb, nkt), np.float64)
    for qb in range(nqb):
        for kt in range(nkt):
            worst = -math.inf
            for i in range(qb * bq, min(S, (qb + 1) * bq)):
                tmax = max(s[i][kt * bk:min(S, (kt + 1) * bk)])
                if kt == 0:
                    d = math.inf
                else:
                    d = float(np.float32(tmax) - np.float32(max(s[i][:kt * bk])))
                worst = max(worst, d)
            out[qb, kt] = worst
    return out


# ------------------------------------------------------------------ the pins
def pin_dense_matches_torch_sdpa(c):
    q, k, v = _rand(1, 150, 16), _rand(2, 150, 16), _rand(3, 150, 24)
    o, lse = c.dense_head(q, k, v, 0.3)
    ro, rl = _sdpa(q, k, v, 0.3)
    assert np.abs(o - ro).max() < 1e-12
    assert np.abs(lse - rl).max() < 1e-12


def pin_dense_bruteforce(c):
    q, k, v = _rand(4, 5, 3), _rand(5, 5, 3), _rand(6, 5, 3)
    o, lse = c.dense_head(q, k, v, 0.7)
    for i in range(5):
        s = [0.7 * sum(q[i][t] * k[j][t] for t in range(3)) for j in range(5)]
        den = sum(math.exp(x) for x in s)
        for t in range(3):
            assert abs(o[i][t] - sum(math.exp(s[j]) * v[j][t] for j in range(5)) / den) < 1e-12
        assert abs(lse[i] - math.log(den)) < 1e-12


def pin_zero_threshold_is_dense(c):
    """No vote: the recurrence is softmax attention (real 64 x 128 tiles,
    ragged: S = 1000 gives a 40-row last block and a 104-key last tile)."""
    q, k, v = _rand(7, 1000, 128), _rand(8, 1000, 128), _rand(9, 1000, 128)
    scale = 1 / math.sqrt(128)
    r = c.skip_head(q, k, v, scale, None)
    ro, rl = _sdpa(q, k, v, scale)
    assert not r.skipped.any() and r.skipped.shape == (16, 8)
    assert np.abs(r.o.reshape(-1, 128)[:1000] - ro).max() < TOL32
    assert np.abs(r.lse.reshape(-1)[:1000] - rl).max() < TOL32


def pin_mask_matches_bruteforce(c):
    """Tile decisions and margins against the closed form by brute force
    (40 and 37 tokens, small tiles, several lambda <= 1)."""
    seen = [0, 0]
    for seed, S, D, bq, bk, scale in ((13, 40, 4, 4, 8, 0.5), (14, 37, 3, 5, 7, 0.6)):
        q, k, v = _peaky_head(seed, S, D)
        want = _bruteforce_margins(q.tolist(), k.tolist(), scale, bq, bk)
        for lam in (1e-4, 1e-3, 1e-2, 0.05, 0.2, 0.5, 0.9, 1.0):
            ln = ln_lambda_f32(lam)
            r = c.skip_head(q, k, v, scale, ln, block_q=bq, block_k=bk)
            fin = np.isfinite(want)
            assert np.abs(r.margin[fin] - want[fin]).max() < BAND
            assert (np.isinf(r.margin) == ~fin).all()
            clear = np.abs(want - float(ln)) > BAND
            assert (r.skipped[clear] == (want < float(ln))[clear]).all(), lam
            seen[0] += int(r.skipped.sum())
            seen[1] += int((~r.skipped).sum())
    assert seen[0] > 20 and seen[1] > 20


def pin_output_is_masked_softmax(c):
    """A skipped tile's keys are simply left out: for decided and forced
    masks the result is softmax attention over the kept tiles' keys."""
    q, k, v = _peaky_head(16, 70, 6)
    scale = 0.45
    masks = [c.skip_head(q, k, v, scale, ln_lambda_f32(lam), block_q=8, block_k=16).skipped
             for lam in (1e-3, 0.3, 1.0, 5.0)]
    rng = np.random.default_rng(17)
    forced = rng.random((9, 5)) < 0.5
    forced[:, 2] = False
    masks.append(forced)
    for skipped in masks:
        r = c.skip_head(q, k, v, scale, None, forced_skip=skipped, block_q=8, block_k=16)
        assert (r.skipped == skipped).all()
        allowed = ~skipped[np.arange(70)[:, None] // 8, np.arange(70)[None, :] // 16]
        ro, rl = _sdpa(q, k, v, scale, allowed)
        assert np.abs(r.o.reshape(-1, 6)[:70] - ro).max() < TOL32
        assert np.abs(r.lse.reshape(-1)[:70] - rl).max() < TOL32


def pin_skipped_weight_bound(c):
    """Every key of a skipped tile has dense softmax weight below lambda."""
    q, k, v = _peaky_head(20, 128, 8, gain=6.0)
    scale = 0.5
    s = scale * q @ k.T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    nskip = 0
    for lam in (1e-4, 1e-2, 0.3):
        r = c.skip_head(q, k, v, scale, ln_lambda_f32(lam), block_q=8, block_k=16)
        nskip += int(r.skipped.sum())
        for qb, kt in zip(*np.nonzero(r.skipped)):
            assert p[qb * 8:(qb + 1) * 8, kt * 16:(kt + 1) * 16].max() < lam * (1 + 1e-4)
    assert nskip > 20


def pin_omitted_mass(c):
    """exp(LSE_skip - LSE_dense) = 1 - omega, omega the dense weight of the
    skipped keys."""
    q, k, v = _peaky_head(21, 128, 8, gain=4.0)
    scale = 0.5
    r = c.skip_head(q, k, v, scale, ln_lambda_f32(0.2), block_q=8, block_k=16)
    assert r.skipped.any()
    s = scale * q @ k.T
    lse_d = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
    p = np.exp(s - lse_d[:, None])
    om = np.array([p[i, r.skipped[i // 8][np.arange(128) // 16]].sum() for i in range(128)])
    assert np.abs(np.exp(r.lse.reshape(-1).astype(np.float64) - lse_d) - (1 - om)).max() < TOL32


def pin_strict_tie_keeps_tile(c):
    """Strict '<': a margin equal to ln(lambda) keeps the tile; one float step
    above ln(lambda) skips it (scores exact in float)."""
    S = 256
    q = np.ones((S, 1))
    k = np.full((S, 1), -10.0)
    k[0] = 0.0
    k[128:] = -3.0
    k[200] = -2.0
    v = _rand(23, S, 1)
    ln = ln_lambda_f32(math.exp(-2.0))
    assert ln == np.float32(-2.0)
    r = c.skip_head(q, k, v, 1.0, ln)
    assert (r.margin[:, 1] == np.float32(-2.0)).all() and not r.skipped.any()
    r2 = c.skip_head(q, k, v, 1.0, np.nextafter(np.float32(-2.0), np.float32(0.0)))
    assert r2.skipped[:, 1].all() and not r2.skipped[:, 0].any()


def pin_running_max_before_update(c):
    """The first tile is always absorbed, and with lambda = e^2 a later tile
    that raises every row's maximum by only 0.5 is skipped."""
    S = 256
    rng = np.random.default_rng(24)
    q = np.ones((S, 1))
    k = _bf(-5.0 + rng.random((S, 1)))
    k[7] = 0.0
    k[128:] = -6.0
    k[130] = 0.5
    v = _bf(rng.standard_normal((S, 3)))
    r = c.skip_head(q, k, v, 1.0, ln_lambda_f32(math.exp(2.0)))
    assert not r.skipped[:, 0].any() and r.skipped[:, 1].all()
    assert np.isinf(r.margin[:, 0]).all()
    s = k[:128, 0]
    p = np.exp(s - s.max())
    assert np.abs(r.o.reshape(-1, 3) - (p @ v[:128]) / p.sum()).max() < TOL32
    assert np.abs(r.lse.reshape(-1) - (s.max() + np.log(p.sum()))).max() < TOL32


def pin_planted_dominant_key(c):
    """A dominant key in tile 0 makes every later tile skippable: the result
    is softmax attention over tile 0 alone (64-row blocks, 128-key tiles)."""
    rng = np.random.default_rng(22)
    S, D = 640, 128
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = _bf(0.2 * rng.standard_normal((S, D)) + 3.0 * u)
    k = _bf(0.2 * rng.standard_normal((S, D)))
    k[5] = _bf(40.0 * u)
    v = _bf(rng.standard_normal((S, D)))
    scale = 1 / math.sqrt(D)
    r = c.skip_head(q, k, v, scale, ln_lambda_f32(1e-3))
    assert r.skipped.shape == (10, 5)
    assert not r.skipped[:, 0].any() and r.skipped[:, 1:].all()
    ro, _ = _sdpa(q, k[:128], v[:128], scale)
    assert np.abs(r.o.reshape(-1, D) - ro).max() < TOL32


def pin_padding_rows_do_not_vote(c):
    """The 4 valid rows of a ragged last block decide alone: a padding row
    would score 0 against every key and keep every tile."""
    rng = np.random.default_rng(25)
    S, D = 260, 8
    q = _bf(-np.abs(rng.standard_normal((S, D))))
    k = _bf(np.abs(rng.standard_normal((S, D))))
    k[3] = _bf(np.full(D, -6.0))   # one key every row prefers strongly
    v = _bf(rng.standard_normal((S, D)))
    r = c.skip_head(q, k, v, 1.0, ln_lambda_f32(1e-2))
    assert r.skipped.shape == (5, 3)
    assert r.skipped[4, 1:].all()


def pin_mask_only_mode(c):
    """The decisions-only entry (no exponentials, no P.V) against the same
    pins the full recurrence's decisions meet: the closed form by brute force
    (lambda <= 1, ragged), the strict tie, the running maximum before the
    update, padding rows that do not vote, and a three-tile cascade
    (lambda = e^2) in which a skipped tile must not raise m: tile 1 raises
    every row's maximum by 0.5 and is skipped, tile 2 by 2.3 over tile 0 and
    must be kept (1.8 over tile 1).  It also equals the full recurrence's
    decisions and margins on a peaked head at lambda below and above 1."""
    for seed, S, D, bq, bk, scale in ((13, 40, 4, 4, 8, 0.5), (14, 37, 3, 5, 7, 0.6)):
        q, k, v = _peaky_head(seed, S, D)
        want = _bruteforce_margins(q.tolist(), k.tolist(), scale, bq, bk)
        for lam in (1e-3, 0.05, 0.5, 1.0):
            ln = ln_lambda_f32(lam)
            sk, mg = c.skip_mask(q, k, scale, ln, block_q=bq, block_k=bk)
            fin = np.isfinite(want)
            assert np.abs(mg[fin] - want[fin]).max() < BAND and (np.isinf(mg) == ~fin).all()
            clear = np.abs(want - float(ln)) > BAND
            assert (sk[clear] == (want < float(ln))[clear]).all(), lam
            full = c.skip_head(q, k, v, scale, ln, block_q=bq, block_k=bk)
            assert np.array_equal(sk, full.skipped) and np.array_equal(mg, full.margin)
    # strict tie
    S = 256
    q = np.ones((S, 1))
    k = np.full((S, 1), -10.0)
    k[0] = 0.0
    k[128:] = -3.0
    k[200] = -2.0
    sk, mg = c.skip_mask(q, k, 1.0, ln_lambda_f32(math.exp(-2.0)))
    assert (mg[:, 1] == np.float32(-2.0)).all() and not sk.any()
    sk, _ = c.skip_mask(q, k, 1.0, np.nextafter(np.float32(-2.0), np.float32(0.0)))
    assert sk[:, 1].all() and not sk[:, 0].any()
    # cascade: a skipped tile leaves m alone, so a later tile is measured against tile 0
    k = np.full((384, 1), -20.0)
    k[3], k[130], k[260] = 0.0, 0.5, 2.3
    sk, mg = c.skip_mask(np.ones((384, 1)), k, 1.0, ln_lambda_f32(math.exp(2.0)))
    assert np.isinf(mg[:, 0]).all() and not sk[:, 0].any()
    assert sk[:, 1].all() and (mg[:, 1] == np.float32(0.5)).all()
    assert not sk[:, 2].any() and (mg[:, 2] == np.float32(2.3)).all()
    # padding rows do not vote
    rng = np.random.default_rng(25)
    q = _bf(-np.abs(rng.standard_normal((260, 8))))
    k = _bf(np.abs(rng.standard_normal((260, 8))))
    k[3] = _bf(np.full(8, -6.0))
    sk, _ = c.skip_mask(q, k, 1.0, ln_lambda_f32(1e-2))
    assert sk.shape == (5, 3) and sk[4, 1:].all()
    # equal to the full recurrence, lambda below and above 1
    q, k, v = _peaky_head(26, 700, 16, gain=4.0)
    for lam in (1e-3, 0.3, 3.0, 50.0):
        ln = ln_lambda_f32(lam)
        sk, mg = c.skip_mask(q, k, 0.4, ln, block_q=64, block_k=128)
        full = c.skip_head(q, k, v, 0.4, ln, block_q=64, block_k=128)
        assert np.array_equal(sk, full.skipped) and np.array_equal(mg, full.margin), lam


PINS = [pin_dense_matches_torch_sdpa, pin_dense_bruteforce, pin_zero_threshold_is_dense,
        pin_mask_matches_bruteforce, pin_output_is_masked_softmax, pin_skipped_weight_bound,
        pin_omitted_mass, pin_strict_tie_keeps_tile, pin_running_max_before_update,
        pin_planted_dominant_key, pin_padding_rows_do_not_vote, pin_mask_only_mode]


@pytest.fixture(scope="module")
def c():
    return c_oracle.COracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_c_oracle_pin(c, pin):
    pin(c)


MUTANTS = {
    1: "non-strict comparison",
    2: "running max taken after absorbing the tile",
    3: "l and O not rescaled",
    4: "score scale dropped",
    5: "padding rows vote",
    6: "skipped tiles still raise m",
    7: "lse without the running max",
    8: "q and k swapped in the dense scores",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_c_oracle_mutant_fails_a_pin(mutant):
    bad = c_oracle.COracle(mutant)
    failed = []
    for pin in PINS:
        try:
            pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{MUTANTS[mutant]}' passed every pin"


def test_c_oracle_agrees_with_python_oracle():
    """Both oracles on the same bf16 grid-locality inputs (the Wan-like
    generator, 2 heads of 2,000 tokens): tile decisions equal outside the
    band, O and LSE within the single-precision tolerance."""
    import oracle
    from skip_softmax_flashattention_amd import inputs
    w = inputs.grid_small(2, (5, 20, 20), heads=2)
    q, k, v = (oracle.from_bf16(t) for t in (w.q, w.k, w.v))
    c = c_oracle.oracle()
    for lam in (1e-3, 0.05):
        ln = ln_lambda_f32(lam)
        for h in range(q.shape[1]):
            ref = oracle.skip_head(q[0, h], k[0, h], v[0, h], w.scale, ln)
            got = c.skip_head(q[0, h], k[0, h], v[0, h], w.scale, ln)
            clear = np.abs(ref.margin.astype(np.float64) - float(ln)) > 1e-3
            assert (got.skipped[clear] == ref.skipped[clear]).all()
            same = got.skipped == ref.skipped
            assert same.all() or (~same).sum() <= (~clear).sum()
            forced = c.skip_head(q[0, h], k[0, h], v[0, h], w.scale, None, forced_skip=ref.skipped)
            S = q.shape[2]
            assert np.abs(forced.o.reshape(-1, 128)[:S] - ref.o.reshape(-1, 128)[:S]).max() < TOL32
            assert np.abs(forced.lse.reshape(-1)[:S] - ref.lse.reshape(-1)[:S]).max() < TOL32
