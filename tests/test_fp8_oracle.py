"""Pins for oracle/fp8.py (E4M3 rounding and the score-operand scaling), and
planted mistakes that each must fail one of them.

What pins it (nothing here comes from the oracle itself):
  * torch's float8_e4m3fn conversion (a library routine, round to nearest
    even) on random values, on exact midpoints between neighbouring codes
    and on the subnormal range;
  * brute force: the nearest of all 254 finite code values, ties to the code
    with an even mantissa;
  * every finite code round-trips;
  * the scaling: each token's (and each key tile's) largest magnitude maps
    to 448 exactly, and every element moves by at most half a unit in the
    last place of its binade (2^-4 relative, or 2^-10 of the scale in the
    subnormal range);
  * the score error bound: with eps set to the classical bound for float32
    summation of 128 exact products, it dominates the error of every
    summation order tried, and is not loose by more than a factor 100.
"""
import os
import types

import numpy as np
import pytest
import torch

from oracle import fp8

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_encode_matches_torch(m):
    rng = np.random.default_rng(0)
    x = np.clip(rng.standard_normal(100000) * 80, -448, 448).astype(np.float32)
    vals = np.sort(np.unique(m.e4m3_decode(FINITE)))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)          # exact ties
    sub = (rng.uniform(-2 ** -6, 2 ** -6, 20000)).astype(np.float32)
    for arr in (x, mids, sub):
        assert (m.e4m3_encode(arr) == _torch_codes(arr)).all()


def pin_encode_bruteforce(m):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.05, 0.05, 3000)]).astype(np.float32)
    vals = m.e4m3_decode(FINITE)
    codes = m.e4m3_encode(x)
    got = m.e4m3_decode(codes)
    for xi, gi in zip(x.astype(np.float64), got):
        d = np.abs(vals - xi)
        best = d.min()
        cand = FINITE[d == best]
        if len(cand) > 1:                              # a tie: the even mantissa wins
            cand = cand[(cand & 1) == 0]
        assert np.isclose(m.e4m3_decode(cand[:1])[0], gi, rtol=0, atol=0) or (gi == 0 and xi == 0)


def pin_all_codes_round_trip(m):
    vals = m.e4m3_decode(FINITE).astype(np.float32)
    assert (m.e4m3_encode(vals) == FINITE).all()
    assert m.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert m.e4m3_decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9


def pin_scales_map_amax_to_448(m):
    rng = np.random.default_rng(2)
    S, D = 300, 128
    q = (rng.standard_normal((S, D)) * rng.uniform(0.01, 30, (S, 1))).astype(np.float32).astype(np.float64)
    k = (rng.standard_normal((S, D)) * 3).astype(np.float32).astype(np.float64)
    q[7] = 0.0
    r = m.quantize_head(q, k)
    dq = m.e4m3_decode(r.q_codes)
    amax = np.abs(dq).max(axis=1)
    assert (amax[np.arange(S) != 7] == 448.0).all() and amax[7] == 0 and r.q_scale[7] == 1.0
    assert r.k_scale.shape == (3,)
    for t in range(3):
        blk = m.e4m3_decode(r.k_codes[128 * t:128 * (t + 1)])
        assert np.abs(blk).max() == 448.0
        assert r.k_scale[t] == np.float32(np.float32(np.abs(k[128 * t:128 * (t + 1)]).max()) / np.float32(448.0))
    # every element within half a unit of its binade
    for x, deq, sc in ((q, r.q, r.q_scale[:, None].astype(np.float64)),
                       (k, r.k, r.k_scale[np.arange(S) // 128][:, None].astype(np.float64))):
        bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc) * (1 + 1e-6)
        assert (np.abs(deq - x) <= bound).all()


def _fp32_sums(prod):
    """Float32 sums of the rows of prod [n_rows, n] (exact float32 values) in
    several orders: sequential, reversed, pairwise, and blocked by 16, 32
    and 64 (each block summed in order, then the block sums in order)."""
    p32 = prod.astype(np.float32)

    def seq(a):
        acc = np.zeros(a.shape[0], np.float32)
        for j in range(a.shape[1]):
            acc = (acc + a[:, j]).astype(np.float32)
        return acc

    def pairwise(a):
        while a.shape[1] > 1:
            if a.shape[1] % 2:
                a = np.concatenate([a, np.zeros((a.shape[0], 1), np.float32)], axis=1)
            a = (a[:, 0::2] + a[:, 1::2]).astype(np.float32)
        return a[:, 0]

    def blocked(a, bs):
        parts = np.stack([seq(a[:, j:j + bs]) for j in range(0, a.shape[1], bs)], axis=1)
        return seq(parts)

    return [seq(p32), seq(p32[:, ::-1]), pairwise(p32), blocked(p32, 16), blocked(p32, 32), blocked(p32, 64)]


def pin_score_error_bound(m):
    """score_error_bound(ops, scale, rows, eps) = eps * scale * q_scale_i *
    k_scale_t * sum_d |q_id| |k_cd| (codes decoded) bounds the error of a score
    whose dot product is summed with relative accuracy eps.  Products of two
    E4M3 values are exact in float32 (4-bit significands), so any float32
    summation order of the D = 128 products is within gamma_127 =
    127u / (1 - 127u) (u = 2^-24) of sum |products| of the exact dot product
    (the classical bound for recursive summation), and the kernel's three
    roundings of the score factor and the product add at most 3u of
    |score| <= the same sum.  So with eps = gamma_131 the bound must dominate
    every order's error (sequential, reversed, pairwise, blocked by 16, 32,
    64); and it must not be loose by a large factor: errors above a
    hundredth of it occur.  Inputs span a wide dynamic range in every row
    and tile (magnitudes over 2^-8 .. 1 times per-row and per-tile gains
    below and above 1), so the quantised codes use most exponents."""
    rng = np.random.default_rng(41)
    S, D = 256, 128
    q = (rng.standard_normal((S, D)) * np.exp2(rng.uniform(-8, 0, (S, D))) * rng.uniform(0.05, 20, (S, 1)))
    k = (rng.standard_normal((S, D)) * np.exp2(rng.uniform(-8, 0, (S, D))))
    k[:128] *= 0.07
    k[128:] *= 13.0
    q = q.astype(np.float32).astype(np.float64)
    k = k.astype(np.float32).astype(np.float64)
    ops = m.quantize_head(q, k)
    scale = float(np.float32(1 / np.sqrt(D)))
    rows = np.arange(0, S, 3)
    aq = m.e4m3_decode(ops.q_codes[rows])
    ak = m.e4m3_decode(ops.k_codes)
    prod = aq[:, None, :] * ak[None, :, :]                        # exact in float64 (and in float32)
    exact_dot = prod.sum(axis=2)                                  # exact: < 53 significant bits
    qs = ops.q_scale[rows].astype(np.float32)
    ks = ops.k_scale[np.arange(S) // 128].astype(np.float32)
    sfac = ((np.float32(scale) * qs)[:, None] * ks[None, :]).astype(np.float32)
    exact = float(scale) * qs.astype(np.float64)[:, None] * ks.astype(np.float64)[None, :] * exact_dot
    u = 2.0 ** -24
    gamma = 131 * u / (1 - 131 * u)
    bound = m.score_error_bound(ops, scale, rows, gamma)
    assert bound.shape == (len(rows), S) and (bound > 0).all()
    worst = 0.0
    for dot32 in _fp32_sums(prod.reshape(-1, D)):
        score = (dot32.reshape(len(rows), S) * sfac).astype(np.float32).astype(np.float64)
        err = np.abs(score - exact)
        assert (err <= bound).all(), float((err / bound).max())
        worst = max(worst, float((err / bound).max()))
    assert worst > 1 / 100, worst


PINS = [pin_encode_matches_torch, pin_encode_bruteforce, pin_all_codes_round_trip, pin_scales_map_amax_to_448,
        pin_score_error_bound]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(fp8)


MUTANTS = [
    ("truncation", "r = np.round(units)", "r = np.floor(units)"),
    ("ties away from zero", "r = np.round(units)", "r = np.floor(units + 0.5)"),
    ("FNUZ maximum 240", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("subnormal spacing of binade -7", "e = np.maximum(e, -6.0)", "e = np.maximum(e, -7.0)"),
    ("one K scale for the whole head", "ks[t] = _scale_of(np.abs(k32[r0:r1]).max())", "ks[t] = _scale_of(np.abs(k32).max())"),
    ("one Q scale for the whole head", "qs = _scale_of(np.abs(q32).max(axis=1))",
     "qs = np.full(S, _scale_of(np.abs(q32).max()), dtype=np.float32)"),
    ("scale multiplied instead of divided", "y = (x32 / scale).astype(np.float32)", "y = (x32 * scale).astype(np.float32)"),
    ("error bound on the signed dot product", "aq = np.abs(e4m3_decode(ops.q_codes[rows]))",
     "aq = e4m3_decode(ops.q_codes[rows])"),
    ("error bound without the q scale", "* ops.q_scale[rows].astype(np.float64)[:, None] \\",
     "* 1.0 \\"),
    ("error bound without the k scale", "* ops.k_scale[key_tile].astype(np.float64)[None, :]",
     "* 1.0"),
    ("error bound on the tile of the wrong key", "key_tile = np.arange(ak.shape[0]) // block_k",
     "key_tile = np.arange(ak.shape[0]) % (ak.shape[0] // block_k)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[x[0] for x in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant '{name}' passed every pin"
