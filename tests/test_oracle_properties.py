"""Randomised checks of the oracle (hypothesis, CPU only): the fixed-seed pins
of tests/oracle_pins.py, generalised over small shapes, tile sizes and
thresholds drawn at random.

  * lambda <= 1: the recurrence's mask equals the closed form on the dense
    prefix maximum, computed here by brute force in plain Python;
  * any lambda: the decisions from per-row tile maxima equal skip_head's
    (the whole-mask GPU checks rest on this);
  * lambda = 0 skips nothing and gives dense attention;
  * the output of any mask is softmax attention over the kept keys, and
    exp(LSE_skip - LSE_dense) equals the kept share of the dense weight.
"""
import math

import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def problems(draw):
    S = draw(st.integers(1, 40))
    D = draw(st.integers(1, 6))
    bq = draw(st.integers(1, 8))
    bk = draw(st.integers(1, 8))
    seed = draw(st.integers(0, 2**31 - 1))
    gain = draw(st.sampled_from([0.5, 1.0, 3.0]))
    rng = np.random.default_rng(seed)
    # bf16-representable values, so that every score is exact in float64
    def bf(x):
        return oracle.from_bf16(torch.from_numpy(x.astype(np.float32)).bfloat16())
    q, k, v = (bf(gain * rng.standard_normal((S, D))) for _ in range(3))
    scale = draw(st.sampled_from([0.25, 0.7, 1.0]))
    return q, k, v, scale, bq, bk


def _closed_form(q, k, scale, ln_lam, bq, bk):
    S, D = q.shape
    s = [[scale * sum(q[i, t] * k[j, t] for t in range(D)) for j in range(S)] for i in range(S)]
    nqb, nkt = -(-S // bq), -(-S // bk)
    mask = np.zeros((nqb, nkt), dtype=bool)
    for qb in range(nqb):
        for kt in range(nkt):
            worst = -math.inf
            for i in range(qb * bq, min(S, (qb + 1) * bq)):
                tmax = max(s[i][kt * bk:min(S, (kt + 1) * bk)])
                d = math.inf if kt == 0 else float(np.float32(tmax) - np.float32(max(s[i][:kt * bk])))
                worst = max(worst, d)
            mask[qb, kt] = worst < ln_lam
    return mask


@SETTINGS
@given(problems(), st.floats(1e-4, 1.0))
def test_mask_is_the_prefix_maximum_closed_form(prob, lam):
    q, k, v, scale, bq, bk = prob
    ln = oracle.ln_lambda_f32(lam)
    r = oracle.skip_head(q, k, v, scale, ln, block_q=bq, block_k=bk)
    assert np.array_equal(r.skipped, _closed_form(q, k, scale, float(ln), bq, bk))


@SETTINGS
@given(problems(), st.floats(1e-4, 50.0))
def test_row_maxima_recurrence_equals_skip_head(prob, lam):
    q, k, v, scale, bq, bk = prob
    ln = oracle.ln_lambda_f32(lam)
    r = oracle.skip_head(q, k, v, scale, ln, block_q=bq, block_k=bk)
    tm = oracle.tile_row_maxima_head(q, k, scale, block_k=bk, chunk=7)
    sk, mg = oracle.skip_mask_from_row_maxima(tm, ln, block_q=bq)
    assert np.array_equal(sk, r.skipped) and np.array_equal(mg, r.margin)


@SETTINGS
@given(problems())
def test_zero_threshold_is_dense(prob):
    q, k, v, scale, bq, bk = prob
    r = oracle.skip_head(q, k, v, scale, oracle.ln_lambda_f32(0.0), block_q=bq, block_k=bk)
    o, lse = oracle.dense_head(q, k, v, scale)
    S = q.shape[0]
    assert not r.skipped.any()
    assert np.abs(r.o.reshape(-1, q.shape[1])[:S] - o).max() < 1e-12
    assert np.abs(r.lse.reshape(-1)[:S] - lse).max() < 1e-12


@SETTINGS
@given(problems(), st.floats(1e-3, 20.0))
def test_output_is_softmax_over_kept_keys(prob, lam):
    q, k, v, scale, bq, bk = prob
    S = q.shape[0]
    r = oracle.skip_head(q, k, v, scale, oracle.ln_lambda_f32(lam), block_q=bq, block_k=bk)
    key_tile = np.arange(S) // bk
    _, lse_dense = oracle.dense_head(q, k, v, scale)
    for i in range(S):
        kept = ~r.skipped[i // bq][key_tile]
        s = scale * (k @ q[i])
        w = np.exp(s - s.max())
        want_o = (w[kept] @ v[kept]) / w[kept].sum()
        got_o = r.o[i // bq, i % bq]
        assert np.abs(got_o - want_o).max() < 1e-10
        share = w[kept].sum() / w.sum()
        assert abs(math.exp(r.lse[i // bq, i % bq] - lse_dense[i]) - share) < 1e-10
