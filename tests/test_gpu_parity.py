"""HIP library against the CPU oracle on seeded inputs (parity proper).

Sizes here let the oracle finish in seconds while still spanning several
64 x 128 tiles and ragged tails; the full-size workloads are in
test_gpu_full.py.  Each case runs the product entry point twice
(determinism), the debug entry point (tile mask), and compares with the
oracle as tests/parity.py describes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from skip_softmax_flashattention_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    return m


def _run(ssa, w, name, **kw):
    print(f"[case] {name} shape={tuple(w.q.shape)} {kw}", flush=True)
    rep = parity.check_fixed(ssa, w, **kw)
    print(f"[case] {name}: {rep}", flush=True)
    parity.assert_bar(rep)
    return rep


# ---- Against the single-precision C oracle ---------------------------------
# The same bar, with the reference recurrence run in float32 by the plain-C
# oracle (oracle/skip_attention_c.c) instead of the float64 Python one.
@pytest.mark.parametrize("factor", [0.0, 0.5, 4.0, 20480.0])
def test_tiny_vs_fp32_oracle(ssa, factor):
    from oracle import c_oracle
    _run(ssa, inputs.tiny(), f"tiny fp32-oracle factor={factor}", factor=factor, ref=c_oracle.oracle().skip_head)


@pytest.mark.parametrize("lam", [1e-4, 1e-3, 1e-2, 0.3])
def test_mid_vs_fp32_oracle(ssa, lam):
    """Every head of the Mid workload (B = 2, H = 8)."""
    from oracle import c_oracle
    _run(ssa, inputs.mid(), f"mid fp32-oracle lambda={lam}", threshold=lam, ref=c_oracle.oracle().skip_head)


def test_wan_like_sampled_vs_fp32_oracle(ssa):
    """Full-size Wan-like problem at the 75%-skip lambda: 16 sampled query
    blocks (first, last and ragged included) of two heads."""
    import json
    import os
    from oracle import c_oracle
    w = inputs.wan()
    S = w.q.shape[2]
    with open(os.path.join(os.path.dirname(__file__), "golden", "wan_lambdas.json")) as f:
        lam = json.load(f)["lambda"]["0.75"]
    nqb = -(-S // 64)
    qbs = np.unique(np.concatenate([[0, 1, nqb - 1], np.random.default_rng(5).choice(nqb, 13, replace=False)]))
    _run(ssa, w, "wan-like fp32-oracle sampled", factor=lam * S, heads=[(0, 0), (0, 39)], qblocks=qbs,
         ref=c_oracle.oracle().skip_head)


# ---- Tiny workload: B=1, H=2, S=1024; factor in {0, 0.5, 4.0} ----------------
# With i.i.d. scores every tile's maximum is close to the running maximum:
# factors 0.5 and 4 (lambda = 0.5/1024, 4/1024) keep every tile.  Skipping
# starts near lambda = 5; factor 20480 (lambda = 20, where kept tiles can
# raise the running maximum after skipped ones) skips about a quarter.
@pytest.mark.parametrize("factor", [0.0, 0.5, 4.0, 20480.0])
def test_tiny(ssa, factor):
    w = inputs.tiny()
    rep = _run(ssa, w, "tiny", factor=factor)
    if factor == 0.0:
        assert rep.skipped == 0
    if factor > 1024:
        assert rep.skipped > 0


def test_tiny_dense_matches_dense_oracle(ssa):
    """lambda = 0 is dense attention: compare with the float64 dense oracle too."""
    w = inputs.tiny()
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    o, lse, cnt = ssa.fwd(q, k, v, factor=0.0)
    torch.cuda.synchronize()
    od, lsed = oracle.dense_attention(*(oracle.from_bf16(t) for t in (w.q, w.k, w.v)), w.scale)
    err = np.abs(o.float().cpu().numpy() - od)
    assert err.max() <= parity.O_MAX and err.mean() <= parity.O_MEAN
    assert np.abs(lse.cpu().numpy() - lsed).max() <= parity.LSE_MAX
    assert int(cnt.sum()) == 0


@pytest.mark.parametrize("S", [128, 4999])
def test_dense_instance_equals_general_instance(ssa, S):
    """Without the skip test the product entry launches the kernel instance
    whose copies are scheduled for dense work; the debug entry always runs the
    general instance.  Same arithmetic in the same order: outputs bitwise
    equal, here over 2 x 5 heads, 40 key tiles and a ragged tail (S = 4999),
    and at exactly one tile (S = 128)."""
    w = inputs.random_qkv(61, 2, 5, S)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    print(f"[case] dense instance S={S}", flush=True)
    o, lse, cnt = ssa.fwd(q, k, v, scale=w.scale, factor=0.0)
    od, lsed, cntd, mask, _ = ssa.fwd_debug(q, k, v, scale=w.scale, factor=0.0)
    torch.cuda.synchronize()
    assert torch.equal(o, od) and torch.equal(lse, lsed)
    assert int(cnt.sum()) == 0 and int(cntd.sum()) == 0 and not bool(mask.any())
    # and one sampled head against the float64 dense oracle
    od64, lse64 = oracle.dense_attention(*(oracle.from_bf16(t[1:, 4:]) for t in (w.q, w.k, w.v)), w.scale)
    err = np.abs(o[1:, 4:].float().cpu().numpy() - od64)
    assert err.max() <= parity.O_MAX and err.mean() <= parity.O_MEAN
    assert np.abs(lse[1:, 4:].cpu().numpy() - lse64).max() <= parity.LSE_MAX


# ---- planted dominant key: every tile after the first is skipped -----------------
def _planted(seed=22, S=640, B=1, H=2):
    rng = np.random.default_rng(seed)
    D = 128
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = 0.2 * rng.standard_normal((B, H, S, D)) + 3.0 * u
    k = 0.2 * rng.standard_normal((B, H, S, D))
    k[:, :, 5] = 40.0 * u
    v = rng.standard_normal((B, H, S, D))
    t = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    return inputs.Workload("planted", t(q), t(k), t(v))


def test_planted_all_later_tiles_skipped(ssa):
    w = _planted()
    rep = _run(ssa, w, "planted", threshold=1e-3)
    nqb, nkt = 10, 5
    assert rep.skipped == 2 * nqb * (nkt - 1)
    # the output is softmax attention over tile 0 alone
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    o, _, _ = ssa.fwd(q, k, v, threshold=1e-3)
    qd, kd, vd = (oracle.from_bf16(t[0, 0]) for t in (w.q, w.k, w.v))
    ref, _ = oracle.dense_head(qd, kd[:128], vd[:128], w.scale)
    assert np.abs(o[0, 0].float().cpu().numpy() - ref).max() <= parity.O_MAX


# ---- grid-local inputs with ragged tails and mixed decisions ----------------------
@pytest.mark.parametrize("grid", [(3, 10, 13), (4, 16, 17), (2, 32, 33)])
@pytest.mark.parametrize("lam", [1e-6, 1e-3, 0.05, 0.5])
def test_grid_ragged(ssa, grid, lam):
    w = inputs.grid_small(5, grid, heads=2)
    _run(ssa, w, f"grid{grid}", threshold=lam)


def test_grid_mixed_decisions_exist(ssa):
    """The grid workload really exercises both branches of the vote."""
    w = inputs.grid_small(5, (4, 16, 17), heads=2)
    rep = _run(ssa, w, "grid-mixed", threshold=0.5)
    assert 0.1 < rep.skipped / rep.tiles < 0.9


# ---- edge sizes --------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 511, 513])
def test_edge_lengths(ssa, S):
    w = inputs.random_qkv(100 + S, 2, 3, S, qk_gain=2.0)
    _run(ssa, w, f"edge S={S}", factor=0.3 * S)


def _sweep_case(i):
    """Seeded case i of the shape sweep: a grid-local problem of a random
    ragged size at a threshold from 0.05 to 10 (below and above 1)."""
    rng = np.random.default_rng(1000 + i)
    grid = (int(rng.integers(2, 6)), int(rng.integers(8, 25)), int(rng.integers(8, 41)))
    w = inputs.grid_small(2000 + i, grid, heads=int(rng.integers(1, 4)))
    return w, (0.05, 0.3, 1.0, 2.0, 5.0, 10.0)[i % 6]


@pytest.mark.parametrize("i", range(16))
def test_random_grid_sweep(ssa, i):
    """Sixteen seeded grid-local problems of random ragged sizes (about 300
    to 5,000 tokens, 1 to 3 heads) at thresholds below and above 1."""
    w, lam = _sweep_case(i)
    S = w.q.shape[2]
    rep = _run(ssa, w, f"sweep {i} S={S} lambda={lam:.4g}", threshold=lam)
    assert rep.tiles > 0


def test_many_heads_small(ssa):
    w = inputs.random_qkv(7, 3, 17, 200, qk_gain=2.0)
    _run(ssa, w, "B3H17", factor=0.0)


def test_seqlen_argument_normalises(ssa):
    """factor / seqlen with seqlen != S (the caller's max_kv_len)."""
    w = inputs.grid_small(9, (3, 10, 13), heads=2)
    _run(ssa, w, "seqlen", factor=20.0, seqlen=100)


# ---- the three controls --------------------------------------------------------------
def test_threshold_entry_equals_factor_entry(ssa):
    w = inputs.grid_small(11, (4, 16, 17), heads=2)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    S = q.shape[2]
    a = ssa.fwd(q, k, v, threshold=0.02)
    b = ssa.fwd(q, k, v, factor=0.02 * S)
    torch.cuda.synchronize()
    # equal lambda up to rounding of 0.02 * S / S: same decisions here
    assert torch.equal(a[2], b[2])


def test_calibrated_entry(ssa):
    w = inputs.grid_small(12, (4, 16, 17), heads=2)
    _run(ssa, w, "calibrated", calib=(3.0, 4.4, 0.5))


@pytest.mark.parametrize("scale,factor", [(0.05, 2.0), (0.3, 0.02), (1.0, 1e-3)])
def test_other_scales(ssa, scale, factor):
    """The score scale enters the vote (tile_max = fl(raw * scale)) and the
    exponent: scales other than 1/sqrt(128), from a flat to a steep softmax."""
    w0 = inputs.grid_small(17, (4, 12, 20), heads=2)
    w = inputs.Workload("grid scale", w0.q, w0.k, w0.v, scale=scale)
    S = w.q.shape[2]
    rep = _run(ssa, w, f"scale {scale}", factor=factor * S)
    assert rep.skipped > 0


def test_lambda_above_one(ssa):
    """Thresholds above 1 are accepted; later decisions depend on earlier ones."""
    w = inputs.grid_small(13, (3, 10, 13), heads=2)
    _run(ssa, w, "lambda>1", threshold=3.0)


# ---- Mid workload: B=2, H=8, S=4096, k = q ----------------------------------------------
# At scale 1/sqrt(128) every later tile's maximum of this problem lies within
# about 2.5 of the running maximum, so the thresholds 1e-4 .. 1e-2 keep every
# tile (the mask is still compared, all kept); 0.1 and 0.3 skip some.
@pytest.mark.parametrize("lam", [1e-4, 1e-3, 1e-2, 0.1, 0.3])
def test_mid(ssa, lam):
    w = inputs.mid()
    rep = _run(ssa, w, "mid", threshold=lam)
    if lam >= 0.1:
        assert rep.skipped > 0


# ---- packed variable-length batches ---------------------------------------------------
def _varlen_check(ssa, w, mode_kw, lambdas):
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    cu = w.cu_seqlens.cuda()
    o, lse, cnt = ssa.fwd_varlen(q, k, v, cu, max(w.seqlens), scale=w.scale, **mode_kw)
    o2, lse2, cnt2 = ssa.fwd_varlen(q, k, v, cu, max(w.seqlens), scale=w.scale, **mode_kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(cnt, cnt2)
    o_np, lse_np, cnt_np = o.float().cpu().numpy(), lse.cpu().numpy(), cnt.cpu().numpy()
    qd, kd, vd = (oracle.from_bf16(t) for t in (w.q, w.k, w.v))
    cuh = w.cu_seqlens.tolist()
    reports, off = [], 0
    for bi, n in enumerate(w.seqlens):
        r0, r1 = cuh[bi], cuh[bi + 1]
        ln = oracle.ln_lambda_f32(lambdas[bi])
        nqb = -(-n // 64)
        for h in range(q.shape[1]):
            # The product entry reports counts, not the mask: compare counts with
            # the oracle's own decisions and the output with the oracle forced to
            # those decisions (no tile of these inputs sits inside the band).
            own = oracle.skip_head(qd[r0:r1, h], kd[r0:r1, h], vd[r0:r1, h], w.scale, ln)
            if ln is not None:
                band = np.abs(own.margin.astype(np.float64) - float(ln)) <= parity.MASK_BAND
                assert not band.any(), "a tile sits inside the threshold band; pick another lambda"
            assert (cnt_np[h, off:off + nqb] == own.skipped.sum(1)).all()
            err = np.abs(o_np[r0:r1, h] - own.o.reshape(-1, 128)[:n])
            lerr = np.abs(lse_np[h, r0:r1] - own.lse.reshape(-1)[:n])
            reports.append(parity.Report(own.skipped.size, int(own.skipped.sum()), 0, float(err.max()),
                                         float(err.mean()), float(lerr.max())))
        off += nqb
    rep = parity.merge(reports)
    print(f"[case] varlen {w.seqlens} {mode_kw}: {rep}", flush=True)
    parity.assert_bar(rep)
    return rep


VARLEN_SMALL = ((1, 7, 10), (3, 10, 13), (2, 8, 9), (1, 1, 1))


@pytest.mark.parametrize("factor", [0.0, 0.02, 3.0])
def test_varlen_factor(ssa, factor):
    w = inputs.varlen(seed=21, heads=3, grids=VARLEN_SMALL)
    lams = [oracle.resolve_lambda(factor=factor, seqlen=n) for n in w.seqlens]
    rep = _varlen_check(ssa, w, dict(factor=factor), lams)
    if factor == 0.0:
        assert rep.skipped == 0


def test_varlen_threshold_and_calibrated(ssa):
    w = inputs.varlen(seed=22, heads=2, grids=VARLEN_SMALL)
    lams = [oracle.resolve_lambda(threshold=0.01)] * len(w.seqlens)
    _varlen_check(ssa, w, dict(threshold=0.01), lams)
    a, b, s = 0.5, 4.0, 0.6
    lams = [oracle.resolve_lambda(a=a, b=b, target_sparsity=s, seqlen=n) for n in w.seqlens]
    _varlen_check(ssa, w, dict(calib=(a, b, s)), lams)


def test_varlen_with_empty_sequence(ssa):
    w = inputs.varlen(seed=23, heads=2, grids=((2, 5, 7), (3, 10, 13)))
    # insert an empty sequence in the middle
    cu = w.cu_seqlens.tolist()
    w.cu_seqlens = torch.tensor([cu[0], cu[1], cu[1], cu[2]], dtype=torch.int32)
    w.seqlens = [w.seqlens[0], 0, w.seqlens[1]]
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    o, lse, cnt = ssa.fwd_varlen(q, k, v, w.cu_seqlens.cuda(), max(w.seqlens), factor=0.0)
    torch.cuda.synchronize()
    od, lsed, _, _ = oracle.skip_attention_varlen(*(oracle.from_bf16(t) for t in (w.q, w.k, w.v)),
                                                   w.cu_seqlens.tolist(), w.scale, [0.0, 0.0, 0.0])
    assert np.abs(o.float().cpu().numpy() - od).max() <= parity.O_MAX
    assert np.abs(lse.cpu().numpy() - lsed).max() <= parity.LSE_MAX


@pytest.mark.parametrize("threshold", [0.0, 0.3, 2.0])
def test_varlen_many_sequences_equal_fixed_calls(ssa, threshold):
    """70 packed sequences (more than one 64-sequence step of the workgroup
    map's scan) of lengths 0 .. 600, empty, one-token and tile-edge lengths
    included, with max_seqlen above the longest: each sequence's output,
    LSE and skip counts equal bitwise those of a fixed-length call on that
    sequence alone (the same rows, tiles and arithmetic; threshold mode gives
    both calls the same ln(lambda)).  Checks that the map covers every
    (sequence, head, query group) once and places it right; lambda = 2
    adds the cascade of decisions that kept tiles cause above 1."""
    rng = np.random.default_rng(71)
    lens = [0, 1, 64, 128, 255, 256, 257, 0] + [int(x) for x in rng.integers(0, 601, 62)]
    H, D = 2, 128
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = (torch.from_numpy(g * rng.standard_normal((T, H, D), dtype=np.float32)).to(torch.bfloat16).cuda()
               for g in (2.0, 2.0, 1.0))
    print(f"[case] varlen 70 sequences T={T} threshold={threshold}", flush=True)
    o, lse, cnt = ssa.fwd_varlen(q, k, v, torch.from_numpy(cu).cuda(), max(lens) + 37, threshold=threshold)
    torch.cuda.synchronize()
    qb_off = 0
    for b, n in enumerate(lens):
        nqb = -(-n // 64)
        if n == 0:
            continue
        r0, r1 = int(cu[b]), int(cu[b + 1])
        qs, ks, vs = (t[r0:r1].transpose(0, 1).unsqueeze(0).contiguous() for t in (q, k, v))
        of, lf, cf = ssa.fwd(qs, ks, vs, threshold=threshold)
        torch.cuda.synchronize()
        assert torch.equal(o[r0:r1], of[0].transpose(0, 1)), f"sequence {b} (length {n}): output"
        assert torch.equal(lse[:, r0:r1], lf[0]), f"sequence {b}: lse"
        assert torch.equal(cnt[:, qb_off:qb_off + nqb], cf[0]), f"sequence {b}: skip counts"
        qb_off += nqb
    assert qb_off == cnt.shape[1]
    if threshold > 0:
        assert int(cnt.sum()) > 0


def test_errors_on_gpu(ssa):
    w = inputs.random_qkv(1, 1, 1, 64)
    q = w.q.cuda()
    with pytest.raises(ssa.SsaError) as e:
        ssa.fwd(q, q, q, factor=-1.0)
    assert e.value.code == -3
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssa.SsaError) as e:
        ssa.fwd(x, x, x, factor=1.0)
    assert e.value.code == -2


# ---- largest softmax weight per row (max_prob = exp(m - LSE) = 1 / l) -----------------
@pytest.mark.parametrize("case", ["tiny", "grid", "planted"])
def test_max_prob(ssa, case):
    if case == "tiny":
        w, kw = inputs.tiny(), dict(factor=4.0)
    elif case == "grid":
        w, kw = inputs.grid_small(31, (3, 10, 13), heads=2), dict(threshold=0.05)
    else:
        w, kw = inputs.grid_small(32, (2, 8, 9), heads=2, sink_frac=0.02), dict(threshold=1e-3)
    print(f"[case] max_prob {case} shape={tuple(w.q.shape)} {kw}", flush=True)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    o, lse, cnt, mp = ssa.fwd_max_prob(q, k, v, scale=w.scale, **kw)
    od, ld, cd, mask, _ = ssa.fwd_debug(q, k, v, scale=w.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, od) and torch.equal(lse, ld) and torch.equal(cnt, cd), "max_prob entry changed the outputs"
    mask_np, mp_np = mask.cpu().numpy().astype(bool), mp.cpu().numpy()
    B, H, S, D = w.q.shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            qd, kd, vd = (oracle.from_bf16(t[b, h]) for t in (w.q, w.k, w.v))
            forced = oracle.skip_head(qd, kd, vd, w.scale, None, forced_skip=mask_np[b, h])
            ref = oracle.max_prob_head(qd, kd, w.scale, mask_np[b, h], forced.lse).reshape(-1)[:S]
            got = mp_np[b, h]
            rel = np.abs(got - ref) / ref
            worst = max(worst, float(rel.max()))
            n_kept = (~mask_np[b, h]).sum(axis=1).repeat(64)[:S] * 128
            assert (got <= 1.0).all() and (got >= 1.0 / n_kept * (1 - 1e-3)).all()
    print(f"[case] max_prob {case}: max relative error {worst:.2e}", flush=True)
    assert worst <= 3e-3


def test_vote_give_up_keeps_every_tile(ssa):
    """The bounded wait for the partner wave's half of the vote, driven from
    the host through the debug entry: with the poll limit at 0 every wave
    gives up at once, so every tile is kept (the exact path), every query
    block's count comes out flagged as -1 - 0, the mask shows no skipped
    tile, and O and LSE equal the dense call's bit for bit (the arithmetic of
    a kept tile does not depend on the vote).  The product entry keeps its
    constant bound meanwhile, and restoring the limit restores the debug
    entry's normal result."""
    w = inputs.grid_small(41, (4, 12, 20), heads=2)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    od, lsed, cd = ssa.fwd(q, k, v, scale=w.scale, factor=0.0)
    o1, l1, c1 = ssa.fwd(q, k, v, scale=w.scale, threshold=0.05)
    torch.cuda.synchronize()
    assert int(c1.sum()) > 0 and int(cd.sum()) == 0
    print(f"[case] vote give-up: normal call skips {int(c1.sum())} tiles", flush=True)
    try:
        ssa.set_vote_poll_limit(0)
        om, lm, cm, mask, _ = ssa.fwd_debug(q, k, v, scale=w.scale, threshold=0.05)
        o0, l0, c0 = ssa.fwd(q, k, v, scale=w.scale, threshold=0.05)
        torch.cuda.synchronize()
    finally:
        ssa.set_vote_poll_limit(16384)
    print(f"[case] vote give-up: debug counts {sorted(set(cm.flatten().tolist()))}, mask skipped "
          f"{int(mask.sum())}; product entry skipped {int(c0.sum())}", flush=True)
    assert (cm == -1).all() and int(mask.sum()) == 0
    assert torch.equal(om, od) and torch.equal(lm, lsed)
    assert torch.equal(o0, o1) and torch.equal(l0, l1) and torch.equal(c0, c1)
    o2, l2, c2, m2, _ = ssa.fwd_debug(q, k, v, scale=w.scale, threshold=0.05)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1) and torch.equal(l2, l1) and torch.equal(c2, c1)
    assert int(m2.sum()) == int(c1.sum())
