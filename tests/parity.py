"""Shared parity check between the HIP library and the CPU oracle.

Bar (tolerances for bf16 inputs and outputs):
  * tile mask: identical to the oracle's own decisions for every tile whose
    oracle margin lies more than 1e-3 away from ln(lambda) (inside that band
    the float32 rounding of two different summation orders may flip it);
  * O: against the oracle run with the GPU's mask forced (so a flip inside the
    band cannot leak into the output check), max |dO| <= 2e-2 and
    mean |dO| <= 2e-3;
  * LSE: max |dLSE| <= 1e-3;
  * skip_counts: equal to the row sums of the GPU's mask.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

import oracle

MASK_BAND = 1e-3
O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


@dataclasses.dataclass
class Report:
    tiles: int
    skipped: int
    exempt: int
    o_max: float
    o_mean: float
    lse_max: float

    def __str__(self):
        return (f"skipped {self.skipped}/{self.tiles} ({self.skipped / max(self.tiles, 1):.3f}), "
                f"band-exempt {self.exempt}, max|dO| {self.o_max:.2e}, mean|dO| {self.o_mean:.2e}, "
                f"max|dLSE| {self.lse_max:.2e}")


def compare_head_blocks(qd, kd, vd, scale, ln_lambda, qblocks, gpu_mask, gpu_o, gpu_lse, gpu_counts,
                        ref=None) -> Report:
    """Compare one head's selected q-blocks.  qd/kd/vd: float64 [S, D];
    gpu_mask [nb, nKT] bool; gpu_o [nb*64 rows clipped to S, D]; gpu_lse
    likewise; gpu_counts [nb].  ``ref`` is the oracle's skip_head (the
    float64 Python oracle by default; the single-precision C oracle's
    skip_head takes the same arguments)."""
    S = qd.shape[0]
    ref = oracle.skip_head if ref is None else ref
    own = ref(qd, kd, vd, scale, ln_lambda, qblocks=qblocks)
    if ln_lambda is None:
        band = np.zeros_like(own.skipped)
    else:
        band = np.abs(own.margin.astype(np.float64) - float(ln_lambda)) <= MASK_BAND
    bad = (gpu_mask != own.skipped) & ~band
    assert not bad.any(), f"{int(bad.sum())} tile decisions differ outside the band (first at {np.argwhere(bad)[:3].tolist()})"
    forced = own if np.array_equal(gpu_mask, own.skipped) else ref(
        qd, kd, vd, scale, None, qblocks=qblocks, forced_skip=gpu_mask)
    rows = (np.asarray(qblocks)[:, None] * oracle.BLOCK_Q + np.arange(oracle.BLOCK_Q)[None, :]).reshape(-1)
    valid = rows < S
    o_ref = forced.o.reshape(-1, qd.shape[1])[valid].astype(np.float64)
    lse_ref = forced.lse.reshape(-1)[valid].astype(np.float64)
    err = np.abs(gpu_o - o_ref)
    lerr = np.abs(gpu_lse - lse_ref)
    assert np.isfinite(gpu_o).all() and np.isfinite(gpu_lse).all()
    assert (gpu_counts == gpu_mask.sum(axis=1)).all(), "skip_counts differ from the mask's row sums"
    return Report(tiles=gpu_mask.size, skipped=int(gpu_mask.sum()), exempt=int((band & (gpu_mask != own.skipped)).sum()),
                  o_max=float(err.max()), o_mean=float(err.mean()), lse_max=float(lerr.max()))


def whole_mask_forced(gpu_mask, margins, ln_lambda):
    """Every tile of one or more heads: the GPU's decisions [..., nQB, nKT]
    against the oracle's margins computed along the GPU's own decisions
    (oracle.skip_mask_from_row_maxima with forced_skip = the GPU's mask), so
    a tile inside MASK_BAND that went the other way cannot move the two
    running maxima apart.  Outside the band every decision must be
    margin < ln(lambda).  Returns (tiles compared exactly, tiles inside the
    band that differ)."""
    want = margins < np.float32(ln_lambda)
    band = np.abs(margins.astype(np.float64) - float(ln_lambda)) <= MASK_BAND
    diff = gpu_mask != want
    bad = diff & ~band
    assert not bad.any(), (f"{int(bad.sum())} tile decisions differ outside the band "
                           f"(first at {np.argwhere(bad)[:3].tolist()})")
    return int((~band).sum()), int((diff & band).sum())


def whole_head_mask_recurrence(gpu_mask, skipped, margins, ln_lambda):
    """Every tile of a head, any lambda: the GPU's decisions [nQB, nKT]
    against the recurrence's own (the single-precision C oracle's decisions
    and margins).  Above lambda = 1 a kept tile can raise the running
    maximum, so after a decision that differs inside the band the two sides
    run on different maxima: the rest of that query block is exempt (and
    counted).  Returns (tiles compared exactly, tiles exempt)."""
    band = np.abs(margins.astype(np.float64) - float(ln_lambda)) <= MASK_BAND
    exact = exempt = 0
    for qb in range(gpu_mask.shape[0]):
        diff = np.nonzero(gpu_mask[qb] != skipped[qb])[0]
        stop = gpu_mask.shape[1]
        if diff.size:
            first = int(diff[0])
            assert band[qb, first], f"query block {qb}: tile {first} differs outside the band"
            stop = first
        exact += stop
        exempt += gpu_mask.shape[1] - stop
    return exact, exempt


def merge(reports: Sequence[Report]) -> Report:
    n = sum(r.tiles for r in reports)
    return Report(tiles=n, skipped=sum(r.skipped for r in reports), exempt=sum(r.exempt for r in reports),
                  o_max=max(r.o_max for r in reports),
                  o_mean=float(np.mean([r.o_mean for r in reports])),
                  lse_max=max(r.lse_max for r in reports))


def assert_bar(rep: Report):
    assert rep.o_max <= O_MAX, rep
    assert rep.o_mean <= O_MEAN, rep
    assert rep.lse_max <= LSE_MAX, rep


def check_fixed(ssa, w, *, factor: Optional[float] = None, threshold: Optional[float] = None,
                calib=None, seqlen: Optional[int] = None, heads: Optional[Sequence] = None,
                qblocks: Optional[Sequence[int]] = None, device="cuda", ref=None) -> Report:
    """Run the product entry point and the debug entry point on one fixed-length
    workload and compare with the oracle on the selected (b, h) heads and
    q-blocks (all by default)."""
    q, k, v = (t.to(device) for t in (w.q, w.k, w.v))
    B, H, S, D = q.shape
    n = S if seqlen is None else seqlen
    if threshold is not None:
        lam = oracle.resolve_lambda(threshold=threshold)
    elif calib is not None:
        lam = oracle.resolve_lambda(a=calib[0], b=calib[1], target_sparsity=calib[2], seqlen=n)
    else:
        lam = oracle.resolve_lambda(factor=factor, seqlen=n)
    ln = oracle.ln_lambda_f32(lam)
    kw = dict(scale=w.scale, factor=factor, threshold=threshold, calib=calib, seqlen=seqlen)
    o, lse, cnt = ssa.fwd(q, k, v, **kw)
    o2, lse2, cnt2 = ssa.fwd(q, k, v, **kw)
    od, lsed, cntd, mask, _ = ssa.fwd_debug(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(cnt, cnt2), "not deterministic"
    assert torch.equal(cnt, cntd), "debug and product entry points disagree on skip counts"
    assert torch.equal(o, od) and torch.equal(lse, lsed), "debug and product entry points disagree"
    mask = mask.cpu().numpy().astype(bool)
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    cnt_np = cnt.cpu().numpy()
    nqb = mask.shape[2]
    qbs = np.arange(nqb) if qblocks is None else np.asarray(qblocks)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    reports = []
    for (b, h) in heads:
        qd, kd, vd = (oracle.from_bf16(t[b, h]) for t in (w.q, w.k, w.v))
        rows = (qbs[:, None] * oracle.BLOCK_Q + np.arange(oracle.BLOCK_Q)[None, :]).reshape(-1)
        rows = rows[rows < S]
        reports.append(compare_head_blocks(qd, kd, vd, w.scale, ln, qbs, mask[b, h][qbs], o_np[b, h][rows],
                                           lse_np[b, h][rows], cnt_np[b, h][qbs], ref=ref))
    return merge(reports)
