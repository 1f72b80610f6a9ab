"""CPU oracle for the Skip-Softmax (BLASST) FlashAttention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code, constant or helper with the HIP library.

Sources (cited by page title and section):
  [design]  "Skip-Softmax" design document of vLLM-Omni (the fork's raw
            markdown), sections "Algorithm" and "From configuration to the
            kernel threshold".
  [docs]    "Skip-Softmax" page of the vLLM-Omni documentation, sections
            "The online-softmax pass", "The skip test", "What this bounds",
            "The threshold".

Precision.  Scores, exponentials and the running sums are float64.  The one
place where floating point decides a discrete outcome, the per-tile skip vote,
is taken in float32 like the kernel: the tile maximum and the running maximum
are rounded to float32, subtracted in float32 and compared with ln(lambda)
rounded to float32.

Inputs are float64 arrays holding exact copies of the bf16 tensors
(``from_bf16``).  Fixed-length tensors are [B, H, S, D].

Every function here is pinned by tests under tests/ (textbook routines,
closed forms, brute force on tiny inputs, invariants the pages state); none
is "parity unpinned" except where a docstring says so.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional, Sequence

import numpy as np

BLOCK_Q = 64    # query rows per tile (the pages leave it open; 64 is the reading taken)
BLOCK_K = 128   # keys per tile ([docs] "The online-softmax pass": tiles of 128 keys)


def from_bf16(t) -> np.ndarray:
    """Exact float64 copy of a bf16 torch tensor (bf16 -> f32 -> f64 is exact)."""
    return t.float().double().cpu().numpy()


# --------------------------------------------------------------------------
# Threshold resolution: [design] "From configuration to the kernel threshold"
# (its table of the two controls) and [docs] "The threshold".
# --------------------------------------------------------------------------
def resolve_lambda(*, factor: Optional[float] = None, seqlen: Optional[int] = None,
                   threshold: Optional[float] = None, a: Optional[float] = None,
                   b: Optional[float] = None, target_sparsity: Optional[float] = None) -> float:
    """Effective threshold lambda, in float64.

    factor + seqlen         : lambda = factor / seqlen (the kernel's own input)
    threshold               : lambda = threshold (the direct control; the factor
                              handed to the kernel is threshold * seqlen, which
                              divides back to threshold)
    a, b, target_sparsity,  : factor = a * exp(b * target_sparsity), then
    seqlen                    lambda = factor / seqlen (the calibrated control)
    """
    if threshold is not None:
        lam = float(threshold)
    elif a is not None:
        lam = float(a) * math.exp(float(b) * float(target_sparsity)) / float(seqlen)
    else:
        lam = float(factor) / float(seqlen)
    if not math.isfinite(lam) or lam < 0.0:
        raise ValueError(f"lambda must be finite and non-negative, got {lam}")
    return lam


def ln_lambda_f32(lam: float) -> Optional[np.float32]:
    """ln(lambda) rounded to float32, or None when lambda == 0 (nothing skipped:
    [design] states that a zero threshold skips no tiles)."""
    if lam == 0.0:
        return None
    return np.float32(math.log(lam))


# --------------------------------------------------------------------------
# Dense softmax attention: the plain definition, float64.
# --------------------------------------------------------------------------
def dense_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
               rows: Optional[np.ndarray] = None, chunk: int = 2048):
    """Softmax attention of one head: O = softmax(scale * q k^T) v and
    LSE = log sum exp(scale * q k^T) per query row (natural log).

    q, k, v: [S, D] float64.  ``rows`` restricts the queries computed.
    Returns (o [R, D], lse [R]).
    """
    if rows is None:
        rows = np.arange(q.shape[0])
    o = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        s = float(scale) * (q[r] @ k.T)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        den = p.sum(axis=1)
        o[c0:c0 + chunk] = (p @ v) / den[:, None]
        lse[c0:c0 + chunk] = mx[:, 0] + np.log(den)
    return o, lse


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """dense_head over every (b, h) of [B, H, S, D] tensors."""
    B, H, S, D = q.shape
    o = np.empty((B, H, S, v.shape[-1]))
    lse = np.empty((B, H, S))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = dense_head(q[b, h], k[b, h], v[b, h], scale)
    return o, lse


# --------------------------------------------------------------------------
# The tiled skip-softmax recurrence: [design] "Algorithm", [docs] "The
# online-softmax pass" and "The skip test".
# --------------------------------------------------------------------------
@dataclasses.dataclass
class HeadResult:
    o: np.ndarray          # [nb, block_q, D] float64 (padding rows included)
    lse: np.ndarray        # [nb, block_q] float64
    skipped: np.ndarray    # [nb, nKT] bool, True = tile skipped
    margin: np.ndarray     # [nb, nKT] float32, max over valid rows of tile_max - running_max
    qblocks: np.ndarray    # [nb] the q-block indices computed


def skip_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              ln_lambda: Optional[np.float32], qblocks: Optional[Iterable[int]] = None,
              forced_skip: Optional[np.ndarray] = None,
              block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> HeadResult:
    """One head of the streaming pass with the per-tile skip test.

    For every block of ``block_q`` query rows, running values m (max score
    so far), l (sum of exp(s - m)) and O (sum of exp(s - m) * v) start at
    -inf, 0, 0.  Key tiles of ``block_k`` keys are visited in ascending key
    order.  For each tile:
      1. scores s = scale * q k^T for the tile (always computed);
      2. tile_max[i] = max over the tile's keys of s[i, :];
      3. the test exp(tile_max[i] - m[i]) < lambda, evaluated as
         tile_max[i] - m[i] < ln(lambda) (the log-space form the design
         page says the kernel uses), with m the running maximum held
         *before* this tile is absorbed; the tile is skipped only when every
         valid row of the block passes (strict '<');
      4. a skipped tile leaves m, l and O untouched (its contribution is
         simply left out);
      5. a kept tile is absorbed exactly: m' = max(m, tile_max),
         l = exp(m - m') l + sum exp(s - m'), O = exp(m - m') O + exp(s - m') v.
    The result is O / l and LSE = m + ln l.

    ``ln_lambda`` None disables the test (lambda = 0).  ``forced_skip`` [nb, nKT]
    replaces the decisions with given ones (used to compare outputs under a
    mask decided elsewhere).  Query rows past S pad the last block and take no
    part in the vote.
    """
    S, D = q.shape
    nqb = -(-S // block_q)
    nkt = -(-S // block_k)
    qblocks = np.arange(nqb) if qblocks is None else np.asarray(list(qblocks), dtype=np.int64)
    nb = len(qblocks)
    rows = qblocks[:, None] * block_q + np.arange(block_q)[None, :]
    valid = rows < S
    qr = np.zeros((nb, block_q, D))
    qr[valid] = q[rows[valid]]

    m = np.full((nb, block_q), -np.inf)
    l = np.zeros((nb, block_q))
    acc = np.zeros((nb, block_q, v.shape[1]))
    skipped = np.zeros((nb, nkt), dtype=bool)
    margin = np.zeros((nb, nkt), dtype=np.float32)

    for kt in range(nkt):
        c0, c1 = kt * block_k, min(S, (kt + 1) * block_k)
        s = float(scale) * (qr @ k[c0:c1].T)                  # [nb, block_q, nk]
        tile_max = s.max(axis=2)                               # [nb, block_q]
        with np.errstate(invalid="ignore"):
            d = tile_max.astype(np.float32) - m.astype(np.float32)   # float32; +inf on the first tile
        d = np.where(valid, d, np.float32(-np.inf))
        margin[:, kt] = d.max(axis=1)
        if forced_skip is not None:
            skip = np.asarray(forced_skip[:, kt], dtype=bool)
        elif ln_lambda is None:
            skip = np.zeros(nb, dtype=bool)
        else:
            skip = margin[:, kt] < np.float32(ln_lambda)
        skipped[:, kt] = skip
        keep = ~skip
        if not keep.any():
            continue
        kb = np.nonzero(keep)[0]
        m_new = np.maximum(m[kb], tile_max[kb])
        alpha = np.exp(m[kb] - m_new)                          # exp(-inf) = 0 on the first kept tile
        p = np.exp(s[kb] - m_new[:, :, None])
        l[kb] = alpha * l[kb] + p.sum(axis=2)
        acc[kb] = alpha[:, :, None] * acc[kb] + p @ v[c0:c1]
        m[kb] = m_new

    with np.errstate(invalid="ignore", divide="ignore"):
        o = acc / l[:, :, None]
        lse = m + np.log(l)
    return HeadResult(o=o, lse=lse, skipped=skipped, margin=margin, qblocks=qblocks)


@dataclasses.dataclass
class SkipResult:
    o: np.ndarray            # [B, H, S, D] float64
    lse: np.ndarray          # [B, H, S] float64
    skipped: np.ndarray      # [B, H, nQB, nKT] bool
    margin: np.ndarray       # [B, H, nQB, nKT] float32
    skip_counts: np.ndarray  # [B, H, nQB] int64: skipped tiles per q-block


def skip_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   ln_lambda: Optional[np.float32], forced_skip: Optional[np.ndarray] = None,
                   block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> SkipResult:
    """skip_head over every (b, h) of [B, H, S, D] tensors."""
    B, H, S, D = q.shape
    nqb, nkt = -(-S // block_q), -(-S // block_k)
    o = np.empty((B, H, S, v.shape[-1]))
    lse = np.empty((B, H, S))
    skipped = np.zeros((B, H, nqb, nkt), dtype=bool)
    margin = np.zeros((B, H, nqb, nkt), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            r = skip_head(q[b, h], k[b, h], v[b, h], scale, ln_lambda,
                          forced_skip=None if forced_skip is None else forced_skip[b, h],
                          block_q=block_q, block_k=block_k)
            o[b, h] = r.o.reshape(-1, v.shape[-1])[:S]
            lse[b, h] = r.lse.reshape(-1)[:S]
            skipped[b, h], margin[b, h] = r.skipped, r.margin
    return SkipResult(o=o, lse=lse, skipped=skipped, margin=margin,
                      skip_counts=skipped.sum(axis=-1))


# --------------------------------------------------------------------------
# Closed forms that follow from the recurrence (used as pins and for
# choosing lambda on large inputs).
# --------------------------------------------------------------------------
def masked_dense_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      skipped: np.ndarray, block_q: int = BLOCK_Q, block_k: int = BLOCK_K):
    """Softmax attention restricted, for each query block, to the keys of its
    kept tiles.  Because m only stabilises the exponentials, the recurrence
    computes exactly this in exact arithmetic for any skip mask.

    skipped: [nQB, nKT] bool.  Returns (o [S, D], lse [S]).
    """
    S = q.shape[0]
    o = np.empty((S, v.shape[1]))
    lse = np.empty(S)
    key_tile = np.arange(S) // block_k
    for qb in range(skipped.shape[0]):
        r0, r1 = qb * block_q, min(S, (qb + 1) * block_q)
        allowed = ~skipped[qb][key_tile]
        s = float(scale) * (q[r0:r1] @ k[allowed].T)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        den = p.sum(axis=1)
        o[r0:r1] = (p @ v[allowed]) / den[:, None]
        lse[r0:r1] = mx[:, 0] + np.log(den)
    return o, lse


def prefix_max_margins_head(q: np.ndarray, k: np.ndarray, scale: float,
                            qblocks: Optional[Iterable[int]] = None,
                            block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> np.ndarray:
    """Per-tile margins with the running maximum replaced by the dense prefix
    maximum: margin[qb, kt] = max over valid rows i of
    f32(max_{c in tile kt} s_ic) - f32(max_{c < block_k * kt} s_ic).

    For lambda <= 1 a skipped tile cannot raise any row's maximum (every row
    has tile_max - m < ln(lambda) <= 0), so the recurrence's running maximum
    before tile kt equals the dense prefix maximum and its mask is exactly
    ``margin < ln(lambda)``.  This gives the whole skip-fraction curve from one
    pass.  Returns [nb, nKT] float32.
    """
    S = q.shape[0]
    nqb, nkt = -(-S // block_q), -(-S // block_k)
    qblocks = np.arange(nqb) if qblocks is None else np.asarray(list(qblocks), dtype=np.int64)
    out = np.empty((len(qblocks), nkt), dtype=np.float32)
    pad = nkt * block_k - S
    for j, qb in enumerate(qblocks):
        r0, r1 = qb * block_q, min(S, (qb + 1) * block_q)
        s = float(scale) * (q[r0:r1] @ k.T)
        if pad:
            s = np.concatenate([s, np.full((s.shape[0], pad), -np.inf)], axis=1)
        tmax = s.reshape(s.shape[0], nkt, block_k).max(axis=2).astype(np.float32)
        prefix = np.concatenate([np.full((s.shape[0], 1), -np.inf, dtype=np.float32),
                                 np.maximum.accumulate(tmax, axis=1)[:, :-1]], axis=1)
        with np.errstate(invalid="ignore"):
            out[j] = (tmax - prefix).max(axis=0)
    return out


def tile_row_maxima_head(q: np.ndarray, k: np.ndarray, scale: float, block_k: int = BLOCK_K,
                         chunk: int = 256) -> np.ndarray:
    """Step 2 of skip_head for every row and tile of a head at once:
    tile_max[i, kt] = f32(max over the keys c of tile kt of scale * q_i . k_c),
    scores in float64, the last tile holding only the keys below S.  Nothing
    here depends on lambda, so one pass serves the decisions of every lambda
    (skip_mask_from_row_maxima).  ``chunk`` rows are scored at a time; it only
    bounds memory.  Returns [S, nKT] float32.
    """
    S = q.shape[0]
    nkt = -(-S // block_k)
    nfull = S // block_k
    kT = np.ascontiguousarray(k.T)
    out = np.empty((S, nkt), dtype=np.float32)
    for r0 in range(0, S, chunk):
        s = float(scale) * (q[r0:r0 + chunk] @ kT)                      # [rows, S]
        out[r0:r0 + chunk, :nfull] = s[:, :nfull * block_k].reshape(s.shape[0], nfull, block_k).max(axis=2)
        if nfull < nkt:
            out[r0:r0 + chunk, nfull] = s[:, nfull * block_k:].max(axis=1)
    return out


def skip_mask_from_row_maxima(tile_max: np.ndarray, ln_lambda: Optional[np.float32],
                              forced_skip: Optional[np.ndarray] = None,
                              block_q: int = BLOCK_Q):
    """Steps 3 and 5 of skip_head, reduced to what decides the mask: each row's
    running maximum m starts at -inf; for each tile in ascending order the
    row's margin is f32(tile_max) - f32(m) in float32 (+inf on the first
    tile), the block's margin is the largest over its valid rows, the tile is
    skipped when that margin is below ln(lambda) in float32, and only a kept
    tile raises m to max(m, tile_max).  The exponentials and sums do not
    enter any decision, so the mask and margins equal skip_head's.

    tile_max: [..., S, nKT] float32 from tile_row_maxima_head (leading axes,
    e.g. heads, are independent problems).  ``forced_skip`` [..., nQB, nKT]
    replaces the decisions (m then follows the given mask), as in skip_head;
    ``ln_lambda`` None skips nothing.  Returns (skipped [..., nQB, nKT] bool,
    margin [..., nQB, nKT] float32).
    """
    tile_max = np.asarray(tile_max, dtype=np.float32)
    lead, (S, nkt) = tile_max.shape[:-2], tile_max.shape[-2:]
    nqb = -(-S // block_q)
    tm = np.full((nkt,) + lead + (nqb * block_q,), -np.inf, dtype=np.float32)   # tile-major
    tm[..., :S] = np.moveaxis(tile_max, -1, 0)
    tm = tm.reshape((nkt,) + lead + (nqb, block_q))
    valid = (np.arange(nqb * block_q) < S).reshape(nqb, block_q)
    m = np.full(lead + (nqb, block_q), -np.inf, dtype=np.float32)
    skipped = np.zeros(lead + (nqb, nkt), dtype=bool)
    margin = np.empty(lead + (nqb, nkt), dtype=np.float32)
    for kt in range(nkt):
        t = tm[kt]
        with np.errstate(invalid="ignore"):
            d = np.where(valid, t - m, np.float32(-np.inf))
        margin[..., kt] = d.max(axis=-1)
        if forced_skip is not None:
            skip = np.asarray(forced_skip[..., kt], dtype=bool)
        elif ln_lambda is None:
            skip = np.zeros(lead + (nqb,), dtype=bool)
        else:
            skip = margin[..., kt] < np.float32(ln_lambda)
        skipped[..., kt] = skip
        m = np.where(skip[..., None], m, np.maximum(m, t))
    return skipped, margin


def skipped_mass_head(q: np.ndarray, k: np.ndarray, scale: float, skipped: np.ndarray,
                      block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> np.ndarray:
    """omega_i: the dense softmax weight that row i puts on keys of its
    block's skipped tiles (float64, [S])."""
    S = q.shape[0]
    key_tile = np.arange(S) // block_k
    out = np.empty(S)
    for qb in range(skipped.shape[0]):
        r0, r1 = qb * block_q, min(S, (qb + 1) * block_q)
        s = float(scale) * (q[r0:r1] @ k.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r1] = p[:, skipped[qb][key_tile]].sum(axis=1)
    return out


def max_prob_head(q: np.ndarray, k: np.ndarray, scale: float, skipped: np.ndarray, lse: np.ndarray,
                  qblocks: Optional[Iterable[int]] = None,
                  block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> np.ndarray:
    """The largest softmax weight of each row over the keys of its block's
    kept tiles: exp(max kept score - LSE_i), which equals 1 / l_i with l_i
    the row sum taken relative to the kept maximum (video-attention blog
    post on Wan 2.2, section "max_prob = 1 / l_i, and why it is free").

    skipped: [nb, nKT] decisions of the listed q-blocks (all by default);
    lse: [nb, block_q] as returned with them.  Returns [nb, block_q]
    (padding rows -inf)."""
    S = q.shape[0]
    qbs = np.arange(-(-S // block_q)) if qblocks is None else np.asarray(list(qblocks))
    key_tile = np.arange(S) // block_k
    out = np.full((len(qbs), block_q), -np.inf)
    for j, qb in enumerate(qbs):
        r0, r1 = int(qb) * block_q, min(S, (int(qb) + 1) * block_q)
        s = float(scale) * (q[r0:r1] @ k.T)
        kept = ~skipped[j][key_tile]
        out[j, : r1 - r0] = np.exp(s[:, kept].max(axis=1) - lse[j, : r1 - r0])
    return out


def lambda_for_skip_fraction(margins: np.ndarray, fraction: float) -> float:
    """Smallest lambda <= 1 whose skip mask, from prefix-maximum margins,
    covers at least ``fraction`` of all tiles; ``margin < ln(lambda)`` skips
    a tile.  Returns 0.0 for fraction 0.  Raises if the fraction needs
    lambda > 1 (where the closed form no longer holds).

    Pinned against brute force over every candidate threshold (the float32
    values just above the margins), ties, first tiles and margins >= 0
    included.  It chooses a workload parameter; it computes no result of the
    method.
    """
    flat = np.sort(margins.reshape(-1).astype(np.float64))
    if fraction <= 0.0:
        return 0.0
    n = flat.size
    need = int(math.ceil(fraction * n))
    if need > n or not np.isfinite(flat[need - 1]) or flat[need - 1] >= 0.0:
        raise ValueError("fraction not reachable with lambda <= 1")
    # skip count(ln_lam) = #{margin < ln_lam}; choose ln_lam just above the need-th margin
    edge = flat[need - 1]
    ln_lam = float(np.nextafter(np.float32(edge), np.float32(np.inf)))
    if ln_lam >= 0.0:
        raise ValueError("fraction not reachable with lambda <= 1")
    return math.exp(ln_lam)


def skip_attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
                          scale: float, lambdas: Sequence[float],
                          block_q: int = BLOCK_Q, block_k: int = BLOCK_K):
    """The recurrence over a packed batch of independent sequences.

    q, k, v: [T, H, D] float64; sequence b spans rows cu_seqlens[b] ..
    cu_seqlens[b+1] and uses its own lambda_b (the threshold is normalised by
    the sequence's own length: [docs] "The threshold").  Tiles never straddle
    two sequences.  Returns (o [T, H, D], lse [H, T], skipped list of
    [H, nQB_b, nKT_b], skip_counts [H, sum_b nQB_b]).
    """
    T, H, D = q.shape
    o = np.empty((T, H, v.shape[-1]))
    lse = np.empty((H, T))
    masks, counts = [], []
    for bi in range(len(cu_seqlens) - 1):
        r0, r1 = int(cu_seqlens[bi]), int(cu_seqlens[bi + 1])
        qs = q[r0:r1].transpose(1, 0, 2)[None]
        ks = k[r0:r1].transpose(1, 0, 2)[None]
        vs = v[r0:r1].transpose(1, 0, 2)[None]
        r = skip_attention(qs, ks, vs, scale, ln_lambda_f32(lambdas[bi]),
                           block_q=block_q, block_k=block_k)
        o[r0:r1] = r.o[0].transpose(1, 0, 2)
        lse[:, r0:r1] = r.lse[0]
        masks.append(r.skipped[0])
        counts.append(r.skip_counts[0])
    return o, lse, masks, np.concatenate(counts, axis=1)


# --------------------------------------------------------------------------
# Virtual tiles for skipped tiles: "Triage: Skip, Skim, or Refine Attention
# Tiles in Video Diffusion Transformers", section 6.1 "Skipping with Virtual
# Tiles".  A skipped tile is replaced by one virtual key, the mean of its
# keys, whose score carries the log of the number of keys it stands for, and
# one virtual value, the mean of its values; the virtual keys join the same
# softmax as the real keys of the kept tiles.  Reading taken here: the
# clusters are the key tiles themselves, and the virtual keys do not enter
# the running maximum of the skip test, so the skip mask is that of the
# plain method and the virtual keys change only l, O and LSE.
# --------------------------------------------------------------------------
def virtual_tile_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      skipped: np.ndarray, qblocks: Optional[Iterable[int]] = None,
                      block_q: int = BLOCK_Q, block_k: int = BLOCK_K):
    """Softmax attention of each query block over the keys of its kept tiles
    plus one virtual key per skipped tile t: key mean(k over t), score
    scale * q . mean(k over t) + ln(n_t), value mean(v over t), with n_t the
    number of keys of t (fewer than block_k for a ragged last tile).

    q, k, v: [S, D] float64; skipped: [nb, nKT] decisions of the listed
    q-blocks (all by default).  Returns (o [nb, block_q, D], lse [nb, block_q]);
    padding rows are NaN.
    """
    S, D = q.shape
    nkt = -(-S // block_k)
    qbs = np.arange(-(-S // block_q)) if qblocks is None else np.asarray(list(qblocks), dtype=np.int64)
    counts = np.array([min(S, (t + 1) * block_k) - t * block_k for t in range(nkt)], dtype=np.float64)
    kmean = np.stack([k[t * block_k:min(S, (t + 1) * block_k)].mean(axis=0) for t in range(nkt)])
    vmean = np.stack([v[t * block_k:min(S, (t + 1) * block_k)].mean(axis=0) for t in range(nkt)])
    key_tile = np.arange(S) // block_k
    o = np.full((len(qbs), block_q, v.shape[1]), np.nan)
    lse = np.full((len(qbs), block_q), np.nan)
    for j, qb in enumerate(qbs):
        r0, r1 = int(qb) * block_q, min(S, (int(qb) + 1) * block_q)
        sk = np.asarray(skipped[j], dtype=bool)
        kept = ~sk[key_tile]
        s_real = float(scale) * (q[r0:r1] @ k[kept].T)
        s_virt = float(scale) * (q[r0:r1] @ kmean[sk].T) + np.log(counts[sk])[None, :]
        s = np.concatenate([s_real, s_virt], axis=1)
        vals = np.concatenate([v[kept], vmean[sk]], axis=0)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        den = p.sum(axis=1)
        o[j, : r1 - r0] = (p @ vals) / den[:, None]
        lse[j, : r1 - r0] = mx[:, 0] + np.log(den)
    return o, lse
