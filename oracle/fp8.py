"""FP8 (OCP E4M3) quantisation of the score operands, for the variant whose
score matmul Q K^T runs in 8-bit floating point while P.V stays in 16-bit.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
imports it.  Source: video-attention blog post on Wan 2.2 on A100, sections
"First, the hardware ceiling" and "Where the 1.33x ceiling comes from,
exactly": only the score matmul moves to the low-precision rate; the value
matmul keeps its 16-bit inputs.  The pages fix neither the format's scaling
nor its granularity; the reading taken (one scale per query token, one per
128-key tile of K, each mapping the block's largest magnitude to 448, the
largest finite E4M3 value) is stated with the functions below.

Formats.  OCP FP8 E4M3 ("E4M3FN"): sign, 4 exponent bits (bias 7), 3
mantissa bits; subnormals 2^-6 * m/8; largest finite value 448; the codes
0x7F and 0xFF are NaN and are never produced here.  Rounding is to nearest,
ties to even, applied to a float32 value; the scaling divisions are IEEE
float32 divisions (numpy float32 arithmetic), the precision the kernel takes
these decisions in.
"""
from __future__ import annotations

import dataclasses

import numpy as np

E4M3_MAX = 448.0
BLOCK_K = 128


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64; NaN codes give NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values with |x| <= 448 to the nearest E4M3 code, ties to
    the even code (the one whose mantissa's last bit is 0).

    The magnitude is split as 2^e * (1 + f) for normals (e >= -6) and
    m * 2^-9 for subnormals; the value in units of the spacing of its binade
    (2^(e-3), or 2^-9 below 2^-6) is rounded half-to-even.  A rounding that
    carries into the next binade lands on that binade's first code."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact
    if np.any(np.abs(x) > E4M3_MAX) or np.any(~np.isfinite(x)):
        raise ValueError("values must be finite with |x| <= 448")
    sign = (np.signbit(x)).astype(np.int64) << 7
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                                   # subnormals share the spacing of binade -6
    # correct a possible off-by-one of log2 on exact powers of two
    e = np.where(a >= np.exp2(e + 1), e + 1, e)
    e = np.where((a < np.exp2(e)) & (e > -6), e - 1, e)
    spacing = np.exp2(e - 3.0)
    units = a / spacing                                       # exact: a is float32, spacing a power of two
    r = np.round(units)                                       # numpy rounds half to even
    # r in [8, 16] for normals (16 carries into the next binade), [0, 8] for subnormals
    normal = a >= 2.0 ** -6
    ebits = np.where(normal, e + 7, 0).astype(np.int64)
    mant = r.astype(np.int64)
    # normals: mantissa field = r - 8; a carry (r == 16) is exponent + 1, mantissa 0
    carry = normal & (mant == 16)
    ebits = np.where(carry, ebits + 1, ebits)
    mant = np.where(normal, np.where(carry, 0, mant - 8), mant)
    # subnormals rounding up to 8 units become the first normal code (exponent field 1, mantissa 0)
    sub_up = (~normal) & (mant == 8)
    ebits = np.where(sub_up, 1, ebits)
    mant = np.where(sub_up, 0, mant)
    codes = sign | (ebits << 3) | mant
    return codes.astype(np.uint8)


def _scale_of(amax: np.ndarray) -> np.ndarray:
    """float32 scale amax / 448 (IEEE float32 division); 1 where amax is 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def _quantize_rows(x32: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes of float32 x / scale (IEEE float32 division, clamped to 448)."""
    y = (x32 / scale).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y)


@dataclasses.dataclass
class Fp8Operands:
    q_codes: np.ndarray   # [S, D] uint8
    q_scale: np.ndarray   # [S] float32: scale of each query token
    k_codes: np.ndarray   # [S, D] uint8
    k_scale: np.ndarray   # [nKT] float32: scale of each 128-key tile
    q: np.ndarray         # [S, D] float64 dequantised: decode(q_codes) * q_scale
    k: np.ndarray         # [S, D] float64 dequantised: decode(k_codes) * k_scale of the key's tile


def quantize_head(q: np.ndarray, k: np.ndarray, block_k: int = BLOCK_K) -> Fp8Operands:
    """Quantise one head's Q and K (float64 arrays holding bf16 values, [S, D]).

    Reading of the pages: Q has one scale per token, q_scale_i =
    max_d |q_id| / 448; K has one scale per tile of block_k keys,
    k_scale_t = max over the tile's keys and channels of |k| / 448.  Each
    element is divided by its scale in float32, clamped to +-448 and rounded
    to the nearest E4M3 value.  The scores of the variant are
    scale * (q_scale_i decode(q_i)) . (k_scale_t decode(k_c)).
    """
    S, D = q.shape
    q32, k32 = q.astype(np.float32), k.astype(np.float32)
    qs = _scale_of(np.abs(q32).max(axis=1))
    qc = _quantize_rows(q32, qs[:, None])
    nkt = -(-S // block_k)
    ks = np.empty(nkt, dtype=np.float32)
    kc = np.empty((S, D), dtype=np.uint8)
    for t in range(nkt):
        r0, r1 = t * block_k, min(S, (t + 1) * block_k)
        ks[t] = _scale_of(np.abs(k32[r0:r1]).max())
        kc[r0:r1] = _quantize_rows(k32[r0:r1], ks[t])
    key_tile = np.arange(S) // block_k
    return Fp8Operands(q_codes=qc, q_scale=qs, k_codes=kc, k_scale=ks,
                       q=e4m3_decode(qc) * qs.astype(np.float64)[:, None],
                       k=e4m3_decode(kc) * ks.astype(np.float64)[key_tile][:, None])


def score_error_bound(ops: Fp8Operands, scale: float, rows: np.ndarray, eps: float,
                      block_k: int = BLOCK_K) -> np.ndarray:
    """eps * scale * q_scale_i * k_scale_t * sum_d |decode(q_id)| |decode(k_cd)| for the
    given query rows and every key: a bound on how far a dot product summed with
    relative accuracy eps (of the sum of the magnitudes of its terms) can be from
    the exact one.  Returns [len(rows), S] float64."""
    aq = np.abs(e4m3_decode(ops.q_codes[rows]))
    ak = np.abs(e4m3_decode(ops.k_codes))
    key_tile = np.arange(ak.shape[0]) // block_k
    return eps * float(scale) * (aq @ ak.T) * ops.q_scale[rows].astype(np.float64)[:, None] \
        * ops.k_scale[key_tile].astype(np.float64)[None, :]
