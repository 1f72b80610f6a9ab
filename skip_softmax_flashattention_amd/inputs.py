"""Seeded synthetic inputs for the Skip-Softmax attention forward.

This module only draws and lays out input tensors; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can be fed from
it without sharing any of the method's code.

Every workload is a bf16 [B, H, S, D] tensor triple (q, k, v) built in float32
and rounded to bf16 with round-to-nearest-even.  Random draws use
``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal(dtype=float32)``,
in the fixed order: q noise, k noise, v, then any sink indices.

The workloads stand in for the attention the pages measure: video-DiT self
attention over a latent grid (Wan 2.2 at 32,760 tokens, where attention takes
most of each denoising step: "video-attention" blog on Wan 2.2 on A100,
opening section) and long video sequences.  No model activations are used; the grid-local positional
embedding gives scores that peak near each token's own grid position, which is
the structure that lets skip-softmax drop tiles.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

HEAD_DIM = 128
SCALE = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))


@dataclasses.dataclass
class Workload:
    """One synthetic attention problem.

    q, k, v: bf16 CPU tensors [B, H, S, D] (fixed length) or, for a packed
    variable-length batch, [T, H, D] with ``cu_seqlens`` [nseq + 1] int32.
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float = SCALE
    cu_seqlens: Optional[torch.Tensor] = None
    seqlens: Optional[List[int]] = None

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens is not None


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def sinusoid_1d(n: int, dim: int) -> np.ndarray:
    """Interleaved sin/cos embedding of positions 0..n-1, frequency 10000^(-2k/dim)."""
    pos = np.arange(n, dtype=np.float64)[:, None]
    k = np.arange(dim // 2, dtype=np.float64)[None, :]
    ang = pos * np.power(10000.0, -2.0 * k / dim)
    out = np.empty((n, dim), dtype=np.float64)
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang)
    return out


def grid_embedding(t: int, h: int, w: int, dim: int = HEAD_DIM) -> np.ndarray:
    """3-D sinusoidal embedding of a T x Hh x W latent grid in raster order.

    Channels [0, 44) encode the frame index, [44, 86) the row, [86, 128) the
    column; each block is a 1-D interleaved sin/cos embedding with entries in
    [-1, 1] (no normalisation, so every row has squared norm dim / 2).
    """
    assert dim == 128
    dt, dh, dw = 44, 42, 42
    et, eh, ew = sinusoid_1d(t, dt), sinusoid_1d(h, dh), sinusoid_1d(w, dw)
    ti, hi, wi = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    ti, hi, wi = ti.reshape(-1), hi.reshape(-1), wi.reshape(-1)
    return np.concatenate([et[ti], eh[hi], ew[wi]], axis=1)


def _grid_qkv(rng, grid, heads, sink_frac=0.0, batch=1):
    t, h, w = grid
    s = t * h * w
    pe = grid_embedding(t, h, w).astype(np.float32)
    shape = (batch, heads, s, HEAD_DIM)
    nq = rng.standard_normal(shape, dtype=np.float32)
    nk = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    q = 3.0 * pe + 0.7 * nq
    k = 3.0 * pe + 0.7 * nk
    if sink_frac > 0.0:
        nsink = int(round(sink_frac * s))
        idx = rng.choice(s, nsink, replace=False)
        k[:, :, idx, :] *= 4.0
    return q, k, v


def tiny(seed: int = 0) -> Workload:
    """B=1, H=2, S=1024: i.i.d. N(0,1) q, k, v with q and k doubled."""
    rng = np.random.default_rng(seed)
    shape = (1, 2, 1024, HEAD_DIM)
    q = 2.0 * rng.standard_normal(shape, dtype=np.float32)
    k = 2.0 * rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return Workload("tiny", _to_bf16(q), _to_bf16(k), _to_bf16(v))


def mid(seed: int = 1) -> Workload:
    """B=2, H=8, S=4096 on a 1-D sequence; k is the same tensor as q.

    q = 4 * P / |P| + 0.5 * N(0,1), P the 1-D sinusoidal embedding of the
    token index (unit norm after division), so scores peak on the diagonal.
    """
    rng = np.random.default_rng(seed)
    b, h, s = 2, 8, 4096
    pe = sinusoid_1d(s, HEAD_DIM)
    pe = (4.0 * pe / np.linalg.norm(pe, axis=1, keepdims=True)).astype(np.float32)
    nq = rng.standard_normal((b, h, s, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((b, h, s, HEAD_DIM), dtype=np.float32)
    q = pe + 0.5 * nq
    qb = _to_bf16(q)
    return Workload("mid", qb, qb.clone(), _to_bf16(v))


def wan(seed: int = 2, heads: int = 40) -> Workload:
    """Wan-like video self-attention: 21 x 30 x 52 grid (S = 32760), H = 40."""
    q, k, v = _grid_qkv(np.random.default_rng(seed), (21, 30, 52), heads)
    return Workload("wan", _to_bf16(q), _to_bf16(k), _to_bf16(v))


def long_seq(seed: int = 3, heads: int = 24) -> Workload:
    """Long sequence: 24 x 32 x 48 grid (S = 36864), H = 24, 2% sink keys x4."""
    q, k, v = _grid_qkv(np.random.default_rng(seed), (24, 32, 48), heads, sink_frac=0.02)
    return Workload("long", _to_bf16(q), _to_bf16(k), _to_bf16(v))


VARLEN_GRIDS = ((4, 32, 32), (16, 32, 32), (21, 30, 52))


def varlen(seed: int = 4, heads: int = 16, grids: Sequence = VARLEN_GRIDS) -> Workload:
    """Packed batch of grid-local sequences (S = 4096, 16384, 32760), H = 16.

    Sequences are drawn one after another from one generator; the result is
    packed as [T, H, D] with cu_seqlens = [0, S0, S0+S1, ...].
    """
    rng = np.random.default_rng(seed)
    qs, ks, vs, lens = [], [], [], []
    for g in grids:
        q, k, v = _grid_qkv(rng, g, heads)
        # [1, H, S, D] -> [S, H, D]
        qs.append(q[0].transpose(1, 0, 2))
        ks.append(k[0].transpose(1, 0, 2))
        vs.append(v[0].transpose(1, 0, 2))
        lens.append(q.shape[2])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return Workload(
        "varlen",
        _to_bf16(np.concatenate(qs, 0)),
        _to_bf16(np.concatenate(ks, 0)),
        _to_bf16(np.concatenate(vs, 0)),
        cu_seqlens=torch.from_numpy(cu),
        seqlens=lens,
    )


def random_qkv(seed: int, b: int, h: int, s: int, d: int = HEAD_DIM, qk_gain: float = 1.0) -> Workload:
    """Generic i.i.d. normal problem for edge-case tests (ragged S, tiny S)."""
    rng = np.random.default_rng(seed)
    shape = (b, h, s, d)
    q = qk_gain * rng.standard_normal(shape, dtype=np.float32)
    k = qk_gain * rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return Workload(f"rand{b}x{h}x{s}x{d}", _to_bf16(q), _to_bf16(k), _to_bf16(v), scale=float(np.float32(1.0 / math.sqrt(d))))


def grid_small(seed: int, grid, heads: int = 2, sink_frac: float = 0.0) -> Workload:
    """Small grid-local problem with the Wan-like generator (for fast parity cases)."""
    q, k, v = _grid_qkv(np.random.default_rng(seed), grid, heads, sink_frac=sink_frac)
    return Workload(f"grid{grid}", _to_bf16(q), _to_bf16(k), _to_bf16(v))


def unpack_varlen(x: torch.Tensor, cu_seqlens) -> List[torch.Tensor]:
    """Split a packed [T, H, D] tensor into per-sequence [1, H, S_b, D] views."""
    cu = [int(c) for c in cu_seqlens]
    return [x[cu[i]:cu[i + 1]].permute(1, 0, 2).unsqueeze(0).contiguous() for i in range(len(cu) - 1)]
