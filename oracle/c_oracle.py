"""ctypes front end of the plain-C oracle (oracle/skip_attention_c.c).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU baseline use it, and it shares nothing
with the HIP library.

The C file holds the two parts of the oracle in compiled form: softmax
attention in double precision, and the tiled skip-softmax recurrence in
single precision ("Skip-Softmax" design document of vLLM-Omni, section
"Algorithm"; "Skip-Softmax" page of the vLLM-Omni documentation, sections
"The online-softmax pass" and "The skip test").  It takes the same readings
as oracle/skip_attention.py and is pinned by tests/test_c_oracle.py.

The library is built with gcc into oracle/_build on first use (or by
__graft_entry__.build()), and rebuilt when the source is newer.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
import tempfile
from typing import Iterable, Optional

import numpy as np

from .skip_attention import BLOCK_K, BLOCK_Q, ln_lambda_f32  # noqa: F401  (same lambda reading)

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "skip_attention_c.c")
BUILD_DIR = os.path.join(HERE, "_build")
CFLAGS = ["-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99"]


def library_path(mutant: int = 0) -> str:
    return os.path.join(BUILD_DIR, "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so")


def build(mutant: int = 0, force: bool = False) -> str:
    """Compile the C oracle (with planted mistake ``mutant``, 0 = none) unless
    an up-to-date build exists.  Returns the library path."""
    path = library_path(mutant)
    if not force and os.path.exists(path) and os.path.getmtime(path) >= os.path.getmtime(SRC):
        return path
    os.makedirs(BUILD_DIR, exist_ok=True)
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=BUILD_DIR)
    os.close(fd)
    try:
        subprocess.run(["gcc", *CFLAGS, f"-DORACLE_MUTANT={int(mutant)}", "-o", tmp, SRC, "-lm"],
                       check=True, capture_output=True, text=True)
        os.replace(tmp, path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return path


@dataclasses.dataclass
class HeadResult:
    o: np.ndarray          # [nb, block_q, Dv] float32 (padding rows included)
    lse: np.ndarray        # [nb, block_q] float32
    skipped: np.ndarray    # [nb, nKT] bool, True = tile skipped
    margin: np.ndarray     # [nb, nKT] float32, max over valid rows of tile_max - running_max
    qblocks: np.ndarray    # [nb] the q-block indices computed


@dataclasses.dataclass
class SkipResult:
    o: np.ndarray            # [B, H, S, Dv] float32
    lse: np.ndarray          # [B, H, S] float32
    skipped: np.ndarray      # [B, H, nQB, nKT] bool
    margin: np.ndarray       # [B, H, nQB, nKT] float32
    skip_counts: np.ndarray  # [B, H, nQB] int64


_P = ctypes.c_void_p
_I = ctypes.c_int


class COracle:
    """The compiled oracle; ``mutant`` selects a build with a planted mistake
    (tests only)."""

    def __init__(self, mutant: int = 0):
        self.lib = ctypes.CDLL(build(mutant))
        self.lib.oracle_threads.restype = _I
        self.lib.oracle_dense_head.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_double, _P, _P]
        self.lib.oracle_dense_head.restype = _I
        self.lib.oracle_skip_head_f32.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_float, _I, ctypes.c_float, _I, _I,
                                                  _P, _I, _P, _P, _P, _P, _P]
        self.lib.oracle_skip_head_f32.restype = _I
        self.lib.oracle_skip_mask_f32.argtypes = [_P, _P, _I, _I, ctypes.c_float, _I, ctypes.c_float, _I, _I, _P, _I,
                                                  _P, _P]
        self.lib.oracle_skip_mask_f32.restype = _I

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def dense_head(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
        """Softmax attention of one head in double precision: (o [S, Dv], lse [S])."""
        q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
        S, D = q.shape
        Dv = v.shape[1]
        o = np.empty((S, Dv))
        lse = np.empty(S)
        rc = self.lib.oracle_dense_head(q.ctypes.data, k.ctypes.data, v.ctypes.data, S, D, Dv, float(scale),
                                        o.ctypes.data, lse.ctypes.data)
        if rc != 0:
            raise MemoryError("oracle_dense_head: out of memory")
        return o, lse

    def dense_attention(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
        """dense_head over every (b, h) of [B, H, S, D] tensors."""
        B, H, S, _ = q.shape
        o = np.empty((B, H, S, v.shape[-1]))
        lse = np.empty((B, H, S))
        for b in range(B):
            for h in range(H):
                o[b, h], lse[b, h] = self.dense_head(q[b, h], k[b, h], v[b, h], scale)
        return o, lse

    def skip_head(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  ln_lambda: Optional[np.float32], qblocks: Optional[Iterable[int]] = None,
                  forced_skip: Optional[np.ndarray] = None,
                  block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> HeadResult:
        """The tiled recurrence of one head in single precision.  ``ln_lambda``
        None disables the test; ``forced_skip`` [nb, nKT] replaces the
        decisions; ``qblocks`` restricts the query blocks computed."""
        q, k, v = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v))
        S, D = q.shape
        Dv = v.shape[1]
        nqb, nkt = -(-S // block_q), -(-S // block_k)
        qb = np.arange(nqb, dtype=np.int64) if qblocks is None else np.ascontiguousarray(list(qblocks), dtype=np.int64)
        nb = len(qb)
        forced = None if forced_skip is None else np.ascontiguousarray(forced_skip, dtype=np.uint8).reshape(nb, nkt)
        o = np.empty((nb, block_q, Dv), np.float32)
        lse = np.empty((nb, block_q), np.float32)
        skipped = np.empty((nb, nkt), np.uint8)
        margin = np.empty((nb, nkt), np.float32)
        vote = ln_lambda is not None
        rc = self.lib.oracle_skip_head_f32(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, S, D, Dv, float(np.float32(scale)), int(vote),
            float(np.float32(ln_lambda)) if vote else 0.0, block_q, block_k, qb.ctypes.data, nb,
            None if forced is None else forced.ctypes.data, o.ctypes.data, lse.ctypes.data, skipped.ctypes.data,
            margin.ctypes.data)
        if rc != 0:
            raise MemoryError("oracle_skip_head_f32: out of memory")
        return HeadResult(o=o, lse=lse, skipped=skipped.astype(bool), margin=margin, qblocks=qb)

    def skip_mask(self, q: np.ndarray, k: np.ndarray, scale: float, ln_lambda: Optional[np.float32],
                  qblocks: Optional[Iterable[int]] = None, block_q: int = BLOCK_Q, block_k: int = BLOCK_K):
        """The tile decisions and margins of the single-precision recurrence
        alone (scores, tile maxima, vote, running maximum of the kept tiles;
        no exponentials and no P.V).  Returns (skipped [nb, nKT] bool,
        margin [nb, nKT] float32), equal to skip_head's."""
        q, k = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k))
        S, D = q.shape
        nqb, nkt = -(-S // block_q), -(-S // block_k)
        qb = np.arange(nqb, dtype=np.int64) if qblocks is None else np.ascontiguousarray(list(qblocks), dtype=np.int64)
        nb = len(qb)
        skipped = np.empty((nb, nkt), np.uint8)
        margin = np.empty((nb, nkt), np.float32)
        vote = ln_lambda is not None
        rc = self.lib.oracle_skip_mask_f32(
            q.ctypes.data, k.ctypes.data, S, D, float(np.float32(scale)), int(vote),
            float(np.float32(ln_lambda)) if vote else 0.0, block_q, block_k, qb.ctypes.data, nb,
            skipped.ctypes.data, margin.ctypes.data)
        if rc != 0:
            raise MemoryError("oracle_skip_mask_f32: out of memory")
        return skipped.astype(bool), margin

    def skip_attention(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       ln_lambda: Optional[np.float32], forced_skip: Optional[np.ndarray] = None,
                       block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> SkipResult:
        """skip_head over every (b, h) of [B, H, S, D] tensors."""
        B, H, S, _ = q.shape
        Dv = v.shape[-1]
        nqb, nkt = -(-S // block_q), -(-S // block_k)
        o = np.empty((B, H, S, Dv), np.float32)
        lse = np.empty((B, H, S), np.float32)
        skipped = np.zeros((B, H, nqb, nkt), dtype=bool)
        margin = np.zeros((B, H, nqb, nkt), dtype=np.float32)
        for b in range(B):
            for h in range(H):
                r = self.skip_head(q[b, h], k[b, h], v[b, h], scale, ln_lambda,
                                   forced_skip=None if forced_skip is None else forced_skip[b, h],
                                   block_q=block_q, block_k=block_k)
                o[b, h] = r.o.reshape(-1, Dv)[:S]
                lse[b, h] = r.lse.reshape(-1)[:S]
                skipped[b, h], margin[b, h] = r.skipped, r.margin
        return SkipResult(o=o, lse=lse, skipped=skipped, margin=margin, skip_counts=skipped.sum(axis=-1))


_default: Optional[COracle] = None


def oracle() -> COracle:
    """The process-wide instance of the (unmutated) C oracle."""
    global _default
    if _default is None:
        _default = COracle()
    return _default
