"""Skip-Softmax (BLASST) FlashAttention forward on AMD Instinct MI355X.

Thin ctypes binding of the C ABI in include/ssa.h (libssa.so, built for
gfx950).  This module only marshals arguments: it checks tensor dtypes,
shapes and devices, allocates the outputs with torch, and passes raw device
pointers and the current HIP stream to the library, which enqueues its
kernels (one per call; two for fwd_virtual and quantize_qk_fp8).  Every step
of the attention runs in the HIP kernels; there is no fallback.  If libssa.so is missing or the device is not gfx950 the calls
raise.

Controls ("Skip-Softmax" design document of vLLM-Omni, section "From
configuration to the kernel threshold"), exactly one per call:
  factor=f           lambda = f / seqlen      (the kernel's own input)
  threshold=t        lambda = t               (direct control)
  calib=(a, b, s)    lambda = a exp(b s) / seqlen   (calibrated control)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "SsaError", "fwd", "fwd_varlen", "fwd_debug", "fwd_max_prob", "fwd_virtual", "virtual_workspace_bytes",
    "quantize_qk_fp8", "fwd_fp8", "resolve_threshold", "device_check", "set_vote_poll_limit", "vote_poll_limit",
    "library_path", "load_library", "BLOCK_Q", "BLOCK_K", "HEAD_DIM",
    "MODE_FACTOR", "MODE_THRESHOLD", "MODE_CALIBRATED",
]

HEAD_DIM = 128
BLOCK_Q = 64
BLOCK_K = 128
MODE_FACTOR, MODE_THRESHOLD, MODE_CALIBRATED = 0, 1, 2

SSA_OK = 0
STATUS_NAMES = {
    0: "SSA_OK", -1: "SSA_ERR_INVALID_ARG", -2: "SSA_ERR_UNSUPPORTED", -3: "SSA_ERR_BAD_THRESHOLD",
    -4: "SSA_ERR_NO_CALIBRATION", -5: "SSA_ERR_DEVICE", -6: "SSA_ERR_LAUNCH", -7: "SSA_ERR_BAD_CONFIG",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class SsaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, "_lib", "libssa.so")


def load_library() -> ctypes.CDLL:
    """Load libssa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m skip_softmax_flashattention_amd.build")
    lib = ctypes.CDLL(path)
    P, I, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.ssa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, F, I, P, P]
    lib.ssa_fwd_threshold.argtypes = [P, P, P, P, P, I, I, I, I, F, F, P, P]
    lib.ssa_fwd_calibrated.argtypes = [P, P, P, P, P, I, I, I, I, F, F, F, F, I, P, P]
    lib.ssa_fwd_varlen.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, D, D, D, P, P]
    lib.ssa_fwd_debug.argtypes = [P, P, P, P, P, I, I, I, I, F, I, D, D, D, I, P, P, P, P]
    lib.ssa_fwd_ex.argtypes = [P, P, P, P, P, I, I, I, I, F, I, D, D, D, I, P, P, P]
    Z = ctypes.c_size_t
    lib.ssa_fwd_virtual.argtypes = [P, P, P, P, P, I, I, I, I, F, I, D, D, D, I, P, P, Z, P]
    lib.ssa_fwd_virtual_workspace_bytes.argtypes = [I, I, I]
    lib.ssa_fwd_virtual_workspace_bytes.restype = Z
    lib.ssa_quantize_qk_fp8.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
    lib.ssa_fwd_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, I, D, D, D, I, P, P, P, P]
    lib.ssa_resolve_threshold.argtypes = [I, D, D, D, I, ctypes.POINTER(F), ctypes.POINTER(I)]
    for name in ("ssa_fwd", "ssa_fwd_threshold", "ssa_fwd_calibrated", "ssa_fwd_varlen", "ssa_fwd_debug", "ssa_fwd_ex",
                 "ssa_fwd_virtual", "ssa_quantize_qk_fp8", "ssa_fwd_fp8",
                 "ssa_resolve_threshold", "ssa_device_check", "ssa_version"):
        getattr(lib, name).restype = I
    lib.ssa_device_check.argtypes = []
    lib.ssa_set_vote_poll_limit.argtypes = [I]
    lib.ssa_set_vote_poll_limit.restype = I
    lib.ssa_vote_poll_limit.argtypes = []
    lib.ssa_vote_poll_limit.restype = I
    lib.ssa_version.argtypes = []
    lib.ssa_strerror.argtypes = [I]
    lib.ssa_strerror.restype = ctypes.c_char_p
    lib.ssa_last_error.argtypes = []
    lib.ssa_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(code: int) -> None:
    if code != SSA_OK:
        lib = load_library()
        raise SsaError(code, lib.ssa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _control(factor, threshold, calib) -> Tuple[int, float, float, float]:
    given = [x is not None for x in (factor, threshold, calib)]
    if sum(given) != 1:
        raise ValueError("give exactly one of factor=, threshold= or calib=(a, b, target_sparsity)")
    if factor is not None:
        return MODE_FACTOR, float(factor), 0.0, 0.0
    if threshold is not None:
        return MODE_THRESHOLD, float(threshold), 0.0, 0.0
    a, b, s = calib
    return MODE_CALIBRATED, float(a), float(b), float(s)


def _check_qkv(q, k, v, ndim):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if t.dim() != ndim or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {ndim}-D tensor")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")


def _check_out(out: torch.Tensor, q: torch.Tensor) -> None:
    """A caller-supplied output must be what the kernel writes: a contiguous
    bf16 tensor of q's shape on q's device."""
    if not isinstance(out, torch.Tensor):
        raise ValueError("out must be a tensor")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or out.device != q.device \
            or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {tuple(q.shape)} on {q.device}")


def _varlen_lengths(cu_seqlens: torch.Tensor, T: int, max_seqlen: int, seqlens: Optional[Sequence[int]],
                    read_back: bool) -> Optional[list]:
    """The sequence lengths of a packed batch on the host: ``seqlens`` when
    given, else read back from the device cu_seqlens when ``read_back``, else
    None.  Lengths known on the host are checked against the packed tensors:
    one per sequence, none negative or above max_seqlen, summing to T."""
    nseq = cu_seqlens.numel() - 1
    if seqlens is not None:
        lens = [int(n) for n in seqlens]
    elif read_back:
        lens = (cu_seqlens[1:] - cu_seqlens[:-1]).tolist()
    else:
        return None
    if len(lens) != nseq:
        raise ValueError(f"seqlens has {len(lens)} entries for {nseq} sequences")
    if any(n < 0 for n in lens):
        raise ValueError("sequence lengths must be non-negative")
    if lens and max(lens) > max_seqlen:
        raise ValueError(f"a sequence of {max(lens)} tokens exceeds max_seqlen = {max_seqlen}")
    if sum(lens) != T:
        raise ValueError(f"the sequence lengths sum to {sum(lens)}, but q holds {T} tokens")
    return lens


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
        factor: Optional[float] = None, threshold: Optional[float] = None, calib=None,
        seqlen: Optional[int] = None, with_lse: bool = True, with_counts: bool = True,
        out: Optional[torch.Tensor] = None):
    """Skip-softmax attention of bf16 [B, H, S, 128] tensors.

    Returns (o, lse, skip_counts): o bf16 [B, H, S, 128], lse float32
    [B, H, S] (or None), skip_counts int32 [B, H, ceil(S/64)] (or None).
    ``seqlen`` (the length lambda is normalised by) defaults to S.  ``out``, if
    given, receives o and must be a contiguous bf16 tensor shaped like q on
    q's device.
    """
    _check_qkv(q, k, v, 4)
    if out is not None:
        _check_out(out, q)
    B, H, S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mode, p0, p1, p2 = _control(factor, threshold, calib)
    n = S if seqlen is None else int(seqlen)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if with_lse else None
    cnt = torch.empty((B, H, -(-S // BLOCK_Q)), dtype=torch.int32, device=q.device) if with_counts else None
    lib = load_library()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D, scale)
    if mode == MODE_FACTOR:
        rc = lib.ssa_fwd(*args, p0, n, _ptr(cnt), _stream(q))
    elif mode == MODE_THRESHOLD:
        rc = lib.ssa_fwd_threshold(*args, p0, _ptr(cnt), _stream(q))
    else:
        rc = lib.ssa_fwd_calibrated(*args, p0, p1, p2, n, _ptr(cnt), _stream(q))
    _check(rc)
    return o, lse, cnt


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
               max_seqlen: int, *, scale: Optional[float] = None, factor: Optional[float] = None,
               threshold: Optional[float] = None, calib=None, with_lse: bool = True,
               with_counts: bool = True, seqlens: Optional[Sequence[int]] = None):
    """Packed variable-length batch: q, k, v bf16 [T, H, 128], cu_seqlens int32
    [nseq + 1] on the device.  Each sequence normalises lambda by its own
    length.  Returns (o [T, H, 128], lse [H, T], skip_counts [H, sum ceil(S_b/64)]).
    The skip counts' size comes from the sequence lengths: pass them on the
    host as ``seqlens`` to avoid reading cu_seqlens back from the device
    (a synchronisation that HIP graph capture does not allow).  ``seqlens``
    must equal the lengths cu_seqlens holds on the device; lengths known on
    the host are checked against q (they must sum to T, and none may exceed
    max_seqlen).  A sequence longer than max_seqlen would be left unwritten
    by the kernel."""
    _check_qkv(q, k, v, 3)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be an int32 1-D tensor on the same device as q")
    T, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mode, p0, p1, p2 = _control(factor, threshold, calib)
    nseq = cu_seqlens.numel() - 1
    if nseq < 0:
        raise ValueError("cu_seqlens must hold at least one entry")
    lens = _varlen_lengths(cu_seqlens, T, int(max_seqlen), seqlens, read_back=with_counts)
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if with_lse else None
    cnt = None
    if with_counts:
        cnt = torch.empty((H, sum(-(-n // BLOCK_Q) for n in lens)), dtype=torch.int32, device=q.device)
    lib = load_library()
    rc = lib.ssa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), nseq,
                            int(max_seqlen), H, D, scale, mode, p0, p1, p2, _ptr(cnt), _stream(q))
    _check(rc)
    return o, lse, cnt


def fwd_max_prob(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
                 factor: Optional[float] = None, threshold: Optional[float] = None, calib=None,
                 seqlen: Optional[int] = None):
    """fwd plus each row's largest softmax weight over the kept keys,
    max_prob = exp(m - LSE) = 1 / l: returns (o, lse, skip_counts, max_prob
    float32 [B, H, S])."""
    _check_qkv(q, k, v, 4)
    B, H, S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mode, p0, p1, p2 = _control(factor, threshold, calib)
    n = S if seqlen is None else int(seqlen)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    cnt = torch.empty((B, H, -(-S // BLOCK_Q)), dtype=torch.int32, device=q.device)
    mp = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    lib = load_library()
    _check(lib.ssa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D, scale, mode, p0, p1, p2, n,
                          _ptr(cnt), _ptr(mp), _stream(q)))
    return o, lse, cnt, mp


def virtual_workspace_bytes(B: int, H: int, S: int) -> int:
    """Bytes of device workspace fwd_virtual needs (the per-tile means)."""
    return int(load_library().ssa_fwd_virtual_workspace_bytes(int(B), int(H), int(S)))


def fwd_virtual(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
                factor: Optional[float] = None, threshold: Optional[float] = None, calib=None,
                seqlen: Optional[int] = None, workspace: Optional[torch.Tensor] = None):
    """fwd with every skipped tile replaced by a virtual key (the tile's mean
    key, score + ln n_t) carrying the tile's mean value ("Triage: Skip, Skim,
    or Refine Attention Tiles in Video Diffusion Transformers", section 6.1).
    The skip mask and counts are those of fwd.  ``workspace`` (a device tensor
    of at least virtual_workspace_bytes(B, H, S) bytes) is allocated when not
    given.  Returns (o, lse, skip_counts)."""
    _check_qkv(q, k, v, 4)
    B, H, S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mode, p0, p1, p2 = _control(factor, threshold, calib)
    n = S if seqlen is None else int(seqlen)
    need = virtual_workspace_bytes(B, H, S)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    cnt = torch.empty((B, H, -(-S // BLOCK_Q)), dtype=torch.int32, device=q.device)
    lib = load_library()
    _check(lib.ssa_fwd_virtual(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D, scale, mode, p0, p1, p2,
                               n, _ptr(cnt), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(q)))
    return o, lse, cnt


def quantize_qk_fp8(q: torch.Tensor, k: torch.Tensor):
    """OCP E4M3 codes of q and k with their scales: returns (q8 uint8 [B, H, S,
    128], k8 uint8 [B, H, S, 128], q_scale float32 [B, H, S] (per token),
    k_scale float32 [B, H, ceil(S/128)] (per 128-key tile))."""
    _check_qkv(q, k, k, 4)
    B, H, S, D = q.shape
    q8 = torch.empty((B, H, S, D), dtype=torch.uint8, device=q.device)
    k8 = torch.empty((B, H, S, D), dtype=torch.uint8, device=q.device)
    qs = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    ks = torch.empty((B, H, -(-S // BLOCK_K)), dtype=torch.float32, device=q.device)
    _check(load_library().ssa_quantize_qk_fp8(_ptr(q), _ptr(k), _ptr(q8), _ptr(k8), _ptr(qs), _ptr(ks), B, H, S, D,
                                              _stream(q)))
    return q8, k8, qs, ks


def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, q_scale: torch.Tensor, k_scale: torch.Tensor, v: torch.Tensor, *,
            scale: Optional[float] = None, factor: Optional[float] = None, threshold: Optional[float] = None,
            calib=None, seqlen: Optional[int] = None, debug: bool = False):
    """Skip-softmax attention with FP8 scores (operands from quantize_qk_fp8)
    and bf16 P.V.  Returns (o, lse, skip_counts), plus (tile_mask, tile_margin)
    when ``debug``."""
    if v.dtype != torch.bfloat16 or v.dim() != 4 or not v.is_contiguous() or v.device.type != "cuda":
        raise ValueError("v must be a contiguous bf16 [B, H, S, 128] CUDA (HIP) tensor")
    B, H, S, D = v.shape
    for name, t, dt, shape in (("q8", q8, torch.uint8, (B, H, S, D)), ("k8", k8, torch.uint8, (B, H, S, D)),
                               ("q_scale", q_scale, torch.float32, (B, H, S)),
                               ("k_scale", k_scale, torch.float32, (B, H, -(-S // BLOCK_K)))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != v.device:
            raise ValueError(f"{name} must be a contiguous {dt} {shape} tensor on the device of v")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mode, p0, p1, p2 = _control(factor, threshold, calib)
    n = S if seqlen is None else int(seqlen)
    nqb, nkt = -(-S // BLOCK_Q), -(-S // BLOCK_K)
    o = torch.empty_like(v)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=v.device)
    cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=v.device)
    mask = torch.empty((B, H, nqb, nkt), dtype=torch.uint8, device=v.device) if debug else None
    margin = torch.empty((B, H, nqb, nkt), dtype=torch.float32, device=v.device) if debug else None
    _check(load_library().ssa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(q_scale), _ptr(k_scale), _ptr(v), _ptr(o), _ptr(lse),
                                      B, H, S, D, scale, mode, p0, p1, p2, n, _ptr(cnt), _ptr(mask), _ptr(margin),
                                      _stream(v)))
    return (o, lse, cnt, mask, margin) if debug else (o, lse, cnt)


def fwd_debug(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
              factor: Optional[float] = None, threshold: Optional[float] = None, calib=None,
              seqlen: Optional[int] = None):
    """fwd with every tile decision: returns (o, lse, skip_counts, tile_mask
    uint8 [B, H, nQB, nKT] (1 = skipped), tile_margin float32 [B, H, nQB, nKT])."""
    _check_qkv(q, k, v, 4)
    B, H, S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mode, p0, p1, p2 = _control(factor, threshold, calib)
    n = S if seqlen is None else int(seqlen)
    nqb, nkt = -(-S // BLOCK_Q), -(-S // BLOCK_K)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=q.device)
    mask = torch.empty((B, H, nqb, nkt), dtype=torch.uint8, device=q.device)
    margin = torch.empty((B, H, nqb, nkt), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.ssa_fwd_debug(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D, scale, mode, p0, p1, p2, n,
                           _ptr(cnt), _ptr(mask), _ptr(margin), _stream(q))
    _check(rc)
    return o, lse, cnt, mask, margin


def resolve_threshold(mode: int, p0: float, p1: float = 0.0, p2: float = 0.0, seqlen: int = 1):
    """Host-only: (ln_lambda as float32, vote enabled) as the library computes them."""
    lib = load_library()
    ln = ctypes.c_float()
    on = ctypes.c_int()
    _check(lib.ssa_resolve_threshold(int(mode), float(p0), float(p1), float(p2), int(seqlen),
                                     ctypes.byref(ln), ctypes.byref(on)))
    return ln.value, bool(on.value)


def device_check() -> None:
    """Raise SsaError unless the current HIP device is gfx950."""
    _check(load_library().ssa_device_check())


def set_vote_poll_limit(polls: int) -> None:
    """Bound of the wait for the partner wave's half of the vote (polls of
    one LDS word) in later fwd_debug calls of this process; 16384 by default,
    the constant the other entries use.  A wave that gives up keeps the tile
    and its query block's count comes out as -1 - count.  0 forces that path
    from the host (tests)."""
    _check(load_library().ssa_set_vote_poll_limit(int(polls)))


def vote_poll_limit() -> int:
    """The current bound of the vote's wait (see set_vote_poll_limit)."""
    return int(load_library().ssa_vote_poll_limit())
