"""The C ABI on the CPU: the library loads, exports every function that
include/ssa.h declares, validates arguments before touching HIP, and resolves
the threshold like the oracle does.  No kernel is launched here."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
import skip_softmax_flashattention_amd as ssa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")

OK, INVALID, UNSUPPORTED, BAD_THRESHOLD, NO_CALIB, DEVICE = 0, -1, -2, -3, -4, -5
FAKE = 1 << 20        # aligned non-null pointer value: validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(ssa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return ssa.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    assert lib.ssa_version() >= 1
    for code in (OK, INVALID, UNSUPPORTED, BAD_THRESHOLD, NO_CALIB, DEVICE, -6, -7):
        assert lib.ssa_strerror(code).decode().startswith(ssa.STATUS_NAMES[code])


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=2, S=256, D=128, scale=0.088, factor=1.0,
         seqlen=256, counts=None):
    return lib.ssa_fwd(q, k, v, o, lse, B, H, S, D, scale, factor, seqlen, counts, None)


def test_argument_errors_before_any_hip_call(lib):
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, o=FAKE + 8) == INVALID                   # misaligned
    assert _fwd(lib, D=64) == UNSUPPORTED
    assert "128" in lib.ssa_last_error().decode()
    assert _fwd(lib, B=-1) == INVALID
    assert _fwd(lib, scale=float("nan")) == INVALID
    assert _fwd(lib, scale=-1.0) == INVALID
    assert _fwd(lib, scale=0.0) == INVALID
    assert _fwd(lib, factor=-1.0) == BAD_THRESHOLD
    assert _fwd(lib, factor=float("inf")) == BAD_THRESHOLD
    assert _fwd(lib, seqlen=0) == BAD_THRESHOLD
    assert "seqlen" in lib.ssa_last_error().decode()
    assert lib.ssa_fwd_threshold(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 128, 0.1, -0.5, None, None) == BAD_THRESHOLD
    # calibrated control without a usable calibration points at the threshold entry
    rc = lib.ssa_fwd_calibrated(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 128, 0.1, 0.0, 4.0, 0.7, 64, None, None)
    assert rc == NO_CALIB
    assert "threshold" in lib.ssa_last_error().decode()
    rc = lib.ssa_fwd_calibrated(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 128, 0.1, float("nan"), 4.0, 0.7, 64, None, None)
    assert rc == NO_CALIB
    rc = lib.ssa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, None, None, 2, 64, 4, 128, 0.1, 0, 1.0, 0, 0, None, None)
    assert rc == INVALID
    rc = lib.ssa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 64, 4, 128, 0.1, 7, 1.0, 0, 0, None, None)
    assert rc == INVALID   # unknown mode
    rc = lib.ssa_fwd_debug(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 128, 0.1, 0, 1.0, 0.0, 0.0, 64, None, None, None, None)
    assert rc == INVALID   # tile_mask is required


def test_empty_inputs_are_ok_without_a_device(lib):
    assert _fwd(lib, B=0) == OK
    assert _fwd(lib, H=0) == OK
    assert _fwd(lib, S=0) == OK
    assert lib.ssa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 0, 4, 128, 0.1, 1, 0.5, 0, 0, None, None) == OK


def test_no_gpu_means_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _fwd(lib) == DEVICE
    assert lib.ssa_device_check() == DEVICE


@pytest.mark.parametrize("lam", [0.0, 1e-12, 3.1e-7, 1e-4, 0.0123, 0.5, 1.0, 1.859, 40.0])
def test_resolve_threshold_matches_oracle(lam):
    ln, on = ssa.resolve_threshold(ssa.MODE_THRESHOLD, lam)
    want = oracle.ln_lambda_f32(oracle.resolve_lambda(threshold=lam))
    assert on == (want is not None)
    if want is not None:
        assert np.float32(ln) == want


@pytest.mark.parametrize("factor,n", [(0.5, 1024), (4.0, 1024), (3e-3, 32760), (60912.68, 32760), (1.0, 1)])
def test_resolve_factor_matches_oracle(factor, n):
    ln, on = ssa.resolve_threshold(ssa.MODE_FACTOR, factor, seqlen=n)
    assert on and np.float32(ln) == oracle.ln_lambda_f32(oracle.resolve_lambda(factor=factor, seqlen=n))


@pytest.mark.parametrize("s", [0.0, 0.5, 0.7, 0.9])
def test_resolve_calibrated_matches_oracle(s):
    a, b = 2822.6209952221557, 4.388250623520793
    for n in (4096, 32760):
        ln, on = ssa.resolve_threshold(ssa.MODE_CALIBRATED, a, b, s, seqlen=n)
        want = oracle.ln_lambda_f32(oracle.resolve_lambda(a=a, b=b, target_sparsity=s, seqlen=n))
        assert on and np.float32(ln) == want


def test_binding_rejects_two_controls():
    import torch
    x = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ssa.fwd(x, x, x, factor=1.0, threshold=0.1)
    with pytest.raises(ValueError):
        ssa.fwd(x, x, x)
    with pytest.raises(ValueError):   # CPU tensors are rejected, never computed on the host
        ssa.fwd(x, x, x, threshold=0.1)


def test_virtual_workspace_size(lib):
    """Mean keys (hi, lo) and mean values in bf16: 3 x 128 x 2 bytes per key tile."""
    assert ssa.virtual_workspace_bytes(1, 40, 32760) == 40 * 256 * 3 * 128 * 2
    assert ssa.virtual_workspace_bytes(2, 3, 129) == 2 * 3 * 2 * 768
    assert ssa.virtual_workspace_bytes(0, 3, 129) == 0


def test_virtual_argument_errors(lib):
    need = ssa.virtual_workspace_bytes(1, 2, 256)

    def call(ws=FAKE, ws_bytes=need, S=256, mode=0, p0=1.0):
        return lib.ssa_fwd_virtual(FAKE, FAKE, FAKE, FAKE, None, 1, 2, S, 128, 0.088, mode, p0, 0.0, 0.0, S,
                                   None, ws, ws_bytes, None)
    assert call(ws=None) == INVALID
    assert call(ws=FAKE + 8) == INVALID                    # misaligned workspace
    assert call(ws_bytes=need - 1) == INVALID               # too small
    assert "smaller" in lib.ssa_last_error().decode()
    assert call(S=2048 * 128 + 1, ws_bytes=1 << 40) == UNSUPPORTED   # more than 2048 key tiles
    assert call(p0=-1.0) == BAD_THRESHOLD


def test_virtual_noalloc_refuses_before_any_hip_call(lib):
    """The static-workspace entry refuses, on the host, calls whose tile means
    need more than SSA_VIRTUAL_NOALLOC_BYTES (B x H x ceil(S/128) above
    16 MiB / 768 = 21,845 tiles), and validates like fwd_virtual."""
    fn = lib.ssa_fwd_virtual_noalloc
    fn.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int] + \
        [ctypes.c_double] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    limit = (16 << 20) // (3 * 128 * 2)
    assert limit == 21845

    def call(B=1, H=2, S=256, p0=1.0):
        return fn(FAKE, FAKE, FAKE, FAKE, None, B, H, S, 128, 0.088, 0, p0, 0.0, 0.0, S, None, None)
    assert call(H=limit + 1, S=128) == UNSUPPORTED
    assert "static workspace" in lib.ssa_last_error().decode()
    assert call(B=11, H=1, S=2048 * 128) == UNSUPPORTED         # 22,528 tiles
    assert call(p0=-1.0) == BAD_THRESHOLD
    assert fn(None, FAKE, FAKE, FAKE, None, 1, 2, 256, 128, 0.088, 0, 1.0, 0.0, 0.0, 256, None, None) == INVALID
    # within the limit the call gets as far as the device (none here)
    assert call(H=limit, S=128) == DEVICE


def test_fp8_argument_errors(lib):
    def quant(q=FAKE, q8=FAKE, D=128, S=256):
        return lib.ssa_quantize_qk_fp8(q, FAKE, q8, FAKE, FAKE, FAKE, 1, 2, S, D, None)
    assert quant(q=None) == INVALID
    assert quant(q8=FAKE + 4) == INVALID                    # codes need 8-byte alignment
    assert quant(D=64) == UNSUPPORTED
    assert quant(S=0) == OK                                 # empty call

    def fwd(S=256, mask=None, margin=None, p0=1.0, D=128):
        return lib.ssa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 2, S, D, 0.088, 0, p0, 0.0, 0.0,
                               max(S, 1), None, mask, margin, None)
    assert fwd(D=64) == UNSUPPORTED
    assert fwd(S=4096 * 128 + 1) == UNSUPPORTED             # more than 4096 key tiles
    assert fwd(margin=FAKE) == INVALID                      # margin without mask
    assert fwd(p0=float("nan")) == BAD_THRESHOLD
    assert fwd(S=0) == OK


def test_vote_poll_limit_hook(lib):
    """The bound of the vote's wait is a process-wide setting checked on the
    host: 0 .. 2^24 polls, default 16384."""
    assert ssa.vote_poll_limit() == 16384
    try:
        ssa.set_vote_poll_limit(0)
        assert ssa.vote_poll_limit() == 0
        for bad in (-1, (1 << 24) + 1):
            with pytest.raises(ssa.SsaError) as e:
                ssa.set_vote_poll_limit(bad)
            assert e.value.code == INVALID
        assert ssa.vote_poll_limit() == 0
    finally:
        ssa.set_vote_poll_limit(16384)
    assert ssa.vote_poll_limit() == 16384


def test_binding_refuses_a_wrong_out():
    """fwd(out=...) takes only a contiguous bf16 tensor of q's shape on q's
    device (the kernel writes B*H*S*128 bf16 values in that layout)."""
    import torch
    q = torch.empty((1, 2, 64, 128), dtype=torch.bfloat16)
    ssa._check_out(torch.empty_like(q), q)
    for bad in (torch.empty((1, 2, 63, 128), dtype=torch.bfloat16),
                torch.empty((1, 2, 64, 128), dtype=torch.float32),
                torch.empty((1, 2, 128, 64), dtype=torch.bfloat16).transpose(-1, -2),
                torch.empty((1, 2, 64, 128), dtype=torch.bfloat16, device="meta"),
                "not a tensor"):
        with pytest.raises(ValueError):
            ssa._check_out(bad, q)


def test_binding_checks_varlen_lengths():
    """Packed-batch lengths known on the host must match the packed tensors:
    one per sequence, none negative or above max_seqlen, summing to T (the
    kernel sizes nothing from them, but the skip-count buffer is sized from
    them and a longer sequence would be left unwritten)."""
    import torch
    cu = torch.tensor([0, 100, 100, 350], dtype=torch.int32)
    assert ssa._varlen_lengths(cu, 350, 250, None, read_back=True) == [100, 0, 250]
    assert ssa._varlen_lengths(cu, 350, 250, [100, 0, 250], read_back=False) == [100, 0, 250]
    assert ssa._varlen_lengths(cu, 350, 250, None, read_back=False) is None
    for T, smax, lens in ((350, 250, [100, 250]),          # too few lengths
                          (351, 250, [100, 0, 250]),       # lengths do not sum to T
                          (350, 249, [100, 0, 250]),       # a sequence above max_seqlen
                          (350, 250, [150, -50, 250])):    # a negative length
        with pytest.raises(ValueError):
            ssa._varlen_lengths(cu, T, smax, lens, read_back=False)
    with pytest.raises(ValueError):
        ssa._varlen_lengths(cu, 349, 250, None, read_back=True)
