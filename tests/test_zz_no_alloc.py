"""ssa_fwd_virtual_noalloc, the virtual-tile entry for callers that cannot
allocate, against ssa_fwd_virtual (the same computation with a caller-owned
workspace), called through the C ABI.

The no-allocation entry keeps the per-tile means in the library's static
per-GPU array, which keeps the previous call's contents: two calls in a row
on different problems, the second smaller, must each equal the workspace
entry's result bit for bit (the same kernels run in the same order on the
same values, so anything short of equality would mean a stale or wrong
workspace).  A problem whose tile means do not fit the array is refused on
the host before any HIP call.
"""
import ctypes

import numpy as np
import pytest
import torch

from skip_softmax_flashattention_amd import inputs

pytestmark = pytest.mark.gpu

P, I, F, D_ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    lib = m.load_library()
    lib.ssa_fwd_virtual_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, F, I, D_, D_, D_, I, P, P]
    lib.ssa_fwd_virtual_noalloc.restype = I
    return m


def _noalloc(ssa, q, k, v, scale, threshold):
    lib = ssa.load_library()
    B, H, S, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    cnt = torch.empty((B, H, -(-S // 64)), dtype=torch.int32, device=q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    rc = lib.ssa_fwd_virtual_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, S, D, scale, ssa.MODE_THRESHOLD, threshold, 0.0, 0.0, S,
                                     cnt.data_ptr(), stream)
    assert rc == 0, lib.ssa_last_error().decode()
    return o, lse, cnt


def test_noalloc_equals_workspace_entry_twice(ssa):
    """Two calls in a row, the second on a smaller problem (so the array still
    holds the first call's larger set of means), each against ssa_fwd_virtual."""
    cases = [(61, (6, 20, 30), 3, 0.05), (62, (4, 12, 20), 2, 0.3)]   # S = 3600 then S = 960
    for seed, grid, heads, thr in cases:
        w = inputs.grid_small(seed, grid, heads=heads)
        q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
        print(f"[case] no-alloc virtual tiles: grid {grid} heads {heads} S={q.shape[2]} threshold {thr}", flush=True)
        ref_o, ref_lse, ref_cnt = ssa.fwd_virtual(q, k, v, scale=w.scale, threshold=thr)
        o, lse, cnt = _noalloc(ssa, q, k, v, w.scale, thr)
        torch.cuda.synchronize()
        assert int(ref_cnt.sum()) > 0, "the case must skip tiles for the virtual keys to matter"
        assert torch.equal(cnt, ref_cnt)
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
        print(f"[case] no-alloc virtual tiles: {int(cnt.sum())} tiles skipped, equal to the workspace entry",
              flush=True)


def test_noalloc_full_size_then_small(ssa):
    """The long-sequence workload (24 heads x 288 key tiles of means, 5.3 MB of
    the 16 MiB array) at threshold 1e-3, then a one-head problem of 351 tokens
    at threshold 3: each equal to the workspace entry."""
    w = inputs.long_seq()
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    print(f"[case] no-alloc virtual tiles: long sequence {tuple(q.shape)}", flush=True)
    ref = ssa.fwd_virtual(q, k, v, scale=w.scale, threshold=1e-3)
    got = _noalloc(ssa, q, k, v, w.scale, 1e-3)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    del q, k, v, ref, got
    w = inputs.grid_small(62, (3, 9, 13), heads=1)
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    ref = ssa.fwd_virtual(q, k, v, scale=w.scale, threshold=3.0)
    got = _noalloc(ssa, q, k, v, w.scale, 3.0)
    torch.cuda.synchronize()
    assert int(ref[2].sum()) > 0
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_noalloc_refuses_what_does_not_fit(ssa):
    """B * H * ceil(S / 128) * 768 bytes above the array: refused on the host."""
    lib = ssa.load_library()
    fake = 1 << 20
    S = 128 * 21846                      # one (batch, head) with 21846 key tiles: 768 bytes too many
    rc = lib.ssa_fwd_virtual_noalloc(fake, fake, fake, fake, None, 1, 1, S, 128, 0.088, 1, 0.01, 0.0, 0.0, S,
                                     None, None)
    assert rc == -2 and "static workspace" in lib.ssa_last_error().decode()
    S = 128 * 2048                       # 2048 tiles x 10 heads = 20480 triples fit
    rc = lib.ssa_fwd_virtual_noalloc(fake, fake, fake, fake, None, 1, 11, S, 128, 0.088, 1, 0.01, 0.0, 0.0, S,
                                     None, None)
    assert rc == -2                      # 22528 triples do not
