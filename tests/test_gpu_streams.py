"""Streams and HIP graphs: the entry points enqueue their kernels on the
caller's current stream and allocate nothing, so they run on a side stream
and under graph capture.

Each graph is replayed several times with eager work and synchronisations
between the replays, and every replay is compared bit for bit with the eager
result of the same call.
"""
import numpy as np
import pytest
import torch

from skip_softmax_flashattention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssa():
    import skip_softmax_flashattention_amd as m
    m.device_check()
    return m


@pytest.fixture(scope="module")
def grid_w():
    return inputs.grid_small(41, (4, 16, 17), heads=3)


def test_side_stream(ssa, grid_w):
    """Launched on a side stream, waited for on that stream only."""
    q, k, v = (t.cuda() for t in (grid_w.q, grid_w.k, grid_w.v))
    ref = ssa.fwd(q, k, v, threshold=0.3, scale=grid_w.scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = ssa.fwd(q, k, v, threshold=0.3, scale=grid_w.scale)
    s.synchronize()
    for a, b in zip(ref, out):
        assert torch.equal(a, b)
    assert int(ref[2].sum()) > 0


def _replays_match(graph, outs, refs, eager):
    for i in range(3):
        graph.replay()
        eager()   # other work between replays
        torch.cuda.synchronize()
        for a, b in zip(outs, refs):
            assert torch.equal(a, b), f"replay {i}"


def test_graph_fixed_length(ssa, grid_w):
    """Dense and skip calls captured together in one graph."""
    q, k, v = (t.cuda() for t in (grid_w.q, grid_w.k, grid_w.v))
    ref_d = ssa.fwd(q, k, v, factor=0.0, scale=grid_w.scale)
    ref_s = ssa.fwd(q, k, v, threshold=0.3, scale=grid_w.scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ssa.fwd(q, k, v, factor=0.0, scale=grid_w.scale)   # warm the allocator outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            out_d = ssa.fwd(q, k, v, factor=0.0, scale=grid_w.scale)
            out_s = ssa.fwd(q, k, v, threshold=0.3, scale=grid_w.scale)
    torch.cuda.synchronize()
    _replays_match(g, list(out_d) + list(out_s), list(ref_d) + list(ref_s),
                   lambda: ssa.fwd(q, k, v, threshold=0.05, scale=grid_w.scale))


def test_graph_varlen_with_host_lengths(ssa):
    """The packed entry under capture, with the lengths given on the host."""
    w = inputs.varlen(seed=42, heads=2, grids=((1, 7, 10), (3, 10, 13), (2, 8, 9)))
    q, k, v = (t.cuda() for t in (w.q, w.k, w.v))
    cu = w.cu_seqlens.cuda()
    smax = max(w.seqlens)
    ref = ssa.fwd_varlen(q, k, v, cu, smax, factor=2.0, scale=w.scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ssa.fwd_varlen(q, k, v, cu, smax, factor=2.0, scale=w.scale, seqlens=w.seqlens)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            out = ssa.fwd_varlen(q, k, v, cu, smax, factor=2.0, scale=w.scale, seqlens=w.seqlens)
    torch.cuda.synchronize()
    _replays_match(g, list(out), list(ref), lambda: ssa.fwd_varlen(q, k, v, cu, smax, factor=0.0, scale=w.scale))
    assert int(ref[2].sum()) > 0


def test_graph_virtual_and_fp8(ssa, grid_w):
    """The two-kernel calls (tile-mean pre-pass + attention; quantiser +
    FP8-score attention) under capture."""
    q, k, v = (t.cuda() for t in (grid_w.q, grid_w.k, grid_w.v))
    B, H, S, _ = q.shape
    ws = torch.empty(ssa.virtual_workspace_bytes(B, H, S), dtype=torch.uint8, device="cuda")
    ref_v = ssa.fwd_virtual(q, k, v, threshold=0.3, scale=grid_w.scale, workspace=ws)
    q8, k8, qs, ks = ssa.quantize_qk_fp8(q, k)
    ref_8 = ssa.fwd_fp8(q8, k8, qs, ks, v, threshold=0.3, scale=grid_w.scale)
    ref_q = (q8.clone(), k8.clone(), qs.clone(), ks.clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ssa.fwd_virtual(q, k, v, threshold=0.3, scale=grid_w.scale, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            out_v = ssa.fwd_virtual(q, k, v, threshold=0.3, scale=grid_w.scale, workspace=ws)
            g8 = ssa.quantize_qk_fp8(q, k)
            out_8 = ssa.fwd_fp8(*g8, v, threshold=0.3, scale=grid_w.scale)
    torch.cuda.synchronize()
    _replays_match(g, list(out_v) + list(out_8) + list(g8), list(ref_v) + list(ref_8) + list(ref_q),
                   lambda: ssa.fwd(q, k, v, threshold=0.05, scale=grid_w.scale))


def test_two_host_threads_two_streams(ssa, grid_w):
    """Two host threads, each on its own stream, call the library at the same
    time (ctypes releases the GIL during the call): one the fixed-length skip
    call, the other the packed entry.  Every result equals the serial one."""
    import threading
    q, k, v = (t.cuda() for t in (grid_w.q, grid_w.k, grid_w.v))
    wv = inputs.varlen(seed=43, heads=2, grids=((1, 7, 10), (3, 10, 13)))
    qv, kv, vv = (t.cuda() for t in (wv.q, wv.k, wv.v))
    cu = wv.cu_seqlens.cuda()
    ref_a = ssa.fwd(q, k, v, threshold=0.3, scale=grid_w.scale)
    ref_b = ssa.fwd_varlen(qv, kv, vv, cu, max(wv.seqlens), factor=2.0, scale=wv.scale)
    torch.cuda.synchronize()
    outs, errors = {"a": [], "b": []}, []

    def run(name, fn):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(8):
                    outs[name].append(fn())
            s.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(e)

    ta = threading.Thread(target=run, args=("a", lambda: ssa.fwd(q, k, v, threshold=0.3, scale=grid_w.scale)))
    tb = threading.Thread(target=run, args=("b", lambda: ssa.fwd_varlen(qv, kv, vv, cu, max(wv.seqlens), factor=2.0,
                                                                        scale=wv.scale, seqlens=wv.seqlens)))
    ta.start()
    tb.start()
    ta.join()
    tb.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for got in outs["a"]:
        assert all(torch.equal(x, y) for x, y in zip(got, ref_a))
    for got in outs["b"]:
        assert all(torch.equal(x, y) for x, y in zip(got, ref_b))
    assert len(outs["a"]) == len(outs["b"]) == 8
